// Grouped GEMM, dGLU epilogue (FC2 dgrad), bf16 operands.
#include "gemm_kernel.h"

namespace moe {

hipError_t launch_gemm_dglu_bf16(const GemmArgs& g, int grid, hipStream_t s) {
  return launch_act<EPI_DGLU, true, false>(g, grid, s);
}

}  // namespace moe
