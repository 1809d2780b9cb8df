// Grouped GEMM, GLU epilogue (FC1 forward), bf16 operands.
#include "gemm_kernel.h"

namespace moe {

hipError_t launch_gemm_glu_bf16(const GemmArgs& g, int grid, hipStream_t s) {
  return launch_act<EPI_GLU, false, false>(g, grid, s);
}

}  // namespace moe
