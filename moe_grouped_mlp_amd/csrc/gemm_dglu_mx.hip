// Grouped GEMM, dGLU epilogue (FC2 dgrad), MXFP8 operands and MXFP8 copies of the output.
#include "gemm_kernel.h"

namespace moe {

hipError_t launch_gemm_dglu_mx(const GemmArgs& g, int grid, hipStream_t s) {
  return launch_act<EPI_DGLU, false, true>(g, grid, s);
}

}  // namespace moe
