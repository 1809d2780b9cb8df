// Grouped GEMM, GLU epilogue (FC1 forward), MXFP8 operands and MXFP8 copies of the output.
#include "gemm_kernel.h"

namespace moe {

hipError_t launch_gemm_glu_mx(const GemmArgs& g, int grid, hipStream_t s) {
  return launch_act<EPI_GLU, false, true>(g, grid, s);
}

}  // namespace moe
