// Grouped GEMM, dGLU epilogue (FC2 dgrad), MXFP4 operands and the MXFP4
// copy of dz (rowwise, the FC1 dgrad operand) written by the epilogue.
#include "gemm_kernel.h"

namespace moe {

hipError_t launch_gemm_dglu_f4(const GemmArgs& g, int grid, hipStream_t s) {
  return launch_act_f4<EPI_DGLU>(g, grid, s);
}

}  // namespace moe
