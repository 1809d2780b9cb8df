// Grouped GEMM, GLU epilogue (FC1 forward), MXFP4 operands and the MXFP4
// copy of a (rowwise, the FC2 operand) written by the epilogue.
#include "gemm_kernel.h"

namespace moe {

hipError_t launch_gemm_glu_f4(const GemmArgs& g, int grid, hipStream_t s) {
  return launch_act_f4<EPI_GLU>(g, grid, s);
}

}  // namespace moe
