// Grouped GEMM, GLU epilogue (FC1 forward), MXFP4 operands and the MXFP4
// copies of a written by the epilogue (rowwise, the FC2 operand, and
// optionally transposed, the weight gradient's).
#include "gemm_kernel.h"

namespace moe {

hipError_t launch_gemm_glu_f4(const GemmArgs& g, int grid, hipStream_t s) {
  return launch_act_f4<EPI_GLU>(g, grid, s);
}

}  // namespace moe
