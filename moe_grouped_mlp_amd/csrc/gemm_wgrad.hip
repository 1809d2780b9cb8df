// Grouped GEMM, weight gradient (dW1 = dZ^T . Xp, dW2 = dYp^T . a per expert):
// bf16 reads the routed activations as stored ([K][M] and [K][N] images,
// LDS transpose reads for both operands); MXFP8 reads their transposed
// copies, K-contiguous like every other MXFP8 operand.
#include "gemm_kernel.h"

namespace moe {

hipError_t launch_gemm_wgrad(const GemmArgs& g, bool mx, int grid, hipStream_t s) {
  dim3 blk(kThreads), grd(grid);
  if (mx) grouped_gemm_kernel<EPI_WGRAD, false, MOE_ACT_SWIGLU, true><<<grd, blk, 0, s>>>(g);
  else grouped_gemm_kernel<EPI_WGRAD, true, MOE_ACT_SWIGLU, false><<<grd, blk, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace moe
