// Grouped GEMM, plain-store epilogue C = bf16(acc) (FC2 forward, FC1 dgrad).
#include "gemm_kernel.h"

namespace moe {

hipError_t launch_gemm_store(const GemmArgs& g, bool b_nn, bool mx, int grid, hipStream_t s) {
  dim3 blk(kThreads), grd(grid);
  // the plain epilogue does not depend on the activation
  if (mx) grouped_gemm_kernel<EPI_STORE, false, MOE_ACT_SWIGLU, true><<<grd, blk, 0, s>>>(g);
  else if (b_nn) grouped_gemm_kernel<EPI_STORE, true, MOE_ACT_SWIGLU, false><<<grd, blk, 0, s>>>(g);
  else grouped_gemm_kernel<EPI_STORE, false, MOE_ACT_SWIGLU, false><<<grd, blk, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace moe
