// Weight-gradient grouped GEMM with MXFP4 operands (dW1 = dZ^T . Xp, dW2 =
// dYp^T . a per expert, from the MXFP4 transposed copies blocked along the
// routed rows): the 4-bit member of the microscaling family ("Boosting MoE
// Training Throughput with Advanced Fusion Kernels", § "Fused MXFP8 and
// NVFP4 quantization": the transposed copies serve the backward).
#include "gemm_kernel.h"

namespace moe {

hipError_t launch_gemm_wgrad_f4(const GemmArgs& g_in, int grid, hipStream_t s) {
  GemmArgs g = g_in;
  g.clk = gemm_clock_slot(grid);
  grouped_gemm_kernel<EPI_WGRAD, false, MOE_ACT_SWIGLU, true, true>
      <<<dim3(grid), dim3(kThreads), 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace moe
