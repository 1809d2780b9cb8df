// Grouped GEMM with MXFP4 operands (E2M1 x E2M1, E8M0 scales per 32 along
// K), plain-store epilogue C = bf16(acc): the 4-bit member of the
// microscaling family on gfx950's scaled MFMA ("Boosting MoE Training
// Throughput with Advanced Fusion Kernels", § "Fused MXFP8 and NVFP4
// quantization" names the 4-bit recipe).
#include "gemm_kernel.h"

namespace moe {

hipError_t launch_gemm_store_f4(const GemmArgs& g_in, int grid, hipStream_t s) {
  GemmArgs g = g_in;
  g.clk = gemm_clock_slot(grid);
  grouped_gemm_kernel<EPI_STORE, false, MOE_ACT_SWIGLU, true, true>
      <<<dim3(grid), dim3(kThreads), 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace moe
