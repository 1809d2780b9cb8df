// Grouped GEMM: launch dispatch over the kernel families, tile geometry
// queries, and the fixed-order reduction of the per-N-tile dprobs partials
// written by the dGLU epilogue.  The kernel itself is in gemm_kernel.h.
#include <atomic>

#include "../../include/moe_gmlp.h"
#include "gemm_kernel.h"

namespace moe {
namespace {

// clock trace (moe_gemm_clock_trace): record area, its slots, next slot
std::atomic<int64_t*> g_clk_records{nullptr};
std::atomic<int> g_clk_slots{0};
std::atomic<unsigned> g_clk_next{0};

// dprobs_p[r] = sum_n part[r][n] for valid rows (fixed order), 0 for pad rows.
__global__ __launch_bounds__(256) void dprobs_reduce_kernel(
    const float* __restrict__ part, int n_part, const int32_t* __restrict__ split,
    const int32_t* __restrict__ padded, int E, int64_t M_cap, float* __restrict__ out) {
  __shared__ int s_pad[kMaxExperts + 1];
  __shared__ int s_split[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    s_pad[e] = padded[e];
    s_split[e] = split[e];
  }
  if (threadIdx.x == 0) s_pad[E] = padded[E];
  __syncthreads();
  const int64_t total = min(static_cast<int64_t>(s_pad[E]), M_cap);
  for (int64_t r = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; r < total;
       r += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (s_pad[mid] <= r) lo = mid; else hi = mid - 1;
    }
    float s = 0.0f;
    if (r < s_pad[lo] + s_split[lo]) {
      const float* p = part + r * n_part;
      for (int n = 0; n < n_part; ++n) s += p[n];
    }
    out[r] = s;
  }
}

}  // namespace

int grouped_gemm_tile_n() { return BN; }
size_t grouped_gemm_split_bytes(int grid) {
  // one fp32 256 x 256 partial tile per slot, slots <= grid, plus counters
  return static_cast<size_t>(grid) * (BM * BN * sizeof(float) + sizeof(int));
}
int grouped_gemm_tile_m() { return BM; }
int grouped_gemm_split_limit() { return kMaxSplit; }

int64_t* gemm_clock_slot(int grid) {
  int64_t* rec = g_clk_records.load(std::memory_order_acquire);
  const int slots = g_clk_slots.load(std::memory_order_acquire);
  if (!rec || slots < 1 || grid > MOE_CLOCK_MAX_WORKGROUPS) return nullptr;
  const unsigned i = g_clk_next.fetch_add(1, std::memory_order_relaxed) % slots;
  return rec + static_cast<int64_t>(i) * MOE_CLOCK_MAX_WORKGROUPS * 2;
}

hipError_t launch_grouped_gemm(const GemmArgs& g_in, int epi, bool b_nn, bool mx, int grid,
                               hipStream_t s) {
  GemmArgs g = g_in;
  g.clk = gemm_clock_slot(grid);
  if (mx && b_nn) return hipErrorInvalidValue;
  if (epi == EPI_STORE) return launch_gemm_store(g, b_nn, mx, grid, s);
  if (epi == EPI_WGRAD) return b_nn ? hipErrorInvalidValue : launch_gemm_wgrad(g, mx, grid, s);
  if (mx) {
    if (epi == EPI_GLU) return launch_gemm_glu_mx(g, grid, s);
    if (epi == EPI_DGLU) return launch_gemm_dglu_mx(g, grid, s);
    return hipErrorInvalidValue;
  }
  if (epi == EPI_GLU && !b_nn) return launch_gemm_glu_bf16(g, grid, s);
  if (epi == EPI_DGLU && b_nn) return launch_gemm_dglu_bf16(g, grid, s);
  return hipErrorInvalidValue;
}

hipError_t launch_dprobs_reduce(const float* part, int n_part, const int32_t* split,
                                const int32_t* padded, int E, int64_t M_cap, float* dprobs_p,
                                hipStream_t s) {
  int64_t blocks = (M_cap + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  dprobs_reduce_kernel<<<static_cast<int>(blocks), 256, 0, s>>>(part, n_part, split, padded, E,
                                                              M_cap, dprobs_p);
  return hipGetLastError();
}

}  // namespace moe

namespace {

// One workgroup per CU (96 KB of LDS each, so no two share a CU and no
// grouped-GEMM workgroup fits beside one), idle until the constant-rate
// counter has advanced by `ticks` or a fixed number of polls has passed.
constexpr int kOccupyLds = 96 * 1024;
constexpr int kOccupyMaxPolls = 1 << 24;

__global__ __launch_bounds__(64) void occupy_kernel(int64_t ticks, int* sink) {
  extern __shared__ int lds_hold[];
  const int64_t t0 = static_cast<int64_t>(__builtin_amdgcn_s_memrealtime());
  int64_t t = t0;
  int polls = 0;
  while (t - t0 < ticks && polls < kOccupyMaxPolls) {
    __builtin_amdgcn_s_sleep(8);
    t = static_cast<int64_t>(__builtin_amdgcn_s_memrealtime());
    ++polls;
  }
  // keep the LDS allocation (and so the CU) with a use the compiler cannot drop
  if (threadIdx.x == 0 && polls < 0) sink[0] = lds_hold[0];
}

}  // namespace

extern "C" moe_status moe_bench_occupy(int workgroups, int64_t ticks, void* stream) {
  if (workgroups < 1 || workgroups > 1024 || ticks < 1 || ticks > 100000000)
    return MOE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(occupy_kernel, dim3(workgroups), dim3(64), kOccupyLds,
                     static_cast<hipStream_t>(stream), ticks, static_cast<int*>(nullptr));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

extern "C" int64_t moe_clock_tick_rate_hz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return static_cast<int64_t>(khz) * 1000;
}

extern "C" moe_status moe_gemm_clock_trace(int64_t* records, int slots) {
  if (records && (slots < 1 || slots > 64)) return MOE_ERR_INVALID_ARG;
  moe::g_clk_records.store(nullptr, std::memory_order_release);
  moe::g_clk_slots.store(records ? slots : 0, std::memory_order_release);
  moe::g_clk_next.store(0, std::memory_order_relaxed);
  moe::g_clk_records.store(records, std::memory_order_release);
  return MOE_OK;
}
