// moe_grouped_mlp_bwd_noalloc: the backward of the expert block for callers
// that cannot allocate device memory (code under stream capture, tight
// training loops, harnesses that forbid allocation).  It is
// moe_grouped_mlp_bwd with its workspace -- the per-row, per-N-tile partial
// sums of the routing-probability gradient, and the split-K area of the FC1
// dgrad when it fits -- taken from a fixed array the library holds on every
// device it runs on, instead of from the caller.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/moe_gmlp.h"
#include "kernels.h"

// The backward's workspace.  Each device holds its own copy for the life of
// the process.  In host code this name is not a device address: the kernels
// get the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[MOE_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_mu;

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
moe_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) {
        (void)hipGetLastError();   // do not leave the error for the next call
        return MOE_ERR_DEVICE;
      }
      g_scratch[dev].store(q, std::memory_order_release);
      p = q;
    }
  }
  *out = p;
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_grouped_mlp_bwd_noalloc(const moe_bwd_args* a, void* stream) {
  if (moe_status st = moe::grouped_mlp_bwd_check(a)) return st;
  // the dprobs partials must fit; the split-K area is used only if it also
  // fits behind them (results then differ from an unsplit run only in the
  // fp32 summation order of the FC1 dgrad's last round)
  const int64_t need = a->M_cap * moe::grouped_mlp_dprobs_parts(a->I) *
                       static_cast<int64_t>(sizeof(float));
  if (need > static_cast<int64_t>(kScratchBytes)) return MOE_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (moe_status st = scratch_address(&ws)) return st;
  return moe::grouped_mlp_bwd_impl(a, ws, kScratchBytes, stream);
}
