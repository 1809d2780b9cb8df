// Top-k router on the device: per token, the softmax of its router logits
// over all E experts, the k largest probabilities kept without
// renormalisation, in descending order, ties to the lower expert id (TE +
// BioNeMo Mixtral tutorial, the sparse MoE block of Fig. 1: a top-2 router
// over eight experts whose outputs are combined as a weighted sum).
//
// One or four lanes per token (router_core.h); moe_router_route runs the
// same code inside its one-launch routing kernel, so both give identical
// bits.
#include "common.h"
#include "kernels.h"
#include "router_core.h"

namespace moe {
namespace {

constexpr int kRouterThreads = 256;

// GS lanes per token (router_core.h); lane j % GS of a token writes pick j
template <int KP, int GS, bool VEC>
__global__ __launch_bounds__(kRouterThreads) void router_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ idx,
    float* __restrict__ probs) {
  const int gt = blockIdx.x * kRouterThreads + threadIdx.x;
  const int t = gt / GS, gl = gt % GS;
  if (t >= T) return;   // whole groups: a token's lanes share t
  const RouterPicks<KP> r =
      router_token<KP, GS, VEC>(logits + static_cast<int64_t>(t) * E, E, k, gl);
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    if (j < k && j % GS == gl) {
      idx[static_cast<int64_t>(t) * k + j] = r.id[j];
      probs[static_cast<int64_t>(t) * k + j] = r.p[j];
    }
  }
}

template <int KP, int GS>
void launch_kp(const float* logits, int T, int E, int k, int32_t* idx, float* probs,
               hipStream_t s) {
  const int64_t threads = static_cast<int64_t>(T) * GS;
  const int blocks = static_cast<int>((threads + kRouterThreads - 1) / kRouterThreads);
  const bool vec = E % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
  if (vec)
    router_topk_kernel<KP, GS, true><<<blocks, kRouterThreads, 0, s>>>(logits, T, E, k, idx, probs);
  else
    router_topk_kernel<KP, GS, false><<<blocks, kRouterThreads, 0, s>>>(logits, T, E, k, idx,
                                                                         probs);
}

template <int GS>
void launch_gs(const float* logits, int T, int E, int k, int32_t* idx, float* probs,
               hipStream_t s) {
  switch (router_kp(k)) {
    case 1: launch_kp<1, GS>(logits, T, E, k, idx, probs, s); break;
    case 2: launch_kp<2, GS>(logits, T, E, k, idx, probs, s); break;
    case 4: launch_kp<4, GS>(logits, T, E, k, idx, probs, s); break;
    default: launch_kp<8, GS>(logits, T, E, k, idx, probs, s); break;
  }
}

}  // namespace

hipError_t launch_router_topk(const float* logits, int T, int E, int k, int32_t* idx,
                              float* probs, hipStream_t s) {
  if (router_gs(E) == 1)
    launch_gs<1>(logits, T, E, k, idx, probs, s);
  else
    launch_gs<4>(logits, T, E, k, idx, probs, s);
  return hipGetLastError();
}

}  // namespace moe
