// Top-k router on the device: per token, the softmax of its router logits
// over all E experts, the k largest probabilities kept without
// renormalisation, in descending order, ties to the lower expert id (TE +
// BioNeMo Mixtral tutorial, the sparse MoE block of Fig. 1: a top-2 router
// over eight experts whose outputs are combined as a weighted sum).
//
// A token takes gs lanes (the smallest power of two >= E, at most 64), so a
// wave routes 64 / gs tokens.  Lane g of a group holds logits g, g + gs, ...;
// the maximum and the sum of exponentials are fixed-order reductions inside
// the group, and each of the k picks is a group arg-max over (logit, lower
// id), so the selection compares the fp32 logits themselves (softmax is
// monotone) and is exact.  The kept probability is exp(logit - max) / sum in
// fp32.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kPerLane = kMaxExperts / kWave;
constexpr int kRouterWaves = 4;   // tokens per workgroup

// Reductions inside aligned groups of gs lanes (gs a power of two <= 64).
MOE_DEV float group_max(float v, int gs) {
  for (int o = gs >> 1; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
MOE_DEV float group_sum(float v, int gs) {
  for (int o = gs >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
// (v, i) := the largest v over the group, the lowest i among equal v
MOE_DEV void group_argmax(float& v, int& i, int gs) {
  for (int o = gs >> 1; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(v, o, kWave);
    const int i2 = __shfl_xor(i, o, kWave);
    if (v2 > v || (v2 == v && i2 < i)) {
      v = v2;
      i = i2;
    }
  }
}

// gs = lanes per token: the smallest power of two >= E, at most 64; a wave
// routes 64 / gs tokens.  Lane g of a group holds logits g, g + gs, ...
__global__ __launch_bounds__(kRouterWaves * kWave) void router_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int gs, int32_t* __restrict__ idx,
    float* __restrict__ probs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int per_wave = kWave / gs;
  const int wave_tok = (blockIdx.x * kRouterWaves + static_cast<int>(threadIdx.x / kWave)) * per_wave;
  if (wave_tok >= T) return;   // uniform across the wave
  const int g = lane & (gs - 1);
  const int t = wave_tok + lane / gs;
  const bool live = t < T;     // lanes of a token past T only join the shuffles
  const float* row = logits + static_cast<int64_t>(live ? t : 0) * E;
  float v[kPerLane];
  float m = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    const int e = g + gs * j;
    v[j] = (live && e < E) ? row[e] : -__builtin_inff();
    m = fmaxf(m, v[j]);
  }
  m = group_max(m, gs);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kPerLane; ++j)
    if (live && g + gs * j < E) s += __expf(v[j] - m);
  const float inv = 1.0f / group_sum(s, gs);
  uint32_t taken = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
    bool have = false;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {   // ascending ids: a tie keeps the lower one
      const int e = g + gs * j;
      if (e < E && !((taken >> j) & 1u) && (!have || v[j] > bv)) {
        bv = v[j];
        bi = e;
        have = true;
      }
    }
    group_argmax(bv, bi, gs);
    if ((bi & (gs - 1)) == g) taken |= 1u << (bi / gs);
    if (live && g == 0) {
      idx[static_cast<int64_t>(t) * k + r] = bi;
      probs[static_cast<int64_t>(t) * k + r] = __expf(bv - m) * inv;
    }
  }
}

}  // namespace

hipError_t launch_router_topk(const float* logits, int T, int E, int k, int32_t* idx,
                              float* probs, hipStream_t s) {
  int gs = 1;
  while (gs < E && gs < kWave) gs <<= 1;
  const int per_block = kRouterWaves * (kWave / gs);
  const int blocks = (T + per_block - 1) / per_block;
  router_topk_kernel<<<blocks, kRouterWaves * kWave, 0, s>>>(logits, T, E, k, gs, idx, probs);
  return hipGetLastError();
}

}  // namespace moe
