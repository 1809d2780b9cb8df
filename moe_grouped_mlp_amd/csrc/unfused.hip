// Unfused activation passes: the GLU forward (a = p * act(z)) and backward
// (dz, dprobs from dA and z) as separate kernels over HBM, the way a layer
// built from plain grouped GEMMs runs them.  They are the like-for-like
// baseline of the fused epilogues, which remove exactly these passes
// ("Boosting MoE Training Throughput with Advanced Fusion Kernels",
// § "Overcoming training bottlenecks in MoE blocks": unfused, the
// activation runs in separate memory-bound kernels; Fig. 3 compares the two).
//
// One workgroup per routed row (grid-stride); a thread takes 4 consecutive
// logical columns, which lie inside one 64-column block of the gate/up
// interleave, so its gate and up values are 8-byte loads.  Pad rows inside
// the groups' padded spans are written as zeros (their dprobs is 0).  dprobs sums each thread's columns in order
// and reduces over the workgroup in a fixed tree, so it is deterministic.
#include "act.h"
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kGluThreads = 256;

MOE_DEV void load4(const uint16_t* p, float* v) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(w.x << 16);
  v[1] = __uint_as_float(w.x & 0xffff0000u);
  v[2] = __uint_as_float(w.y << 16);
  v[3] = __uint_as_float(w.y & 0xffff0000u);
}
MOE_DEV void store4(uint16_t* p, const float* v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// Expert of padded row r and whether r holds data (s_pad [E + 1], s_split [E]).
MOE_DEV bool row_valid(int64_t r, const int* s_pad, const int* s_split, int E) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pad[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return r >= s_pad[lo] && r < s_pad[lo] + s_split[lo];
}

MOE_DEV void load_groups(const int32_t* split, const int32_t* padded, int E, int* s_pad,
                         int* s_split) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    s_pad[e] = padded[e];
    s_split[e] = max(split[e], 0);
  }
  if (threadIdx.x == 0) s_pad[E] = padded[E];
  __syncthreads();
}

// Packed column of logical gate column j (up: + MOE_INTERLEAVE).
MOE_DEV int gate_col(int j) {
  return (j / MOE_INTERLEAVE) * 2 * MOE_INTERLEAVE + (j % MOE_INTERLEAVE);
}

template <int ACT>
__global__ __launch_bounds__(kGluThreads) void glu_fwd_kernel(
    const int32_t* split, const int32_t* padded, int E, int I, int64_t rows,
    const float* __restrict__ probs, const uint16_t* __restrict__ z, uint16_t* __restrict__ a,
    float* amax, ActP act) {
  __shared__ int s_pad[kMaxExperts + 1];
  __shared__ int s_split[kMaxExperts];
  __shared__ float s_red[kGluThreads / kWave];
  load_groups(split, padded, E, s_pad, s_split);
  constexpr bool gated = ACT != MOE_ACT_SRELU;
  const int64_t ldz = gated ? 2 * I : I;
  float m = 0.0f;
  const int64_t padded_end = min(static_cast<int64_t>(s_pad[E]), rows);
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    uint16_t* ar = a + r * static_cast<int64_t>(I);
    if (!row_valid(r, s_pad, s_split, E)) {
      // pad rows of a group hold zeros (MXFP8 column blocks span them)
      if (r < padded_end)
        for (int j = 4 * threadIdx.x; j < I; j += 4 * kGluThreads)
          *reinterpret_cast<uint2*>(ar + j) = make_uint2(0, 0);
      continue;
    }
    const float p = probs[r];
    const uint16_t* zr = z + r * ldz;
    for (int j = 4 * threadIdx.x; j < I; j += 4 * kGluThreads) {
      float g[4], u[4], o[4];
      if constexpr (gated) {
        load4(zr + gate_col(j), g);
        load4(zr + gate_col(j) + MOE_INTERLEAVE, u);
        for (int i = 0; i < 4; ++i) o[i] = p * glu_eval<ACT>(g[i], u[i], act).s;
      } else {
        load4(zr + j, g);
        for (int i = 0; i < 4; ++i) {
          const float rl = fmaxf(fminf(fmaxf(g[i], act.glo), act.ghi), 0.0f);
          o[i] = p * rl * rl;
        }
      }
      const uint2 w = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
      *reinterpret_cast<uint2*>(ar + j) = w;
      // amax of the stored (bf16) values
      m = fmaxf(m, fmaxf(fmaxf(fabsf(__uint_as_float(w.x << 16)),
                               fabsf(__uint_as_float(w.x & 0xffff0000u))),
                         fmaxf(fabsf(__uint_as_float(w.y << 16)),
                               fabsf(__uint_as_float(w.y & 0xffff0000u)))));
    }
  }
  if (amax) {
    m = wave_max(m);
    if ((threadIdx.x & (kWave - 1)) == 0) s_red[threadIdx.x / kWave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      float b = 0.0f;
      for (int w = 0; w < kGluThreads / kWave; ++w) b = fmaxf(b, s_red[w]);
      atomic_max_nonneg(amax, b);
    }
  }
}

template <int ACT>
__global__ __launch_bounds__(kGluThreads) void glu_bwd_kernel(
    const int32_t* split, const int32_t* padded, int E, int I, int64_t rows,
    const float* __restrict__ probs, const uint16_t* __restrict__ z,
    const uint16_t* __restrict__ da, uint16_t* __restrict__ dz, float* __restrict__ dprobs,
    ActP act) {
  __shared__ int s_pad[kMaxExperts + 1];
  __shared__ int s_split[kMaxExperts];
  __shared__ float s_red[kGluThreads];
  load_groups(split, padded, E, s_pad, s_split);
  constexpr bool gated = ACT != MOE_ACT_SRELU;
  const int64_t ldz = gated ? 2 * I : I;
  const int64_t padded_end = min(static_cast<int64_t>(s_pad[E]), rows);
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    if (!row_valid(r, s_pad, s_split, E)) {
      if (threadIdx.x == 0) dprobs[r] = 0.0f;
      if (r < padded_end) {   // pad rows of a group hold zeros
        uint16_t* dzr = dz + r * ldz;
        for (int64_t j = 4 * threadIdx.x; j < ldz; j += 4 * kGluThreads)
          *reinterpret_cast<uint2*>(dzr + j) = make_uint2(0, 0);
      }
      continue;
    }
    const float p = probs[r];
    const uint16_t* zr = z + r * ldz;
    const uint16_t* dar = da + r * static_cast<int64_t>(I);
    uint16_t* dzr = dz + r * ldz;
    float dp = 0.0f;
    for (int j = 4 * threadIdx.x; j < I; j += 4 * kGluThreads) {
      float d[4];
      load4(dar + j, d);
      if constexpr (gated) {
        float g[4], u[4], dg[4], du[4];
        load4(zr + gate_col(j), g);
        load4(zr + gate_col(j) + MOE_INTERLEAVE, u);
        for (int i = 0; i < 4; ++i) {
          const GluVal v = glu_eval<ACT>(g[i], u[i], act);
          const float ds = p * d[i];
          dg[i] = v.g_in ? ds * v.u * v.df : 0.0f;
          du[i] = v.u_in ? ds * v.f : 0.0f;
          dp += d[i] * v.s;
        }
        store4(dzr + gate_col(j), dg);
        store4(dzr + gate_col(j) + MOE_INTERLEAVE, du);
      } else {
        float g[4], o[4];
        load4(zr + j, g);
        for (int i = 0; i < 4; ++i) {
          const bool in = (g[i] >= act.glo) && (g[i] <= act.ghi);
          const float rl = fmaxf(fminf(fmaxf(g[i], act.glo), act.ghi), 0.0f);
          o[i] = in ? p * d[i] * 2.0f * rl : 0.0f;
          dp += d[i] * rl * rl;
        }
        store4(dzr + j, o);
      }
    }
    s_red[threadIdx.x] = dp;
    __syncthreads();
    for (int h = kGluThreads / 2; h > 0; h >>= 1) {   // fixed-order tree
      if (threadIdx.x < h) s_red[threadIdx.x] += s_red[threadIdx.x + h];
      __syncthreads();
    }
    if (threadIdx.x == 0) dprobs[r] = s_red[0];
    __syncthreads();   // s_red is reused by the next row
  }
}

}  // namespace

hipError_t launch_glu_unfused(int direction, const int32_t* split, const int32_t* padded, int E,
                              int I, int64_t rows, const ActP& act, const float* probs,
                              const void* z, void* a, float* amax, const void* da, void* dz,
                              float* dprobs, hipStream_t s) {
  // a bounded grid striding over the rows: the forward pass ends with one
  // amax atomic per workgroup, which contend on one address
  const int blocks = static_cast<int>(rows < 2048 ? rows : 2048);
  const dim3 grd(blocks > 0 ? blocks : 1), blk(kGluThreads);
  const auto* zz = static_cast<const uint16_t*>(z);
#define MOE_GLU_CASE(ACT)                                                                  \
  if (direction == 0)                                                                      \
    glu_fwd_kernel<ACT><<<grd, blk, 0, s>>>(split, padded, E, I, rows, probs, zz,          \
                                            static_cast<uint16_t*>(a), amax, act);         \
  else                                                                                     \
    glu_bwd_kernel<ACT><<<grd, blk, 0, s>>>(split, padded, E, I, rows, probs, zz,          \
                                            static_cast<const uint16_t*>(da),              \
                                            static_cast<uint16_t*>(dz), dprobs, act);
  switch (act.act) {
    case MOE_ACT_SWIGLU:
      if (act_unclamped(act)) { MOE_GLU_CASE(kActSwigluFree) } else { MOE_GLU_CASE(MOE_ACT_SWIGLU) }
      break;
    case MOE_ACT_GEGLU: MOE_GLU_CASE(MOE_ACT_GEGLU) break;
    case MOE_ACT_SRELU: MOE_GLU_CASE(MOE_ACT_SRELU) break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_GLU_CASE
  return hipGetLastError();
}

}  // namespace moe
