// Routing metadata on the device: per-expert token counts (split sizes),
// group offsets and the expert-major row map, with no host round trip
// ("Boosting MoE Training Throughput with Advanced Fusion Kernels",
// § "Eliminating host-device synchronization and CPU launch overhead";
// split sizes as GroupedLinear takes them: TE + BioNeMo Mixtral tutorial,
// § "Challenge 1: fragmented expert kernels").
//
// Three launches, all deterministic (integer work only):
//   count    one workgroup per chunk of 256 tokens: per-expert counts of the
//            chunk into workspace [n_chunks][E] (LDS integer atomics; the
//            counts do not depend on arrival order).
//   scan     one workgroup: per expert, exclusive scan of the chunk counts
//            over chunks (chunk bases, in place), split sizes, offsets and
//            padded offsets (group starts aligned to MOE_GROUP_ALIGN rows).
//   scatter  one workgroup per chunk: a bitmap per expert of the chunk's
//            tokens that picked it gives each slot its rank in the chunk
//            (the row order inside a group is ascending token id); adds the
//            chunk base and writes row_id_map / row_src / probs_p.  Extra
//            workgroups mark pad rows (row_src = -1, probs_p = 0).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kChunk = kRouteChunk;

MOE_DEV int local_expert(int id, int first, int E) {
  int e = id - first;
  return (e >= 0 && e < E) ? e : -1;
}

__global__ __launch_bounds__(kChunk) void route_count_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, int first,
    int32_t* __restrict__ counts, int32_t* err_flag) {
  __shared__ int s_cnt[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_cnt[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kChunk + threadIdx.x;
  if (t < T) {
    int seen[kMaxTopK];
    for (int s = 0; s < k; ++s) {
      int e = local_expert(idx[static_cast<int64_t>(t) * k + s], first, E);
      seen[s] = e;
      if (e < 0) continue;
      bool dup = false;
      for (int s2 = 0; s2 < s; ++s2) dup |= (seen[s2] == e);
      if (dup) {
        set_err(err_flag, MOE_DEVERR_DUP_EXPERT);
        continue;  // a repeated expert keeps the row of its first slot
      }
      atomicAdd(&s_cnt[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    counts[static_cast<int64_t>(blockIdx.x) * E + e] = s_cnt[e];
}

__global__ __launch_bounds__(256) void route_scan_kernel(
    int32_t* __restrict__ counts, int n_chunks, int E, int64_t M_cap,
    int32_t* __restrict__ split, int32_t* __restrict__ offsets,
    int32_t* __restrict__ padded, int32_t* err_flag) {
  __shared__ int s_split[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int c0 = 0; c0 < n_chunks; c0 += 16) {
      // sixteen independent loads in flight, then the bases (in place)
      int v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        v[j] = c0 + j < n_chunks ? counts[static_cast<int64_t>(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (c0 + j < n_chunks) {
          counts[static_cast<int64_t>(c0 + j) * E + e] = run;  // chunk base
          run += v[j];
        }
      }
    }
    s_split[e] = run;
    split[e] = run;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t o = 0, p = 0;
    for (int e = 0; e < E; ++e) {
      if (offsets) offsets[e] = static_cast<int32_t>(o);
      padded[e] = static_cast<int32_t>(p);
      o += s_split[e];
      p += (s_split[e] + MOE_GROUP_ALIGN - 1) / MOE_GROUP_ALIGN * MOE_GROUP_ALIGN;
    }
    if (offsets) offsets[E] = static_cast<int32_t>(o);
    padded[E] = static_cast<int32_t>(p);
    if (p > M_cap) set_err(err_flag, MOE_DEVERR_MCAP_OVERFLOW);
  }
}

__global__ __launch_bounds__(kChunk) void route_scatter_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ probs, int T, int k, int E,
    int first, int n_chunks, int64_t M_cap, const int32_t* __restrict__ chunk_base,
    const int32_t* __restrict__ split, const int32_t* __restrict__ padded,
    int32_t* __restrict__ row_id_map, int32_t* __restrict__ row_src,
    float* __restrict__ probs_p) {
  if (static_cast<int>(blockIdx.x) >= n_chunks) {
    // ---- pad rows: row_src = -1, probs_p = 0 ----
    __shared__ int s_pad[kMaxExperts + 1];
    __shared__ int s_split[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      s_pad[e] = padded[e];
      s_split[e] = split[e];
    }
    if (threadIdx.x == 0) s_pad[E] = padded[E];
    __syncthreads();
    const int64_t stride = static_cast<int64_t>(gridDim.x - n_chunks) * blockDim.x;
    for (int64_t r = static_cast<int64_t>(blockIdx.x - n_chunks) * blockDim.x + threadIdx.x;
         r < M_cap; r += stride) {
      bool pad = r >= s_pad[E];
      if (!pad) {
        int lo = 0, hi = E - 1;
        while (lo < hi) {
          int mid = (lo + hi + 1) >> 1;
          if (s_pad[mid] <= r) lo = mid; else hi = mid - 1;
        }
        pad = r >= s_pad[lo] + s_split[lo];
      }
      if (pad) {
        row_src[r] = -1;
        probs_p[r] = 0.0f;
      }
    }
    return;
  }

  // ---- token rows ----
  // tokens of the chunk that picked each expert, one bit per token (LDS
  // atomic OR: the result does not depend on arrival order); a slot's rank
  // in the chunk is the count of bits below its token, so rows inside a
  // group follow ascending token id, and a token that lists an expert twice
  // maps both slots to one row (the first slot's)
  __shared__ uint64_t s_mask[kMaxExperts][kChunk / 64];
  for (int i = threadIdx.x; i < E * (kChunk / 64); i += blockDim.x)
    s_mask[i / (kChunk / 64)][i % (kChunk / 64)] = 0;
  __syncthreads();

  const int tl = threadIdx.x;
  const int t = blockIdx.x * kChunk + tl;
  int my_e[kMaxTopK];
  for (int s = 0; s < kMaxTopK; ++s) {
    my_e[s] = -1;
    if (s < k && t < T) {
      my_e[s] = local_expert(idx[static_cast<int64_t>(t) * k + s], first, E);
      if (my_e[s] >= 0)
        atomicOr(reinterpret_cast<unsigned long long*>(&s_mask[my_e[s]][tl >> 6]),
                 1ull << (tl & 63));
    }
  }
  __syncthreads();
  int my_rank[kMaxTopK];
  for (int s = 0; s < kMaxTopK; ++s) {
    my_rank[s] = 0;
    if (my_e[s] >= 0) {
      const uint64_t* mk = s_mask[my_e[s]];
      int rank = __popcll(mk[tl >> 6] & ((1ull << (tl & 63)) - 1));
      for (int w = 0; w < (tl >> 6); ++w) rank += __popcll(mk[w]);
      my_rank[s] = rank;
    }
  }

  if (t < T) {
    for (int s = 0; s < k; ++s) {
      const int e = my_e[s];
      int32_t r = -1;
      if (e >= 0) {
        const int base = padded[e] + chunk_base[static_cast<int64_t>(blockIdx.x) * E + e];
        const int64_t row = static_cast<int64_t>(base) + my_rank[s];
        if (row < M_cap) {
          r = static_cast<int32_t>(row);
          row_src[row] = t;
          probs_p[row] = probs[static_cast<int64_t>(t) * k + s];
        }
      }
      row_id_map[static_cast<int64_t>(t) * k + s] = r;
    }
  }
}

}  // namespace

hipError_t launch_route(const moe_permute_args& a, hipStream_t s) {
  const int n_chunks = (a.T + kChunk - 1) / kChunk;
  int32_t* counts = static_cast<int32_t*>(a.workspace);
  if (n_chunks > 0) {
    route_count_kernel<<<n_chunks, kChunk, 0, s>>>(a.expert_idx, a.T, a.k, a.E,
                                                   a.first_expert, counts, a.err_flag);
  }
  route_scan_kernel<<<1, 256, 0, s>>>(counts, n_chunks, a.E, a.M_cap, a.split_sizes, a.offsets,
                                      a.padded_offsets, a.err_flag);
  int64_t pad_blocks = (a.M_cap + kChunk - 1) / kChunk;
  if (pad_blocks > 256) pad_blocks = 256;
  if (pad_blocks < 1) pad_blocks = 1;
  route_scatter_kernel<<<n_chunks + static_cast<int>(pad_blocks), kChunk, 0, s>>>(
      a.expert_idx, a.probs, a.T, a.k, a.E, a.first_expert, n_chunks, a.M_cap, counts,
      a.split_sizes, a.padded_offsets, a.row_id_map, a.row_src, a.probs_p);
  return hipGetLastError();
}

}  // namespace moe
