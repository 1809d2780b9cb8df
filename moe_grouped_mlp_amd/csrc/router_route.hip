// Router and routing metadata in one launch ("Boosting MoE Training
// Throughput with Advanced Fusion Kernels", § "Eliminating host-device
// synchronization and CPU launch overhead": per-group counts live on the
// device; the AI-digest summary of the same work lists gating, top-k and
// routing fused into a single launch).
//
// One workgroup of 256 threads per chunk of P = 256 / GS tokens (GS lanes
// per token, router_core.h), all workgroups resident at once (the launcher
// keeps the grid within what the CUs hold).  Three phases around two
// grid-wide barriers:
//   A  router (softmax, top-k, ties to the lower id) for each token, kept
//      in registers; each pick of a local expert sets its token's bit in
//      that expert's P-bit chunk bitmap (LDS atomic OR, so the result does
//      not depend on arrival order); a pick's rank in its chunk is the count
//      of bits below its token (rows inside a group follow ascending token
//      id); the chunk's per-expert counts (bits set) go to workspace
//      counts [G][E].
//   B  per expert (spread over the grid), the exclusive scan of its column
//      of chunk counts (chunk bases, in place) and the total (split size).
//   C  every workgroup scans the split sizes (offsets, padded offsets:
//      group starts aligned to MOE_GROUP_ALIGN rows; workgroup 0 stores
//      them), then writes its tokens' expert_idx, probs and row_id_map and
//      the rows' row_src / probs_p, and marks its share of the pad rows
//      (row_src = -1, probs_p = 0).
// Outputs are written only in C, so a barrier's release writes back little
// more than the count matrix.  A barrier (grid_barrier) is an agent-scope
// release, an arrival through one of eight group counters and a bounded
// wait; if the wait runs out (which only a device that cannot hold the
// whole grid at once would cause) the workgroup sets MOE_DEVERR_SYNC_TIMEOUT
// and writes no rows.  The counters a call leaves behind are those the next
// call (or graph replay) expects.
#include "common.h"
#include "kernels.h"
#include "router_core.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxSpin = 1 << 21;        // ~0.5 s of s_sleep 8
// workspace header: the arrival counter (int 0), the generation (int 64)
// and NG <= 8 group counters (ints 128 + 64 i), 256 bytes apart
constexpr int kHeaderInts = 1024;
constexpr int kTop = 0, kGen = 64, kSub0 = 128;

// Grid-wide barrier number `phase` (1, 2) of this call.  Workgroup g arrives
// at group counter g % NG (NG = min(G, 8)); the last arrival of a group
// returns its counter to zero and then adds one to the arrival counter,
// which the others wait for: gen + phase * NG, gen being the arrival
// counter's value when the call started.  The arrival counter is never
// reset; the last arrival of the last barrier stores it as the next call's
// generation.  Every wave's stores reach L2 before thread 0 releases at
// agent scope (one L2 write-back per workgroup) and thread 0's acquire
// invalidates the caches the other waves then read through.
MOE_DEV bool grid_barrier(int32_t* hdr, int gen, int phase, int32_t* err, int* s_ok) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int G = gridDim.x, g = blockIdx.x;
    const int NG = G < 8 ? G : 8;
    const int grp = g % NG;
    const int members = (G - grp + NG - 1) / NG;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    int32_t* sub = hdr + kSub0 + 64 * grp;
    const int old = __hip_atomic_fetch_add(sub, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == members - 1) {
      __hip_atomic_store(sub, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int top = __hip_atomic_fetch_add(hdr + kTop, 1, __ATOMIC_RELEASE,
                                             __HIP_MEMORY_SCOPE_AGENT);
      if (phase == 2 && static_cast<unsigned>(top) == static_cast<unsigned>(gen) + 2 * NG - 1)
        __hip_atomic_store(hdr + kGen, static_cast<int>(static_cast<unsigned>(gen) + 2 * NG),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int target = static_cast<int>(static_cast<unsigned>(gen) + phase * NG);
    int ok = 1;
    int spins = 0;
    // wrap-safe: the arrival counter only grows, modulo 2^32
    while (static_cast<int>(static_cast<unsigned>(__hip_atomic_load(
               hdr + kTop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) -
                            static_cast<unsigned>(target)) < 0) {
      __builtin_amdgcn_s_sleep(8);
      if (++spins >= kMaxSpin) {
        ok = 0;
        break;
      }
    }
    if (!ok) set_err(err, MOE_DEVERR_SYNC_TIMEOUT);
    *s_ok = ok;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  return *s_ok != 0;
}

// Exclusive scans over the E experts of a and b (small ints); every thread
// of the workgroup calls it.  Totals in *ta, *tb.
MOE_DEV void scan2(const int* a, const int* b, int E, int* sa, int* sb, int* s_tmp, int* ta,
                   int* tb) {
  constexpr int kW = kThreads / kWave;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (E + kThreads - 1) / kThreads;
  const int e0 = tid * per;
  int xa = 0, xb = 0;
  for (int i = 0; i < per; ++i) {
    if (e0 + i < E) {
      xa += a[e0 + i];
      xb += b[e0 + i];
    }
  }
  int ia = xa, ib = xb;    // inclusive scans inside the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ya = __shfl_up(ia, o, kWave), yb = __shfl_up(ib, o, kWave);
    if (lane >= o) {
      ia += ya;
      ib += yb;
    }
  }
  if (lane == 63) {
    s_tmp[2 * wave] = ia;
    s_tmp[2 * wave + 1] = ib;
  }
  __syncthreads();
  int ba = 0, bb = 0, sum_a = 0, sum_b = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    if (w < wave) {
      ba += s_tmp[2 * w];
      bb += s_tmp[2 * w + 1];
    }
    sum_a += s_tmp[2 * w];
    sum_b += s_tmp[2 * w + 1];
  }
  int ra = ba + ia - xa, rb = bb + ib - xb;
  for (int i = 0; i < per; ++i) {
    if (e0 + i < E) {
      sa[e0 + i] = ra;
      sb[e0 + i] = rb;
      ra += a[e0 + i];
      rb += b[e0 + i];
    }
  }
  *ta = sum_a;
  *tb = sum_b;
  __syncthreads();
}

// Exclusive scan of one column of chunk counts (expert e) by one wave, in
// place; returns the column total (every lane).  Each lane loads its run
// of up to eight chunks at once.
MOE_DEV int wave_column_scan(int32_t* counts, int G, int E, int e, int lane) {
  const int per = (G + kWave - 1) / kWave;   // <= 8 (G <= 512)
  const int c0 = lane * per;
  int v[8];
  int x = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = (i < per && c0 + i < G) ? counts[static_cast<int64_t>(c0 + i) * E + e] : 0;
    x += v[i];
  }
  int inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += y;
  }
  const int total = __shfl(inc, 63, kWave);
  int run = inc - x;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i < per && c0 + i < G) {
      counts[static_cast<int64_t>(c0 + i) * E + e] = run;
      run += v[i];
    }
  }
  return total;
}

struct RouteArgs {
  const float* logits;
  int T, E_all, k, E, first;
  int64_t M_cap;
  int32_t* idx;
  float* probs;
  int32_t* split;
  int32_t* offsets;
  int32_t* padded;
  int32_t* row_id_map;
  int32_t* row_src;
  float* probs_p;
  int32_t* err;
  int32_t* ws;
};

template <int KP, int GS, bool VEC>
__global__ __launch_bounds__(kThreads) void router_route_kernel(RouteArgs a) {
  constexpr int P = kThreads / GS;        // tokens per workgroup
  constexpr int W = P / 64;               // bitmap words per expert
  __shared__ uint64_t s_mask[kMaxExperts][W];
  __shared__ int s_split[kMaxExperts];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_psize[kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_pad[kMaxExperts + 1];
  __shared__ int s_tmp[2 * (kThreads / kWave)];
  __shared__ int s_ok;
  const int G = gridDim.x, g = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E;
  int32_t* hdr = a.ws;
  int32_t* counts = a.ws + kHeaderInts;   // [G][E]
  // this call's generation (only the previous call, complete, wrote it)
  if (tid == 0) s_ok = __hip_atomic_load(hdr + kGen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int gen = s_ok;

  // ---- A: router (kept in registers), chunk bitmaps, chunk counts ----
  for (int i = tid; i < E * W; i += kThreads) s_mask[i / W][i % W] = 0;
  const int tl = tid / GS, gl = tid % GS;    // token in the chunk, lane in its group
  const int t = g * P + tl;
  RouterPicks<KP> r;
  if (t < a.T)
    r = router_token<KP, GS, VEC>(a.logits + static_cast<int64_t>(t) * a.E_all, a.E_all, a.k,
                                  gl);
  __syncthreads();   // bitmaps cleared
  int my_e[KP];      // local expert of the picks this lane writes (j % GS == gl)
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    my_e[j] = -1;
    if (t < a.T && j < a.k && j % GS == gl) {
      const int e = r.id[j] - a.first;
      if (e >= 0 && e < E) {
        my_e[j] = e;
        atomicOr(reinterpret_cast<unsigned long long*>(&s_mask[e][tl >> 6]), 1ull << (tl & 63));
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) c += __popcll(s_mask[e][w]);
    counts[static_cast<int64_t>(g) * E + e] = c;
  }

  bool ok = grid_barrier(hdr, gen, 1, a.err, &s_ok);

  // ---- B: per expert, chunk bases (in place) and the split size ----
  if (ok) {
    if (E <= 4 * G) {
      // one wave per expert column
      for (int e = g * 4 + wave; e < E; e += 4 * G) {
        const int total = wave_column_scan(counts, G, E, e, lane);
        if (lane == 0) a.split[e] = total;
      }
    } else {
      // one thread per expert column, eight loads at a time
      for (int e = g * kThreads + tid; e < E; e += G * kThreads) {
        int run = 0;
        for (int c0 = 0; c0 < G; c0 += 8) {
          int v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            v[j] = c0 + j < G ? counts[static_cast<int64_t>(c0 + j) * E + e] : 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (c0 + j < G) {
              counts[static_cast<int64_t>(c0 + j) * E + e] = run;
              run += v[j];
            }
          }
        }
        a.split[e] = run;
      }
    }
    ok = grid_barrier(hdr, gen, 2, a.err, &s_ok);
  }

  // ---- C: offsets, then every output of this chunk ----
  if (ok) {
    for (int e = tid; e < E; e += kThreads) {
      const int n = a.split[e];
      s_split[e] = n;
      s_base[e] = counts[static_cast<int64_t>(g) * E + e];
      s_psize[e] = (n + MOE_GROUP_ALIGN - 1) / MOE_GROUP_ALIGN * MOE_GROUP_ALIGN;
    }
    __syncthreads();
    int total, total_pad;
    scan2(s_split, s_psize, E, s_off, s_pad, s_tmp, &total, &total_pad);
    if (tid == 0) s_pad[E] = total_pad;
    __syncthreads();
    if (g == 0) {
      for (int e = tid; e <= E; e += kThreads) {
        a.padded[e] = s_pad[e];
        if (a.offsets) a.offsets[e] = e < E ? s_off[e] : total;
      }
      if (tid == 0 && total_pad > a.M_cap) set_err(a.err, MOE_DEVERR_MCAP_OVERFLOW);
    }
    if (t < a.T) {
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        if (j < a.k && j % GS == gl) {
          const int64_t slot = static_cast<int64_t>(t) * a.k + j;
          a.idx[slot] = r.id[j];
          a.probs[slot] = r.p[j];
          int32_t row_out = -1;
          const int e = my_e[j];
          if (e >= 0) {
            const uint64_t* mk = s_mask[e];
            int rank = __popcll(mk[tl >> 6] & ((1ull << (tl & 63)) - 1));
#pragma unroll
            for (int w = 0; w < W; ++w)
              if (w < (tl >> 6)) rank += __popcll(mk[w]);
            const int64_t row = static_cast<int64_t>(s_pad[e]) + s_base[e] + rank;
            if (row < a.M_cap) {
              row_out = static_cast<int32_t>(row);
              a.row_src[row] = t;
              a.probs_p[row] = r.p[j];
            }
          }
          a.row_id_map[slot] = row_out;
        }
      }
    }
    // pad rows, spread over the grid
    const int64_t stride = static_cast<int64_t>(G) * kThreads;
    for (int64_t rr = static_cast<int64_t>(g) * kThreads + tid; rr < a.M_cap; rr += stride) {
      bool pad = rr >= s_pad[E];
      if (!pad) {
        int lo = 0, hi = E - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_pad[mid] <= rr) lo = mid; else hi = mid - 1;
        }
        pad = rr >= s_pad[lo] + s_split[lo];
      }
      if (pad) {
        a.row_src[rr] = -1;
        a.probs_p[rr] = 0.0f;
      }
    }
  }

}

template <int KP, int GS>
void launch_kp(const RouteArgs& a, int G, hipStream_t s) {
  const bool vec = a.E_all % 4 == 0 && (reinterpret_cast<uintptr_t>(a.logits) & 15) == 0;
  if (vec)
    router_route_kernel<KP, GS, true><<<G, kThreads, 0, s>>>(a);
  else
    router_route_kernel<KP, GS, false><<<G, kThreads, 0, s>>>(a);
}

template <int GS>
void launch_gs(const RouteArgs& a, int G, hipStream_t s) {
  switch (router_kp(a.k)) {
    case 1: launch_kp<1, GS>(a, G, s); break;
    case 2: launch_kp<2, GS>(a, G, s); break;
    case 4: launch_kp<4, GS>(a, G, s); break;
    default: launch_kp<8, GS>(a, G, s); break;
  }
}

}  // namespace

int router_route_chunks(int T, int E_total) {
  const int P = kThreads / router_gs(E_total);
  return (T + P - 1) / P;
}

size_t router_route_workspace_bytes(int T, int E_total, int E) {
  return sizeof(int32_t) *
         (kHeaderInts + static_cast<size_t>(router_route_chunks(T, E_total)) * E);
}

hipError_t launch_router_route(const moe_router_route_args& r, hipStream_t s) {
  RouteArgs a;
  a.logits = r.logits;
  a.T = r.T;
  a.E_all = r.E_total;
  a.k = r.k;
  a.E = r.E;
  a.first = r.first_expert;
  a.M_cap = r.M_cap;
  a.idx = r.expert_idx;
  a.probs = r.probs;
  a.split = r.split_sizes;
  a.offsets = r.offsets;
  a.padded = r.padded_offsets;
  a.row_id_map = r.row_id_map;
  a.row_src = r.row_src;
  a.probs_p = r.probs_p;
  a.err = r.err_flag;
  a.ws = static_cast<int32_t*>(r.workspace);
  const int G = router_route_chunks(r.T, r.E_total);
  if (router_gs(r.E_total) == 1)
    launch_gs<1>(a, G, s);
  else
    launch_gs<4>(a, G, s);
  return hipGetLastError();
}

}  // namespace moe
