// Token data movement of the expert block (HBM-bound, no MFMA):
//   gather     Xp[row_id_map[t][s]] = X[t]: each token row is read once and
//              written to each of its local slots (push form), in 16-byte
//              vectors, one wave per row; pad rows of every group are zeroed.
//   unpermute  out[t] = bf16(sum_s Yp[row_id_map[t][s]]) in fp32, slot order:
//              the index-add combine of the per-expert loop (TE + BioNeMo
//              Mixtral tutorial, § "Challenge 1: fragmented expert kernels")
//              in gather form, so no atomics and a deterministic result.
//   repack     row permutation of the FC1 weight into gate/up blocks
//              ("Boosting MoE Training Throughput with Advanced Fusion
//              Kernels", § "Optimizing GLU activations with fused GEMM
//              epilogues", Fig. 2).
#include "common.h"
#include "kernels.h"
#include "mx.h"

namespace moe {
namespace {

constexpr int kBlock = 256;
constexpr int kRowsPerBlock = kBlock / kWave;

// ------------------------------------------------------------- gather ---
// Each wave pushes one token row to its k rows.  With MXFP8 output the row
// is encoded once (a quad of lanes holds one 32-value block: four 16-byte
// chunks) and the same codes and scale go to every slot.
// F4: the MX copy is MXFP4 (E2M1 codes two a byte, [M_cap][H / 2]) instead.
template <bool F4>
__global__ __launch_bounds__(kBlock) void gather_kernel(
    const i32x4* __restrict__ x, int T, int k, int H8, const int32_t* __restrict__ row_id_map,
    int64_t M_cap, i32x4* __restrict__ xp, uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
    int tok_blocks, const int32_t* __restrict__ split, const int32_t* __restrict__ padded, int E) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int H = 8 * H8;
  constexpr int kCodeBytes = F4 ? 4 : 8;   // code bytes of a lane's 8 values
  if (static_cast<int>(blockIdx.x) < tok_blocks) {
    for (int t = blockIdx.x * kRowsPerBlock + wave; t < T; t += tok_blocks * kRowsPerBlock) {
      int rows[kMaxTopK];
      for (int s = 0; s < kMaxTopK; ++s) {
        const int r = s < k ? row_id_map[static_cast<int64_t>(t) * k + s] : -1;
        rows[s] = (r >= 0 && r < M_cap) ? r : -1;
      }
      const i32x4* src = x + static_cast<int64_t>(t) * H8;
      auto put = [&](int c, const i32x4 v) {
        if (xp) {
#pragma unroll
          for (int s = 0; s < kMaxTopK; ++s)
            if (rows[s] >= 0) xp[static_cast<int64_t>(rows[s]) * H8 + c] = v;
        }
        if (xq) {
          uint32_t m = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t w = static_cast<uint32_t>(v[i]);
            m = max(m, max(bf16_abs_bits(w), bf16_abs_bits(w >> 16)));
          }
          m = mx_quad_max(m);
          const float am = __uint_as_float(m << 16);
          const int e = F4 ? mx4_exponent(am) : mx_exponent(am);
          const float scale = mx_scale_f32(e);
          const uint2 lo = make_uint2(v[0], v[1]), hi = make_uint2(v[2], v[3]);
          uint2 q;
          if constexpr (F4) {
            q.x = mx4_codes4_bf16(lo, scale) | (mx4_codes4_bf16(hi, scale) << 16);
            q.y = 0;
          } else {
            q.x = mx_codes4_bf16(lo, scale);
            q.y = mx_codes4_bf16(hi, scale);
          }
#pragma unroll
          for (int s = 0; s < kMaxTopK; ++s) {
            if (rows[s] < 0) continue;
            uint8_t* dst = xq + static_cast<int64_t>(rows[s]) * (H / (F4 ? 2 : 1)) + kCodeBytes * c;
            if constexpr (F4) *reinterpret_cast<uint32_t*>(dst) = q.x;
            else *reinterpret_cast<uint2*>(dst) = q;
            if ((c & 3) == 0) xs[mx_scale_off(rows[s], c >> 2, H)] = mx_scale_code(e);
          }
        }
      };
      if (!xq) {
        // plain copy: four of the row's 16-byte chunks per lane are loaded
        // before any is stored, so several loads are in flight at once (a
        // chunk past the row re-reads the first one, which is in range, and
        // is not stored); measured faster for bf16 rows, not for MX rows
        for (int c0 = lane; c0 < H8; c0 += 4 * kWave) {
          i32x4 vs[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int c = c0 + u * kWave;
            vs[u] = src[c < H8 ? c : c0];
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (c0 + u * kWave < H8) put(c0 + u * kWave, vs[u]);
        }
      } else {
        for (int c = lane; c < H8; c += kWave) put(c, src[c]);
      }
    }
    return;
  }
  // pad rows: [padded[e] + split[e], padded[e+1]) for every expert
  const int pb = blockIdx.x - tok_blocks;
  const int n_pb = gridDim.x - tok_blocks;
  const i32x4 zero = {0, 0, 0, 0};
  for (int e = pb; e < E; e += n_pb) {
    const int64_t r0 = static_cast<int64_t>(padded[e]) + split[e];
    const int64_t r1 = min(static_cast<int64_t>(padded[e + 1]), M_cap);
    for (int64_t r = r0 + wave; r < r1; r += kRowsPerBlock) {
      for (int c = lane; c < H8; c += kWave) {
        if (xp) xp[r * H8 + c] = zero;
        if (xq) {
          uint8_t* dst = xq + r * (H / (F4 ? 2 : 1)) + kCodeBytes * c;
          if constexpr (F4) *reinterpret_cast<uint32_t*>(dst) = 0u;
          else *reinterpret_cast<uint2*>(dst) = make_uint2(0, 0);
          if ((c & 3) == 0) xs[mx_scale_off(r, c >> 2, H)] = 0;
        }
      }
    }
  }
}

// ---------------------------------------------------------- unpermute ---
__global__ __launch_bounds__(kBlock) void unpermute_kernel(
    const i32x4* __restrict__ yp, int T, int k, int H8, int64_t M_cap,
    const int32_t* __restrict__ row_id_map, i32x4* __restrict__ out,
    const float* __restrict__ dprobs_p, float* __restrict__ dprobs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int t = blockIdx.x * kRowsPerBlock + wave; t < T; t += gridDim.x * kRowsPerBlock) {
    int rows[kMaxTopK];
    for (int s = 0; s < kMaxTopK; ++s) {
      int r = s < k ? row_id_map[static_cast<int64_t>(t) * k + s] : -1;
      rows[s] = (r >= 0 && r < M_cap) ? r : -1;
    }
    if (dprobs && lane < k) {
      int r = -1;
      for (int s = 0; s < kMaxTopK; ++s) if (s == lane) r = rows[s];
      dprobs[static_cast<int64_t>(t) * k + lane] = r >= 0 ? dprobs_p[r] : 0.0f;
    }
    // two 16-byte chunks per lane per pass, so that 2k loads are in flight;
    // each chunk still sums its slots in slot order (a second chunk past
    // the row re-reads the first, which is in range, and is not stored)
    for (int c0 = lane; c0 < H8; c0 += 2 * kWave) {
      const bool two = c0 + kWave < H8;
      const int c1 = two ? c0 + kWave : c0;
      i32x4 v0[kMaxTopK], v1[kMaxTopK];
#pragma unroll
      for (int s = 0; s < kMaxTopK; ++s) {
        if (rows[s] < 0) continue;
        const i32x4* row = yp + static_cast<int64_t>(rows[s]) * H8;
        v0[s] = row[c0];
        v1[s] = row[c1];
      }
      float acc0[8], acc1[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc0[i] = acc1[i] = 0.0f;
#pragma unroll
      for (int s = 0; s < kMaxTopK; ++s) {
        if (rows[s] < 0) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w0 = static_cast<uint32_t>(v0[s][i]);
          const uint32_t w1 = static_cast<uint32_t>(v1[s][i]);
          acc0[2 * i] += __uint_as_float(w0 << 16);
          acc0[2 * i + 1] += __uint_as_float(w0 & 0xffff0000u);
          acc1[2 * i] += __uint_as_float(w1 << 16);
          acc1[2 * i + 1] += __uint_as_float(w1 & 0xffff0000u);
        }
      }
      i32x4 o0, o1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o0[i] = static_cast<int>(pack_bf16x2(acc0[2 * i], acc0[2 * i + 1]));
        o1[i] = static_cast<int>(pack_bf16x2(acc1[2 * i], acc1[2 * i + 1]));
      }
      i32x4* dst = out + static_cast<int64_t>(t) * H8;
      dst[c0] = o0;
      if (two) dst[c1] = o1;
    }
  }
}

// ------------------------------------------------------------- repack ---
// dst row p of expert e <- src row logical(p) (forward) or the reverse.
__global__ __launch_bounds__(kBlock) void repack_kernel(
    const i32x4* __restrict__ src, i32x4* __restrict__ dst, int E, int I, int H8, int blk,
    int inverse) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t rows = static_cast<int64_t>(E) * 2 * I;
  for (int64_t gr = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave; gr < rows;
       gr += static_cast<int64_t>(gridDim.x) * kRowsPerBlock) {
    const int e = static_cast<int>(gr / (2 * I));
    const int p = static_cast<int>(gr % (2 * I));  // packed row
    const int b = p / (2 * blk), w = p % (2 * blk);
    const int logical = (w < blk) ? b * blk + w : I + b * blk + (w - blk);
    const int64_t base = static_cast<int64_t>(e) * 2 * I;
    const int64_t s_row = base + (inverse ? p : logical);
    const int64_t d_row = base + (inverse ? logical : p);
    const i32x4* s = src + s_row * H8;
    i32x4* d = dst + d_row * H8;
    for (int c = lane; c < H8; c += kWave) d[c] = s[c];
  }
}

__global__ void fill_f32_kernel(float* p, float v, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

int blocks_for(int64_t rows, int cap) {
  int64_t b = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (b > cap) b = cap;
  return b < 1 ? 1 : static_cast<int>(b);
}

}  // namespace

hipError_t launch_gather(const moe_permute_args& a, hipStream_t s) {
  const int H8 = a.H / 8;
  const int tok_blocks = blocks_for(a.T, 2048);
  const int pad_blocks = a.E < 256 ? a.E : 256;
  const bool mx8 = a.flags & MOE_PERMUTE_WRITE_MX, mx4 = a.flags & MOE_PERMUTE_WRITE_MX4;
  if (mx4)
    gather_kernel<true><<<tok_blocks + pad_blocks, kBlock, 0, s>>>(
        static_cast<const i32x4*>(a.x), a.T, a.k, H8, a.row_id_map, a.M_cap,
        static_cast<i32x4*>(a.xp), a.xp_q, a.xp_s, tok_blocks, a.split_sizes, a.padded_offsets,
        a.E);
  else
    gather_kernel<false><<<tok_blocks + pad_blocks, kBlock, 0, s>>>(
        static_cast<const i32x4*>(a.x), a.T, a.k, H8, a.row_id_map, a.M_cap,
        static_cast<i32x4*>(a.xp), mx8 ? a.xp_q : nullptr, mx8 ? a.xp_s : nullptr, tok_blocks,
        a.split_sizes, a.padded_offsets, a.E);
  return hipGetLastError();
}

hipError_t launch_unpermute(const moe_unpermute_args& a, hipStream_t s) {
  const int H8 = a.H / 8;
  unpermute_kernel<<<blocks_for(a.T, 2048), kBlock, 0, s>>>(
      static_cast<const i32x4*>(a.yp), a.T, a.k, H8, a.M_cap, a.row_id_map,
      static_cast<i32x4*>(a.out), a.dprobs_p, a.dprobs);
  return hipGetLastError();
}

hipError_t launch_repack_interleave(const void* src, void* dst, int E, int I, int H, int block,
                                    int inverse, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(E) * 2 * I;
  repack_kernel<<<blocks_for(rows, 4096), kBlock, 0, s>>>(static_cast<const i32x4*>(src),
                                                          static_cast<i32x4*>(dst), E, I, H / 8,
                                                          block, inverse);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, float v, int64_t n, hipStream_t s) {
  int64_t b = (n + 255) / 256;
  if (b > 1024) b = 1024;
  if (b < 1) b = 1;
  fill_f32_kernel<<<static_cast<int>(b), 256, 0, s>>>(p, v, n);
  return hipGetLastError();
}

}  // namespace moe
