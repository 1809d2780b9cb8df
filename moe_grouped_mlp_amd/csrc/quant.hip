// Stand-alone bf16 -> MXFP8 / MXFP4 quantization (memory-bound): the weight
// copies the MX GEMMs read, from the bf16 master weights ("NVIDIA Transformer
// Engine 优化 MoE 生物基础模型训练", § "Challenge 3: quantization overhead":
// bf16 masters are cast before the low-precision GEMM; § "Challenge 2",
// Fig. 3: E4M3 codes with one E8M0 scale per 32 values).
//
// All kernels produce the tiled scale layout in units of 32 output rows x
// 64 K positions (2 blocks per row).
//   ROW  blocks along the contiguous axis.  A wave encodes one unit with
//        four loads of 8 rows x 128 bytes (whole lines); a 32-value block
//        is a quad of lanes, its maximum two DPP exchanges.
//   COL  blocks along rows, output transposed: a workgroup stages a 128-row
//        x 128-column slice of x in LDS and encodes columns from it.
//   BOTH the COL kernel also encodes the staged slice along its rows, so x
//        is read once for both copies.
// MXFP8 COL / BOTH: transpose reads give each lane a whole 32-row column
// block; MXFP4 COL / BOTH: a thread gathers its column block from LDS.
#include "common.h"
#include "kernels.h"
#include "mx.h"

namespace moe {
namespace {

MOE_DEV float amax_of_bits(uint32_t m) { return __uint_as_float(m << 16); }

// Largest magnitude of 8 bf16 values (4 packed words), as a bit pattern.
MOE_DEV uint32_t amax8_bits(const uint4& v) {
  const uint32_t a = max(max(bf16_abs_bits(v.x), bf16_abs_bits(v.x >> 16)),
                         max(bf16_abs_bits(v.y), bf16_abs_bits(v.y >> 16)));
  const uint32_t b = max(max(bf16_abs_bits(v.z), bf16_abs_bits(v.z >> 16)),
                         max(bf16_abs_bits(v.w), bf16_abs_bits(v.w >> 16)));
  return max(a, b);
}

// The block exponent of a 32-value block whose largest magnitude has bit
// pattern m: MXFP8 floor(log2 amax) - 8, MXFP4 floor(log2 amax) - 2.
template <bool F4>
MOE_DEV int block_exp(uint32_t m) {
  return F4 ? mx4_exponent(__uint_as_float(m << 16)) : mx_exponent(__uint_as_float(m << 16));
}

// A lane's 8 values of a block (scale 2^e) -> MXFP8: 8 codes, MXFP4: 8
// nibbles (one word, element 2 i in the low nibble of byte i), stored at
// code offset `off` (values) of q.
template <bool F4>
MOE_DEV void store_codes8(const uint4& v, float scale, uint8_t* q, int64_t off) {
  if constexpr (F4) {
    *reinterpret_cast<uint32_t*>(q + off / 2) =
        mx4_codes4_bf16(make_uint2(v.x, v.y), scale) |
        (mx4_codes4_bf16(make_uint2(v.z, v.w), scale) << 16);
  } else {
    *reinterpret_cast<uint2*>(q + off) = make_uint2(mx_codes4_bf16(make_uint2(v.x, v.y), scale),
                                                    mx_codes4_bf16(make_uint2(v.z, v.w), scale));
  }
}

// x [batch][rows][cols] -> q [batch][rows][cols] (MXFP4: [rows][cols / 2]),
// s tiled (R = rows, K = cols).  A wave encodes one 32 x 64 unit: load j
// covers rows 8 j .. 8 j + 7, lane l row 8 j + l / 8 and 16-byte chunk l % 8
// (8 values), so each load instruction reads eight whole 128-byte lines.
template <bool F4>
__global__ __launch_bounds__(256) void quant_row_kernel(const uint16_t* __restrict__ x,
                                                        int64_t x_stride, int batch, int rows,
                                                        int cols, uint8_t* __restrict__ q,
                                                        uint8_t* __restrict__ s,
                                                        float* __restrict__ amax,
                                                        const int32_t* __restrict__ live) {
  const int lane = threadIdx.x & 63;
  const int units_r = rows / 32, units_c = cols / 64;
  const int64_t units = static_cast<int64_t>(batch) * units_r * units_c;
  const int64_t per_batch = static_cast<int64_t>(rows) * cols;
  const int rl = lane >> 3, ch = lane & 7;
  uint32_t wmax = 0;
  for (int64_t u = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / 64; u < units;
       u += static_cast<int64_t>(gridDim.x) * blockDim.x / 64) {
    const int bi = static_cast<int>(u / (static_cast<int64_t>(units_r) * units_c));
    if (live && live[bi] == 0) continue;   // wave-uniform
    const int rem = static_cast<int>(u % (static_cast<int64_t>(units_r) * units_c));
    const int ur = rem / units_c, uc = rem % units_c;
    const int64_t off0 = bi * per_batch + static_cast<int64_t>(ur * 32 + rl) * cols + uc * 64 + 8 * ch;
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = *reinterpret_cast<const uint4*>(x + (off0 - bi * per_batch) + bi * x_stride +
                                             static_cast<int64_t>(8 * j) * cols);
    // the unit's 64 scale bytes: block b of row r at 32 b + r
    uint8_t* sb = s + bi * (per_batch / 32) + (static_cast<int64_t>(ur) * units_c + uc) * 64 +
                  (ch >> 2) * 32 + rl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t m = mx_quad_max(amax8_bits(v[j]));
      const int e = block_exp<F4>(m);
      store_codes8<F4>(v[j], mx_scale_f32(e), q, off0 + static_cast<int64_t>(8 * j) * cols);
      if ((lane & 3) == 0) sb[8 * j] = mx_scale_code(e);
      if (!F4 && amax) wmax = max(wmax, m);
    }
  }
  if (!F4 && amax) {
    const float m = wave_max(amax_of_bits(wmax));
    if (lane == 0) atomic_max_nonneg(amax, m);
  }
}

// Encodes 32 bf16 values (16 packed words) into 32 E2M1 codes (4 words,
// element 2 i in the low nibble of byte i); returns the scale exponent
// floor(log2 amax) - 2 (2 being the exponent of E2M1's largest value 6),
// clamped to -127.  The codes come from gfx950's scaled conversion of the
// packed words (mx4_codes4_bf16).
MOE_DEV int mx4_encode32(const uint32_t (&w)[16], uint32_t (&packed)[4]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = max(m, max(bf16_abs_bits(w[i]), bf16_abs_bits(w[i] >> 16)));
  const int e = mx4_exponent(__uint_as_float(m << 16));
  const float scale = mx_scale_f32(e);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    packed[i] = mx4_codes4_bf16(make_uint2(w[4 * i], w[4 * i + 1]), scale) |
                (mx4_codes4_bf16(make_uint2(w[4 * i + 2], w[4 * i + 3]), scale) << 16);
  return e;
}

// MXFP4 COL / BOTH.  x [batch][rows][cols] -> q [batch][cols][rows / 2]
// (two E2M1 codes a byte), s tiled (R = cols, K = rows); ROW (the BOTH
// mode): also qr [batch][rows][cols / 2], sr tiled (R = rows, K = cols),
// from the same staged slice.  A thread encodes one column block (32 rows)
// gathered from LDS, then one row block.
constexpr int kColTileR = 128, kColTileC = 128;
constexpr int kColPitch = kColTileC + 2;  // bf16 per LDS row (odd word stride)

template <bool ROW>
__global__ __launch_bounds__(256) void quant_col4_kernel(const uint16_t* __restrict__ x,
                                                         int64_t x_stride, int batch, int rows,
                                                         int cols, uint8_t* __restrict__ q,
                                                         uint8_t* __restrict__ s,
                                                         uint8_t* __restrict__ qr,
                                                         uint8_t* __restrict__ sr,
                                                         const int32_t* __restrict__ live) {
  __shared__ uint16_t tile[kColTileR * kColPitch];
  const int t = threadIdx.x;
  const int tiles_r = (rows + kColTileR - 1) / kColTileR;
  const int tiles_c = (cols + kColTileC - 1) / kColTileC;
  const int64_t tiles = static_cast<int64_t>(batch) * tiles_r * tiles_c;
  const int64_t per_batch_q = static_cast<int64_t>(rows) * cols;
  for (int64_t id = blockIdx.x; id < tiles; id += gridDim.x) {
    const int bi = static_cast<int>(id / (static_cast<int64_t>(tiles_r) * tiles_c));
    if (live && live[bi] == 0) continue;   // uniform over the workgroup
    const int rem = static_cast<int>(id % (static_cast<int64_t>(tiles_r) * tiles_c));
    const int r0 = (rem / tiles_c) * kColTileR, c0 = (rem % tiles_c) * kColTileC;
    const int rr = min(kColTileR, rows - r0);  // 64 or 128
    const int cw = min(kColTileC, cols - c0);  // 64 or 128
    const uint16_t* xb = x + bi * x_stride;
    // stage: rr rows x cw columns, 8 bf16 per thread-iteration
    for (int i = t; i < rr * (cw / 8); i += 256) {
      const int r = i / (cw / 8), c8 = i % (cw / 8);
      const uint4 v = *reinterpret_cast<const uint4*>(xb + static_cast<int64_t>(r0 + r) * cols +
                                                      c0 + 8 * c8);
      uint32_t* d = reinterpret_cast<uint32_t*>(tile + r * kColPitch + 8 * c8);
      d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
    __syncthreads();
    // COL: column c, rows 32 h .. 32 h + 31 of the slice
    for (int u = t; u < cw * (rr / 32); u += 256) {
      const int c = u % cw, h = u / cw;
      uint32_t w[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 32 * h + 2 * i;
        w[i] = static_cast<uint32_t>(tile[r * kColPitch + c]) |
               (static_cast<uint32_t>(tile[(r + 1) * kColPitch + c]) << 16);
      }
      const int cc = c0 + c;
      const int64_t qoff = bi * per_batch_q + static_cast<int64_t>(cc) * rows + r0 + 32 * h;
      uint32_t packed[4];
      const int e = mx4_encode32(w, packed);
      *reinterpret_cast<uint4*>(q + qoff / 2) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      s[bi * (per_batch_q / 32) + mx_scale_off(cc, r0 / 32 + h, rows)] = mx_scale_code(e);
    }
    if constexpr (ROW) {
      // row r of the slice, its 32-column block b: consecutive threads take
      // the blocks of a row, so a wave's reads (rows at a 65-word pitch,
      // blocks 16 words apart) fall on distinct banks
      for (int u = t; u < rr * (cw / 32); u += 256) {
        const int r = u / (cw / 32), b = u % (cw / 32);
        uint32_t w[16];
        const uint32_t* src = reinterpret_cast<const uint32_t*>(tile + r * kColPitch + 32 * b);
#pragma unroll
        for (int i = 0; i < 16; ++i) w[i] = src[i];
        const int64_t row = r0 + r;
        const int col = c0 + 32 * b;
        uint32_t packed[4];
        const int e = mx4_encode32(w, packed);
        *reinterpret_cast<uint4*>(qr + (bi * per_batch_q + row * cols + col) / 2) =
            make_uint4(packed[0], packed[1], packed[2], packed[3]);
        sr[bi * (per_batch_q / 32) + mx_scale_off(row, col / 32, cols)] = mx_scale_code(e);
      }
    }
    __syncthreads();
  }
}

// MXFP8 COL / BOTH.  x [batch][rows][cols] -> q [batch][cols][rows], s tiled
// (R = cols, K = rows); ROW (the BOTH mode): also qr [batch][rows][cols], sr
// tiled (R = rows, K = cols).  A workgroup takes slices of up to 128 rows x
// 128 columns in turn:
// - loads: thread t takes 16-byte chunks t + 256 j (j < 8) of the slice in
//   row order, so a wave instruction reads whole lines; the next slice's
//   loads are issued as soon as this one sits in LDS;
// - ROW: each thread reads its own chunks back (8 values of one row block;
//   the block is a quad of lanes);
// - COL: LDS transpose reads.  A 16-lane group takes 16 columns x 32 rows;
//   read i fetches rows 4 i .. 4 i + 3 (lane s addresses row s / 4, columns
//   4 (s % 4) ..) and lane s receives column s of them.  The four groups of
//   a wave take the four 32-row blocks of the same 16 columns, so one store
//   instruction writes whole 128-byte lines of the transposed copy.
constexpr int kSlPitch = 144;   // bf16 per LDS row: 8-byte aligned, rows 4 apart 1152 bytes
constexpr int kSlR = 128, kSlC = 128;

struct SliceGeo {
  int bi, r0, c0, rr, cw, cpr, nload;   // cpr: 16-byte chunks per row; nload: chunks per thread
};

struct SliceJob {
  const uint16_t* x;
  int64_t x_stride, per_b, tiles, per_batch;
  int rows, cols, tiles_c;

  MOE_DEV SliceGeo geo(int64_t id) const {
    SliceGeo g;
    g.bi = static_cast<int>(id / per_b);
    const int rem = static_cast<int>(id % per_b);
    g.r0 = (rem / tiles_c) * kSlR;
    g.c0 = (rem % tiles_c) * kSlC;
    g.rr = min(kSlR, rows - g.r0);   // 64 or 128
    g.cw = min(kSlC, cols - g.c0);   // 64 or 128
    g.cpr = g.cw / 8;
    g.nload = g.rr * g.cpr / 256;
    return g;
  }
  // the next slice at or after id whose batch entry is live
  MOE_DEV int64_t next_live(const int32_t* live, int64_t id) const {
    while (id < tiles && live && live[id / per_b] == 0) id += gridDim.x;
    return id;
  }
  // chunks past an edge slice re-read chunk t (in range), so every load is
  // unconditional and v stays in registers
  MOE_DEV void load(uint4 (&v)[8], int64_t id, int t) const {
    if (id >= tiles) return;
    const SliceGeo g = geo(id);
    const uint16_t* xb = x + g.bi * x_stride;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = j < g.nload ? t + 256 * j : t;
      const int r = k / g.cpr, c = k % g.cpr;
      v[j] = *reinterpret_cast<const uint4*>(xb + static_cast<int64_t>(g.r0 + r) * cols + g.c0 +
                                             8 * c);
    }
  }
};

template <bool ROW>
__global__ __launch_bounds__(256) void quant_slice8_kernel(const uint16_t* __restrict__ x,
                                                           int64_t x_stride, int batch, int rows,
                                                           int cols, uint8_t* __restrict__ q,
                                                           uint8_t* __restrict__ s,
                                                           float* __restrict__ amax,
                                                           uint8_t* __restrict__ qr,
                                                           uint8_t* __restrict__ sr,
                                                           const int32_t* __restrict__ live) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kSlR * kSlPitch];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  SliceJob job;
  job.x = x;
  job.x_stride = x_stride;
  job.rows = rows;
  job.cols = cols;
  job.tiles_c = (cols + kSlC - 1) / kSlC;
  job.per_b = static_cast<int64_t>((rows + kSlR - 1) / kSlR) * job.tiles_c;
  job.tiles = static_cast<int64_t>(batch) * job.per_b;
  job.per_batch = static_cast<int64_t>(rows) * cols;
  uint32_t wmax = 0;
  uint4 v[8];
  int64_t id = job.next_live(live, blockIdx.x);
  job.load(v, id, t);
  while (id < job.tiles) {
    const SliceGeo g = job.geo(id);
    // LDS image, written word by word (a 16-byte struct copy would keep v in
    // scratch memory)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < g.nload) {
        const int k = t + 256 * j;
        uint32_t* d = reinterpret_cast<uint32_t*>(tile + (k / g.cpr) * kSlPitch + 8 * (k % g.cpr));
        d[0] = v[j].x; d[1] = v[j].y; d[2] = v[j].z; d[3] = v[j].w;
      }
    }
    const int64_t nid = job.next_live(live, id + gridDim.x);
    job.load(v, nid, t);
    if constexpr (ROW) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < g.nload) {
          const int k = t + 256 * j;
          const int r = k / g.cpr, c = k % g.cpr;
          const uint4 w = *reinterpret_cast<const uint4*>(tile + r * kSlPitch + 8 * c);
          const uint32_t m = mx_quad_max(amax8_bits(w));
          const int e = block_exp<false>(m);
          const int64_t row = g.r0 + r;
          const int col = g.c0 + 8 * c;
          store_codes8<false>(w, mx_scale_f32(e), qr, g.bi * job.per_batch + row * cols + col);
          if ((lane & 3) == 0)
            sr[g.bi * (job.per_batch / 32) + mx_scale_off(row, col / 32, cols)] = mx_scale_code(e);
          wmax = max(wmax, m);
        }
      }
    }
    __syncthreads();
    const int grp = lane >> 4, sl = lane & 15;
    const int nrb = g.rr / 32;
    const int items = (g.cw / 16) * nrb;
    for (int it = wave * 4 + grp; it < items; it += 16) {
      const int cg = it / nrb, rb = it % nrb;
      const uint16_t* src = tile + (32 * rb + (sl >> 2)) * kSlPitch + 16 * cg + 4 * (sl & 3);
      const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
          (__attribute__((address_space(3))) void*)src));
      static_assert(4 * kSlPitch * 2 == 1152, "row offsets of the reads below");
      typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
      u32x2_t r0_, r1_, r2_, r3_, r4_, r5_, r6_, r7_;
      // one asm block that waits for its own reads (a read the compiler
      // issued would also wait for the slice loads in flight)
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8\n\t"
          "ds_read_b64_tr_b16 %1, %8 offset:1152\n\t"
          "ds_read_b64_tr_b16 %2, %8 offset:2304\n\t"
          "ds_read_b64_tr_b16 %3, %8 offset:3456\n\t"
          "ds_read_b64_tr_b16 %4, %8 offset:4608\n\t"
          "ds_read_b64_tr_b16 %5, %8 offset:5760\n\t"
          "ds_read_b64_tr_b16 %6, %8 offset:6912\n\t"
          "ds_read_b64_tr_b16 %7, %8 offset:8064\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(r0_), "=&v"(r1_), "=&v"(r2_), "=&v"(r3_), "=&v"(r4_), "=&v"(r5_), "=&v"(r6_),
            "=&v"(r7_)
          : "v"(addr)
          : "memory");
      // cc[i]: rows 4 i .. 4 i + 3 of the column, the first in the low half
      const uint2 cc[8] = {make_uint2(r0_.x, r0_.y), make_uint2(r1_.x, r1_.y),
                           make_uint2(r2_.x, r2_.y), make_uint2(r3_.x, r3_.y),
                           make_uint2(r4_.x, r4_.y), make_uint2(r5_.x, r5_.y),
                           make_uint2(r6_.x, r6_.y), make_uint2(r7_.x, r7_.y)};
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        m = max(m, max(max(bf16_abs_bits(cc[i].x), bf16_abs_bits(cc[i].x >> 16)),
                       max(bf16_abs_bits(cc[i].y), bf16_abs_bits(cc[i].y >> 16))));
      const int e = block_exp<false>(m);
      const float sc = mx_scale_f32(e);
      const int col = g.c0 + 16 * cg + sl;
      uint32_t p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = mx_codes4_bf16(cc[i], sc);
      uint4* dst = reinterpret_cast<uint4*>(q + g.bi * job.per_batch +
                                            static_cast<int64_t>(col) * rows + g.r0 + 32 * rb);
      dst[0] = make_uint4(p[0], p[1], p[2], p[3]);
      dst[1] = make_uint4(p[4], p[5], p[6], p[7]);
      s[g.bi * (job.per_batch / 32) + mx_scale_off(col, (g.r0 + 32 * rb) / 32, rows)] =
          mx_scale_code(e);
      if (!ROW) wmax = max(wmax, m);
    }
    __syncthreads();   // the next slice's image replaces this one
    id = nid;
  }
  if (amax) {
    const float m = wave_max(amax_of_bits(wmax));
    if (lane == 0) atomic_max_nonneg(amax, m);
  }
}

// Workgroups for the ROW kernel (4 units each): at most 512, which streamed
// the large weight shapes fastest (5.1-5.4 TB/s against 4.1-4.5 at 768 and
// more); the slice kernels: at most 2048 (four fit a CU at once).
int row_grid(int64_t units) {
  const int64_t b = (units + 3) / 4;
  return static_cast<int>(b < 1 ? 1 : (b > 512 ? 512 : b));
}
int slice_grid(int64_t tiles, int cap) {
  return static_cast<int>(tiles < 1 ? 1 : (tiles > cap ? cap : tiles));
}

}  // namespace

hipError_t launch_quantize_mxfp4(const moe_quant_args& a, hipStream_t st) {
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  if (a.mode == MOE_QUANT_ROW) {
    const int64_t units = static_cast<int64_t>(a.batch) * (a.rows / 32) * (a.cols / 64);
    quant_row_kernel<true><<<row_grid(units), 256, 0, st>>>(x, a.x_stride, a.batch, a.rows, a.cols,
                                                            a.q, a.s, nullptr, a.live);
  } else {
    const int64_t tiles = static_cast<int64_t>(a.batch) * ((a.rows + kColTileR - 1) / kColTileR) *
                          ((a.cols + kColTileC - 1) / kColTileC);
    // BOTH: the COL copy goes to qT / sT, the ROW copy to q / s
    if (a.mode == MOE_QUANT_BOTH)
      quant_col4_kernel<true><<<slice_grid(tiles, 8192), 256, 0, st>>>(
          x, a.x_stride, a.batch, a.rows, a.cols, a.qT, a.sT, a.q, a.s, a.live);
    else
      quant_col4_kernel<false><<<slice_grid(tiles, 8192), 256, 0, st>>>(
          x, a.x_stride, a.batch, a.rows, a.cols, a.q, a.s, nullptr, nullptr, a.live);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp8(const moe_quant_args& a, hipStream_t st) {
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  if (a.mode == MOE_QUANT_ROW) {
    const int64_t units = static_cast<int64_t>(a.batch) * (a.rows / 32) * (a.cols / 64);
    quant_row_kernel<false><<<row_grid(units), 256, 0, st>>>(x, a.x_stride, a.batch, a.rows,
                                                             a.cols, a.q, a.s, a.amax, a.live);
  } else {
    const int64_t tiles = static_cast<int64_t>(a.batch) * ((a.rows + kSlR - 1) / kSlR) *
                          ((a.cols + kSlC - 1) / kSlC);
    if (a.mode == MOE_QUANT_BOTH)
      quant_slice8_kernel<true><<<slice_grid(tiles, 2048), 256, 0, st>>>(
          x, a.x_stride, a.batch, a.rows, a.cols, a.qT, a.sT, a.amax, a.q, a.s, a.live);
    else
      quant_slice8_kernel<false><<<slice_grid(tiles, 2048), 256, 0, st>>>(
          x, a.x_stride, a.batch, a.rows, a.cols, a.q, a.s, a.amax, nullptr, nullptr, a.live);
  }
  return hipGetLastError();
}

}  // namespace moe
