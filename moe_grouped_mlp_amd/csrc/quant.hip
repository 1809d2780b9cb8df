// Stand-alone bf16 -> MXFP8 quantization (memory-bound): the weight copies
// the MXFP8 GEMMs read, from the bf16 master weights ("NVIDIA Transformer
// Engine 优化 MoE 生物基础模型训练", § "Challenge 3: quantization overhead":
// bf16 masters are cast before the low-precision GEMM; § "Challenge 2",
// Fig. 3: E4M3 codes with one E8M0 scale per 32 values).
//
// Both kernels produce the tiled scale layout in units of 32 output rows x
// 64 K positions (2 blocks per row); one wave encodes one such unit, each
// lane one whole 32-value block, so the block maximum needs no cross-lane
// reduction and the unit's 64 scale bytes are one contiguous store.
//   ROW  blocks along the contiguous axis: lane l reads 64 contiguous bytes
//        of row l % 32 (its block l / 32) with four 16-byte loads.
//   COL  blocks along rows, output transposed: a workgroup stages a 128-row
//        x 128-column slice of x in LDS; a thread encodes one column over 32
//        rows and writes those 32 codes contiguously.
//   BOTH the COL kernel also encodes the staged slice along its rows (a
//        thread per row block), so x is read once for both copies.
#include "common.h"
#include "kernels.h"
#include "mx.h"

namespace moe {
namespace {

// Encodes 32 bf16 values (as 16 packed words) into 32 codes (8 words);
// returns the scale exponent.  The codes come from gfx950's scaled
// conversion of the packed words (mx_codes4_bf16).
MOE_DEV int mx_encode32(const uint32_t (&w)[16], uint32_t (&codes)[8]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    m = max(m, bf16_abs_bits(w[i]));
    m = max(m, bf16_abs_bits(w[i] >> 16));
  }
  const int e = mx_exponent(__uint_as_float(m << 16));
  const float scale = mx_scale_f32(e);
#pragma unroll
  for (int i = 0; i < 8; ++i) codes[i] = mx_codes4_bf16(make_uint2(w[2 * i], w[2 * i + 1]), scale);
  return e;
}

MOE_DEV float amax_of_bits(uint32_t m) { return __uint_as_float(m << 16); }

// x [batch][rows][cols] -> q [batch][rows][cols], s tiled (R = rows, K = cols)
__global__ __launch_bounds__(256) void quant_row_kernel(const uint16_t* __restrict__ x,
                                                        int64_t x_stride, int batch, int rows,
                                                        int cols, uint8_t* __restrict__ q,
                                                        uint8_t* __restrict__ s,
                                                        float* __restrict__ amax,
                                                        const int32_t* __restrict__ live) {
  const int lane = threadIdx.x & 63;
  const int units_r = rows / 32, units_c = cols / 64;
  const int64_t units = static_cast<int64_t>(batch) * units_r * units_c;
  const int64_t per_batch_q = static_cast<int64_t>(rows) * cols;
  uint32_t wmax = 0;
  for (int64_t u = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / 64; u < units;
       u += static_cast<int64_t>(gridDim.x) * blockDim.x / 64) {
    const int bi = static_cast<int>(u / (static_cast<int64_t>(units_r) * units_c));
    if (live && live[bi] == 0) continue;   // wave-uniform
    const int rem = static_cast<int>(u % (static_cast<int64_t>(units_r) * units_c));
    const int ur = rem / units_c, uc = rem % units_c;
    const int row = ur * 32 + (lane & 31);
    const int col = uc * 64 + 32 * (lane >> 5);
    const uint4* src = reinterpret_cast<const uint4*>(x + bi * x_stride +
                                                      static_cast<int64_t>(row) * cols + col);
    uint32_t w[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = src[j];
      w[4 * j] = v.x; w[4 * j + 1] = v.y; w[4 * j + 2] = v.z; w[4 * j + 3] = v.w;
    }
    uint32_t codes[8];
    const int e = mx_encode32(w, codes);
    uint4* dst = reinterpret_cast<uint4*>(q + bi * per_batch_q + static_cast<int64_t>(row) * cols + col);
    dst[0] = make_uint4(codes[0], codes[1], codes[2], codes[3]);
    dst[1] = make_uint4(codes[4], codes[5], codes[6], codes[7]);
    s[bi * (per_batch_q / 32) + (static_cast<int64_t>(ur) * units_c + uc) * 64 + lane] =
        mx_scale_code(e);
    if (amax) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        wmax = max(wmax, max(bf16_abs_bits(w[i]), bf16_abs_bits(w[i] >> 16)));
    }
  }
  if (amax) {
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

// x [batch][rows][cols] -> q [batch][cols][rows], s tiled (R = cols, K = rows);
// F4: MXFP4 codes, q [batch][cols][rows / 2], no amax.
// ROW (the BOTH mode): also qr [batch][rows][cols] (F4: cols / 2 bytes a row),
// sr tiled (R = rows, K = cols), from the same staged slice.
constexpr int kColTileR = 128, kColTileC = 128;
constexpr int kColPitch = kColTileC + 2;  // bf16 per LDS row (odd word stride)

// Encodes one 32-value block (16 packed bf16 words) and stores its codes
// (MXFP8: 32 bytes, MXFP4: 16) at dst; returns the scale exponent.
template <bool F4>
MOE_DEV int encode_store32(const uint32_t (&w)[16], uint8_t* dst) {
  if constexpr (F4) {
    uint32_t packed[4];
    const int e = mx4_encode32(w, packed);
    *reinterpret_cast<uint4*>(dst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    return e;
  } else {
    uint32_t codes[8];
    const int e = mx_encode32(w, codes);
    reinterpret_cast<uint4*>(dst)[0] = make_uint4(codes[0], codes[1], codes[2], codes[3]);
    reinterpret_cast<uint4*>(dst)[1] = make_uint4(codes[4], codes[5], codes[6], codes[7]);
    return e;
  }
}

// A workgroup stages a slice of up to 128 rows x 128 columns: a column's
// codes of the slice (128 rows) are then one whole 128-byte line (MXFP8).
template <bool F4, bool ROW>
__global__ __launch_bounds__(256) void quant_col_kernel(const uint16_t* __restrict__ x,
                                                        int64_t x_stride, int batch, int rows,
                                                        int cols, uint8_t* __restrict__ q,
                                                        uint8_t* __restrict__ s,
                                                        float* __restrict__ amax,
                                                        uint8_t* __restrict__ qr,
                                                        uint8_t* __restrict__ sr,
                                                        const int32_t* __restrict__ live) {
  __shared__ uint16_t tile[kColTileR * kColPitch];
  const int t = threadIdx.x;
  const int tiles_r = (rows + kColTileR - 1) / kColTileR;
  const int tiles_c = (cols + kColTileC - 1) / kColTileC;
  const int64_t tiles = static_cast<int64_t>(batch) * tiles_r * tiles_c;
  const int64_t per_batch_q = static_cast<int64_t>(rows) * cols;
  constexpr int kDiv = F4 ? 2 : 1;   // values per code byte
  uint32_t wmax = 0;
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
      const int e = encode_store32<F4>(w, q + qoff / kDiv);
      s[bi * (per_batch_q / 32) + mx_scale_off(cc, r0 / 32 + h, rows)] =
          static_cast<uint8_t>(e + 127);
      if (!F4 && amax) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          wmax = max(wmax, max(bf16_abs_bits(w[i]), bf16_abs_bits(w[i] >> 16)));
      }
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
        const int e = encode_store32<F4>(w, qr + (bi * per_batch_q + row * cols + col) / kDiv);
        sr[bi * (per_batch_q / 32) + mx_scale_off(row, col / 32, cols)] =
            static_cast<uint8_t>(e + 127);
      }
    }
    __syncthreads();
  }
  if (amax) {
    const float m = wave_max(amax_of_bits(wmax));
    if ((t & 63) == 0) atomic_max_nonneg(amax, m);
  }
}

int quant_grid(int64_t work_items, int per_block) {
  int64_t b = (work_items + per_block - 1) / per_block;
  if (b > 8192) b = 8192;
  return b < 1 ? 1 : static_cast<int>(b);
}

// x [batch][rows][cols] -> q [batch][rows][cols / 2] (two E2M1 codes a byte,
// element 2 i in the low nibble), s tiled (R = rows, K = cols); the MXFP8
// row kernel's unit walk, a lane encoding one 32-value block into 16 bytes.
// Scale 2^(floor(log2 amax) - 2), 2 being the exponent of E2M1's largest
// value 6; the bf16 input times 2^-e is exact in fp32.
__global__ __launch_bounds__(256) void quant_row_fp4_kernel(const uint16_t* __restrict__ x,
                                                            int64_t x_stride, int batch,
                                                            int rows, int cols,
                                                            uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ s,
                                                            const int32_t* __restrict__ live) {
  const int lane = threadIdx.x & 63;
  const int units_r = rows / 32, units_c = cols / 64;
  const int64_t units = static_cast<int64_t>(batch) * units_r * units_c;
  const int64_t per_batch = static_cast<int64_t>(rows) * cols;
  for (int64_t u = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / 64; u < units;
       u += static_cast<int64_t>(gridDim.x) * blockDim.x / 64) {
    const int bi = static_cast<int>(u / (static_cast<int64_t>(units_r) * units_c));
    if (live && live[bi] == 0) continue;   // wave-uniform
    const int rem = static_cast<int>(u % (static_cast<int64_t>(units_r) * units_c));
    const int ur = rem / units_c, uc = rem % units_c;
    const int row = ur * 32 + (lane & 31);
    const int col = uc * 64 + 32 * (lane >> 5);
    const uint4* src = reinterpret_cast<const uint4*>(x + bi * x_stride +
                                                      static_cast<int64_t>(row) * cols + col);
    uint32_t w[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = src[j];
      w[4 * j] = v.x; w[4 * j + 1] = v.y; w[4 * j + 2] = v.z; w[4 * j + 3] = v.w;
    }
    uint32_t packed[4];
    const int e = mx4_encode32(w, packed);
    uint4* dst = reinterpret_cast<uint4*>(q + bi * (per_batch / 2) +
                                          (static_cast<int64_t>(row) * cols + col) / 2);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    s[bi * (per_batch / 32) + (static_cast<int64_t>(ur) * units_c + uc) * 64 + lane] =
        static_cast<uint8_t>(e + 127);
  }
}

}  // namespace

hipError_t launch_quantize_mxfp4(const moe_quant_args& a, hipStream_t st) {
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  if (a.mode == MOE_QUANT_ROW) {
    const int64_t units = static_cast<int64_t>(a.batch) * (a.rows / 32) * (a.cols / 64);
    quant_row_fp4_kernel<<<quant_grid(units, 4), 256, 0, st>>>(x, a.x_stride, a.batch, a.rows,
                                                               a.cols, a.q, a.s, a.live);
  } else {
    const int64_t tiles = static_cast<int64_t>(a.batch) * ((a.rows + kColTileR - 1) / kColTileR) *
                          ((a.cols + kColTileC - 1) / kColTileC);
    // BOTH: the COL copy goes to qT / sT, the ROW copy to q / s
    if (a.mode == MOE_QUANT_BOTH)
      quant_col_kernel<true, true><<<quant_grid(tiles, 1), 256, 0, st>>>(
          x, a.x_stride, a.batch, a.rows, a.cols, a.qT, a.sT, nullptr, a.q, a.s, a.live);
    else
      quant_col_kernel<true, false><<<quant_grid(tiles, 1), 256, 0, st>>>(
          x, a.x_stride, a.batch, a.rows, a.cols, a.q, a.s, nullptr, nullptr, nullptr, a.live);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp8(const moe_quant_args& a, hipStream_t st) {
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  if (a.mode == MOE_QUANT_ROW) {
    const int64_t units = static_cast<int64_t>(a.batch) * (a.rows / 32) * (a.cols / 64);
    quant_row_kernel<<<quant_grid(units, 4), 256, 0, st>>>(x, a.x_stride, a.batch, a.rows, a.cols,
                                                           a.q, a.s, a.amax, a.live);
  } else {
    const int64_t tiles = static_cast<int64_t>(a.batch) * ((a.rows + kColTileR - 1) / kColTileR) *
                          ((a.cols + kColTileC - 1) / kColTileC);
    if (a.mode == MOE_QUANT_BOTH)
      quant_col_kernel<false, true><<<quant_grid(tiles, 1), 256, 0, st>>>(
          x, a.x_stride, a.batch, a.rows, a.cols, a.qT, a.sT, a.amax, a.q, a.s, a.live);
    else
      quant_col_kernel<false, false><<<quant_grid(tiles, 1), 256, 0, st>>>(
          x, a.x_stride, a.batch, a.rows, a.cols, a.q, a.s, a.amax, nullptr, nullptr, a.live);
  }
  return hipGetLastError();
}

}  // namespace moe
