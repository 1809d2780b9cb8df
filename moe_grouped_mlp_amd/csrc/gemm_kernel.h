#pragma once

// Persistent grouped GEMM for gfx950 (CDNA4) with fused MoE epilogues.
//
// One launch covers every expert: C_e = A_e . B_e for the row group of each
// local expert, with the per-group row counts (split sizes) and padded group
// starts read from device memory, so the host never learns the shapes
// ("Boosting MoE Training Throughput with Advanced Fusion Kernels",
// § "Eliminating host-device synchronization and CPU launch overhead").
//
// Work decomposition
//   * Output tile 256 x 256, 4 waves of 64 lanes in a 2 x 2 layout, each wave
//     owning a 128 x 128 sub-tile as 4 x 4 blocks of 32 x 32 MFMA outputs
//     (fp32 accumulators, 256 per lane).
//       bf16:  v_mfma_f32_32x32x16_bf16, 32-deep K steps (two MFMA K steps)
//       MXFP8: v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, one E8M0
//              scale per 32 K values per row), 64-deep K steps
//     Either way a K step moves 64 bytes per operand row, so both share the
//     loaders and the LDS image; a lane's MXFP8 operand (32 bytes) is exactly
//     the pair of 16-byte chunks a bf16 lane reads for its two K sub-steps.
//   * Operands go from HBM straight into LDS (buffer_load_dwordx4 ... lds):
//     two stages of 2 x 32 KB (128 bytes of every operand row each); the
//     loads of stage k + 2 go out as soon as every wave is done with stage k,
//     into its buffer, one stage ahead of their use.  Each lane fetches the
//     16-byte chunk that belongs at its slot of the swizzled image, so there
//     is no VGPR staging and no ds_write.  MXFP8 scales ride along: 2 KB per
//     stage (8 row groups x 128 bytes for A and for B, the tiled scale
//     layout).
//   * K-contiguous operands ([rows][K]: activations, and the weights of every
//     GEMM except the bf16 dgrad ones): LDS rows of 64 bytes, 16-byte chunk c
//     of row r stored at c ^ ((r >> 2) & 3), which keeps the operand reads (16
//     consecutive rows, same chunk, per LDS cycle) free of bank conflicts.
//   * bf16 dgrad GEMMs read the weight along its other axis ([K][N]): the tile
//     is copied as is (512-byte rows, chunk c at c ^ 4 (k % 8)) and the MFMA
//     operand is read with ds_read_b64_tr_b16 (LDS transpose read).  MXFP8
//     dgrad GEMMs instead take weight copies quantized along their K, so all
//     MXFP8 operands are K-contiguous.
//   * The K loop is unrolled by four over statically named stages, barriers
//     carry no fence (a fence would also wait for loads in flight), and the
//     loads of later stages are interleaved with the MFMAs.
//       bf16:  the operands of a stage's second sub-step are read while the
//              first sub-step's MFMAs run; the next stage is waited for in
//              the middle of a step.
//       MXFP8: the whole next stage is read into a second register set while
//              the current one feeds the MFMAs, so a stage's LDS slot is free
//              as soon as the step starts and loads run a full three steps
//              ahead.
//   * Persistent scheduling: every workgroup first builds, in LDS, the tile
//     prefix over the experts (ceil(M_e / BM) * ceil(N / BN) tiles each),
//     then walks tile ids with stride gridDim.  Consecutive workgroup ids
//     are dispatched round-robin over the 8 XCDs, so ids are remapped to give
//     each XCD a contiguous run of tiles; inside an expert tiles are ordered
//     in bands of `group_m` row tiles so that the tiles an XCD holds at one
//     time share their weight panels in that XCD's L2.  The first K steps of
//     the next tile are issued before the epilogue of the current one.
//
// Epilogues (fp32 math on the accumulators, bf16 round-to-nearest-even):
//   STORE  C = bf16(acc)                                     (FC2, FC1 dgrad)
//   GLU    z = bf16(acc); a = bf16(p * act(gate, up))        (FC1 forward)
//          The FC1 weight is interleaved in blocks of 64 rows (gate, up,
//          gate, up, ...), so a wave's 128 output columns hold 64 gate and
//          the 64 matching up columns, and each lane holds both halves of
//          its outputs in registers ("... Advanced Fusion Kernels",
//          § "Optimizing GLU activations with fused GEMM epilogues", Fig. 2).
//          Also raises amax = max|a|.
//   DGLU   with dA = acc: reads the saved z, recomputes s = act(g, u), writes
//          dz = bf16(dact(z, p * dA)) in the interleaved layout and the
//          per-row, per-N-tile partial sums of dA * s (the gradient of the
//          routing probability), reduced in fixed order by a second kernel
//          (same section: the backward epilogue applies dSwiGLU to the GEMM
//          output).
//   With MXFP8, GLU and DGLU also encode their stored bf16 output (a, dz) as
//   MXFP8 blocked along the row (the next GEMM's operand) and, optionally,
//   transposed and blocked along M inside each group (§ "Fused MXFP8 and
//   NVFP4 quantization": the epilogue writes the quantized tensor and its
//   transposed copy).  A row block's 32 values sit in a lane and its partner
//   (lane ^ 32); a column's 32 values sit in the 32 lanes of a half-wave and
//   are reduced with DPP, and the transposed codes are regrouped by a 4 x 4
//   byte transpose inside each quad so that every lane stores 4 rows of one
//   column at once.
#include <utility>

#include "act.h"
#include "common.h"
#include "kernels.h"
#include "mx.h"

namespace moe {
namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int kRowBytes = 128;        // bytes of every operand row per stage
constexpr int BK = kRowBytes / 2;     // bf16 K values per stage (64)
constexpr int BKQ = kRowBytes;        // E4M3 K values per stage (128)
constexpr int kStageBytes = BM * kRowBytes;  // 32 KB per operand per stage
constexpr int kThreads = 256;
constexpr int kWaveM = 128;  // rows of a wave's sub-tile
constexpr int kWaveN = 128;  // cols of a wave's sub-tile
constexpr int kMaxSplit = 8;  // K parts of a split tail tile

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;
typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int kStageS = 2048;  // bytes of MXFP8 scales per stage (A then B)

// Compile-time loop: f(integral_constant<int, 0>) ... f(<N-1>), so indices
// into accumulator arrays stay constants (registers, never scratch).
template <typename F, int... Is>
MOE_DEV void sfor_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
MOE_DEV void sfor(F&& f) {
  sfor_impl(f, std::make_integer_sequence<int, N>{});
}

MOE_DEV int swz(int row) { return (row ^ (row >> 3)) & 7; }

// ------------------------------------------------------------ loaders ---
// Buffer resource over `bytes` bytes at `base`.  Raw (untyped) loads whose
// VGPR offset reaches num_records return zero without touching memory; row
// indices therefore always go into the VGPR offset (the scalar offset only
// carries the K position, and never takes a valid row past its end), so
// partial tiles need no clamping.
MOE_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

constexpr int kOutOfRange = 0x7fffffff;  // VGPR offset past any num_records

MOE_DEV void dma16(__amdgpu_buffer_rsrc_t r, void* lds_block, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_block, 16, voff, soff, 0, 0);
}
MOE_DEV void dma4(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 4, voff, soff, 0, 0);
}

// Chunk swizzle of the K-contiguous LDS image: 16-byte chunk c of row r is
// stored at c ^ ((r >> 1) & 7).  An operand read (ds_read_b128) serves 16
// lanes per cycle: 16 consecutive rows, one logical chunk; rows 128 bytes
// apart land on bank groups 32 (r % 2) + 4 (c ^ ((r >> 1) & 7)), all 16
// distinct.
MOE_DEV int kswz(int row) { return (row >> 1) & 7; }

// K-contiguous tile of 256 rows x 128 bytes (64 bf16 or 128 E4M3 values) of
// a [rows][K] operand straight from HBM into one LDS stage.  Whole 128-byte
// lines: one DMA instruction moves 8 rows x 128 bytes (1 KB), so every L2
// request returns a full line (a 64-byte-per-row pattern halves what the L1
// can stream).  Wave w fills 1 KB blocks 8w .. 8w+7; lane l of block b
// lands on row 8 b + l / 8, stored chunk l % 8, so it fetches logical chunk
// (l % 8) ^ kswz(row).  With MXFP8 and K % 128 == 64 the chunks past K of
// the last stage are zero-filled per lane.
struct KLoader {
  __amdgpu_buffer_rsrc_t rsrc;
  int voff[8];    // bytes
  int kbyte[2];   // byte position of the lane's chunk in a stage row (even / odd j)

  // trim: bytes cut from the end of the range (a base moved into a row by
  // that many bytes then still ends where the last row does)
  MOE_DEV void init(const void* base, int64_t rows_avail, int ld_bytes, int wave, int lane,
                    int trim = 0) {
    const int64_t rows = rows_avail < 256 ? rows_avail : 256;
    rsrc = make_rsrc(base, static_cast<uint32_t>(rows > 0 ? rows * ld_bytes - trim : 0));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 64 * wave + 8 * j + (lane >> 3);
      const int kc = (lane & 7) ^ kswz(row);   // depends on j only through j % 2
      if (j < 2) kbyte[j] = kc * 16;
      voff[j] = row * ld_bytes + kc * 16;
    }
  }
  // kt: stage (128 bytes per row); valid == false fills the stage with
  // zeros; k_bytes: bytes per row of the operand (for the per-lane K tail)
  template <bool TAIL>
  MOE_DEV void issue(uint16_t* stage, int kt, int wave_s, bool valid, int k_bytes) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bool ok = valid;
      if constexpr (TAIL) ok = ok && (kt * kRowBytes + kbyte[j & 1] < k_bytes);
      dma16(rsrc, stage + (8 * wave_s + j) * 512, ok ? voff[j] : kOutOfRange,
            valid ? kt * kRowBytes : 0);
    }
  }
};

// N-contiguous tile of 64 K rows x 256 columns of a [K][N] bf16 matrix,
// copied as is (512-byte rows, whole lines) into one LDS stage: 16-byte chunk
// c of row k stored at c ^ (4 (k % 8)).  The MFMA operand is then read with
// the LDS transpose load.  Wave w fills 1 KB blocks 8w .. 8w+7 (two rows
// each).  Column chunks past N are clamped to the last chunk (their results
// are discarded), so every address lies inside the matrix.
struct NLoader {
  __amdgpu_buffer_rsrc_t rsrc;
  int voff[8];   // bytes

  MOE_DEV void init(const uint16_t* mat, uint32_t mat_bytes, int N, int col0, int wave, int lane) {
    rsrc = make_rsrc(mat, mat_bytes);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 16 * wave + 2 * j + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (row & 7));
      const int col = min(col0 + 8 * c, N - 8);
      voff[j] = (row * N + col) * 2;
    }
  }
  // soff: byte offset of the stage's first row, k0 * N * 2 (a wave-uniform
  // value the caller computes from the kernel arguments)
  MOE_DEV void issue(uint16_t* stage, int soff, int wave_s, bool valid) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      dma16(rsrc, stage + (8 * wave_s + j) * 512, valid ? voff[j] : kOutOfRange, valid ? soff : 0);
  }
  // Same, reading zeros for K rows at or past row_end: stage kk holds rows
  // 64 kk .. 64 kk + 63, lane l of instruction j row 16 w + 2 j + l / 32.
  MOE_DEV void issue_lim(uint16_t* stage, int soff, int wave_s, bool valid, int kk, int row_end,
                         int lane) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = valid && 64 * kk + 16 * wave_s + 2 * j + (lane >> 5) < row_end;
      dma16(rsrc, stage + (8 * wave_s + j) * 512, ok ? voff[j] : kOutOfRange, valid ? soff : 0);
    }
  }
};

// MXFP8 scales of one stage (two 64-deep K steps) for a 256-row A tile and
// a 256-row B tile.  In the tiled layout the scales of a 32-row group for
// steps 2 kt and 2 kt + 1 are one contiguous 128-byte run; the stage image
// is [A | B] x 8 row groups x [step][64 bytes] = 2 KB.  Waves 0, 1 copy A
// groups 4w .. 4w+3, waves 2, 3 copy B's, two dword DMAs each: lane l of
// instruction i fetches bytes 4 (l % 32) .. +3 of the run of group
// 4 (w % 2) + 2 i + l / 32, which lands at byte 4 l of the instruction's
// 256 bytes.  A step past K (K % 128 == 64) is zero-filled per lane.
template <bool F4>
struct ScaleLoader {
  // MXFP4: a stage holds four 64-deep steps (256 bytes per row group): lane
  // l of instruction i fetches bytes 4 l .. +3 of group 4 (w % 2) + i's run,
  // landing at byte 4 l of the instruction's 256 bytes; step l / 16.
  static constexpr int kInstr = F4 ? 4 : 2;
  __amdgpu_buffer_rsrc_t rsrc;
  int voff[kInstr];
  int step;       // step inside the stage this lane fetches

  // s_tile: scales of the tile's first row group; groups_avail: row groups
  // of 32 that exist from there on
  MOE_DEV void init(const uint8_t* s_tile, int64_t groups_avail, int K, int wave, int lane,
                    int trim = 0) {
    const int64_t groups = groups_avail < 8 ? (groups_avail > 0 ? groups_avail : 0) : 8;
    const int per_group = (K / 64) * 64;
    rsrc = make_rsrc(s_tile, static_cast<uint32_t>(groups > 0 ? groups * per_group - trim : 0));
    if constexpr (F4) {
      step = lane >> 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) voff[i] = (4 * (wave & 1) + i) * per_group + 4 * lane;
    } else {
      step = (lane >> 4) & 1;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        voff[i] = (4 * (wave & 1) + 2 * i + (lane >> 5)) * per_group + 4 * (lane & 31);
    }
  }
  MOE_DEV void issue(uint8_t* stage, int kt, int wave_s, bool valid, int k_steps64) {
    constexpr int kSteps = F4 ? 4 : 2;        // 64-deep steps per stage
    constexpr int kHalf = 8 * kSteps * 64;    // one operand's scales: 8 row groups
    const bool ok = valid && (kSteps * kt + step < k_steps64);
#pragma unroll
    for (int i = 0; i < kInstr; ++i)
      dma4(rsrc, stage + (wave_s >> 1) * kHalf + (wave_s & 1) * (kHalf / 2) + i * 256,
           ok ? voff[i] : kOutOfRange, valid ? kt * kSteps * 64 : 0);
  }
};

// z rows of a dGLU tile, staged for its epilogue in the two stage buffers
// (the K loop is done with them): chunk c holds tile rows wm * 128 + 32 c +
// r (r < 32) of both wave rows wm, rows of wm = 0 in the A buffer and of
// wm = 1 in the B buffer, ROWB bytes each (the tile's 512 gated or 256
// sReLU z columns).  Whole rows per DMA instruction (one 1 KB row, or two
// 512-byte rows), 16-byte chunk c of staged row r stored at c ^ (r % 16):
// the epilogue's 8-byte reads of one chunk by 32 rows then fall on 16
// distinct bank groups.  Rows past the group's data and chunks past the z
// row are zero-filled.  Wave w fills rows 16 (w % 2) .. +15 of half w / 2.
template <int ROWB>
struct ZLoader {
  static constexpr int kRowsPerInstr = 1024 / ROWB;   // 1 or 2
  static constexpr int kInstr = 16 / kRowsPerInstr;   // DMA loads per wave
  __amdgpu_buffer_rsrc_t rsrc;
  int rows;      // rows of the tile with data
  int ld_bytes;  // bytes per z row
  int col_byte;  // byte of the tile's first z column in a z row

  MOE_DEV void init(const uint16_t* zin, int64_t ldz, int64_t row0, int rows_valid, int zc0) {
    rows = rows_valid > 0 ? rows_valid : 0;
    ld_bytes = static_cast<int>(ldz * 2);
    col_byte = zc0 * 2;
    rsrc = make_rsrc(zin + row0 * ldz, static_cast<uint32_t>(static_cast<int64_t>(rows) * ldz * 2));
  }
  MOE_DEV void issue(uint16_t* a_st, uint16_t* b_st, int c, int wave_s, int lane) {
    uint16_t* st = wave_s < 2 ? a_st : b_st;
    const int wm = wave_s >> 1, r0 = 16 * (wave_s & 1);
#pragma unroll
    for (int j = 0; j < kInstr; ++j) {
      const int r = r0 + kRowsPerInstr * j + (kRowsPerInstr == 2 ? (lane >> 5) : 0);
      const int chunk = (kRowsPerInstr == 2 ? (lane & 31) : lane) ^ (r & 15);
      const int trow = wm * 128 + 32 * c + r;
      const int cb = col_byte + 16 * chunk;
      const bool ok = trow < rows && cb < ld_bytes;
      dma16(rsrc, st + (r0 + kRowsPerInstr * j) * (ROWB / 2), ok ? trow * ld_bytes + cb : kOutOfRange,
            0);
    }
  }
};

// 4 bf16 of a staged z row.  zb: the row's staged bytes plus the lane's
// column base (the 16-byte chunk 32 wn, gated, or 16 wn, and its 8-byte
// half); k < 32 (gated) or 16: the chunk within the lane's columns.  The
// swizzle r16 < 16 leaves the column base's chunk bits alone.
MOE_DEV uint2 zread(const char* zb, int r16, int k) {
  return *reinterpret_cast<const uint2*>(zb + ((k ^ r16) << 4));
}

// Makes v opaque to the optimizer at this point, so address arithmetic
// derived from it is recomputed where it is used instead of being hoisted
// out of the tile loop and kept live (spilled) across the K loop.
MOE_DEV int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most `n` vector
// memory loads of this wave are outstanding.
constexpr int wait_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)

// --------------------------------------------------- epilogue helpers ---
// 4 consecutive accumulator values v[r0 .. r0+3] -> 4 bf16 at p (8 bytes).
MOE_DEV void store_bf16x4(uint16_t* p, const f32x16& v, int r0) {
  uint2 w;
  w.x = pack_bf16x2(v[r0], v[r0 + 1]);
  w.y = pack_bf16x2(v[r0 + 2], v[r0 + 3]);
  *reinterpret_cast<uint2*>(p) = w;
}

MOE_DEV void store_f32x4_bf16(uint16_t* p, const float* v) {
  uint2 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<uint2*>(p) = w;
}

// Stores bf16(v[0..3]) and returns max |bf16(v[i])|.
MOE_DEV float store_bf16x4_amax(uint16_t* p, const float* v) {
  uint2 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<uint2*>(p) = w;
  const float a0 = fmaxf(fabsf(__uint_as_float(w.x << 16)), fabsf(__uint_as_float(w.x & 0xffff0000u)));
  const float a1 = fmaxf(fabsf(__uint_as_float(w.y << 16)), fabsf(__uint_as_float(w.y & 0xffff0000u)));
  return fmaxf(a0, a1);
}

MOE_DEV void load_bf16x4(const uint16_t* p, float* v) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(w.x << 16);
  v[1] = __uint_as_float(w.x & 0xffff0000u);
  v[2] = __uint_as_float(w.y << 16);
  v[3] = __uint_as_float(w.y & 0xffff0000u);
}

// Value of lane l ^ 32 (hf = l / 32) by v_permlane32_swap, a VALU
// exchange between the wave halves (no LDS round trip as with a shuffle).
// swap(a, b) gives the high half of a the low half of b and the low half of
// b the high half of a; with a = b = v a high lane finds its partner's value
// in the new a, a low lane in the new b.
MOE_DEV float partner32(float v, int hf) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(hf ? r[0] : r[1]);
}

// ------------------------------------------------ MXFP8 epilogue helpers ---
// The MXFP8 copies an epilogue writes of its [M_cap][n] bf16 output.
struct MxOut {
  uint8_t* q;     // rowwise codes [M_cap][n]
  uint8_t* s;     // their scales, tiled (R = M_cap, K = n)
  uint8_t* qT;    // transposed codes [n][M_cap] (nullable)
  uint8_t* sT;    // their scales, tiled (R = n, K = M_cap)
  int n;
  int64_t M_cap;
};

// A lane's 16 values of one 32 x 32 output block, as the packed bf16
// words the epilogue computed: w[rg] holds columns 8 rg + 4 hf .. + 3
// (hf = lane / 32) of the lane's row (lane % 32), value 0 in the low half
// of w[rg].x; zero for rows that hold no data.  Block maxima are taken on
// the bit patterns (bf16 magnitudes order like unsigned integers) and the
// codes come from gfx950's scaled conversions of the packed words.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// max |v| over 16 packed bf16 values, as a magnitude bit pattern.
MOE_DEV uint32_t bf16_amax_bits(const uint2 (&w)[4]) {
  u16x2_t m = {0, 0};
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) {
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, w[rg].x & 0x7fff7fffu));
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, w[rg].y & 0x7fff7fffu));
  }
  return m.x > m.y ? m.x : m.y;
}

// The maximum over a lane and its partner (lane ^ 32).
MOE_DEV uint32_t pair_max_bits(uint32_t am, int hf) {
  const auto pa = __builtin_amdgcn_permlane32_swap(am, am, false, false);
  return max(am, hf ? pa[0] : pa[1]);
}

// Block exponent from the block maximum's bit pattern: floor(log2 amax)
// (its exponent field) minus the exponent of the format's largest value
// (8 for E4M3, 2 for E2M1), at least -127.
template <int EMAX>
MOE_DEV int block_exponent(uint32_t amax_bits) {
  const int e = static_cast<int>(amax_bits >> 7) - 127 - EMAX;
  return e < -127 ? -127 : e;
}

// Rowwise MXFP8: the row's 32 values, this lane's and its partner's, give
// one scale; codes go to the block's 32 bytes of the row (q_lane: its half
// 16 hf ..), the scale to *s_byte.  The lane's four code words (columns
// 8 rg + 4 hf ..) are exchanged with the partner's (v_permlane32_swap) so
// that each lane stores 16 contiguous codes: the low lane columns 0 .. 15,
// the high lane 16 .. 31.  Returns the lane's own maximum (bit pattern).
MOE_DEV uint32_t mx_row_block(const uint2 (&w)[4], uint8_t* q_lane, uint8_t* s_byte, int hf) {
  const uint32_t am = bf16_amax_bits(w);
  const int e = block_exponent<8>(pair_max_bits(am, hf));
  const float scale = mx_scale_f32(e);
  uint32_t c[4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) c[rg] = mx_codes4_bf16(w[rg], scale);
  // swap(a, b): the high half of a takes the low half of b and the low half
  // of b the high half of a.  Low lanes end with (own c0, partner c0, own
  // c1, partner c1), high lanes with (partner c2, own c2, partner c3, own c3)
  const auto s0 = __builtin_amdgcn_permlane32_swap(c[0], c[2], false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(c[1], c[3], false, false);
  *reinterpret_cast<uint4*>(q_lane) = make_uint4(s0[0], s0[1], s1[0], s1[1]);
  if (hf == 0) *s_byte = mx_scale_code(e);
  return am;
}

// MXFP4 rowwise (no transposed copy): the row's 32 values give one E8M0
// scale and 32 E2M1 codes (16 bytes, element 2 i in the low nibble of byte
// i).  A lane's four values of columns 8 rg + 4 hf .. make a 16-bit half of
// the word of columns 8 rg ..; the halves are exchanged with the partner
// (v_permlane32_swap) so that the low lane stores the words of columns
// 0 .. 15 and the high lane 16 .. 31 (8 bytes each, q_lane = the block's
// row start + 8 hf).  Returns the lane's own maximum (bit pattern).
MOE_DEV uint32_t mx4_row_block(const uint2 (&w)[4], uint8_t* q_lane, uint8_t* s_byte, int hf) {
  const uint32_t am = bf16_amax_bits(w);
  const int e = block_exponent<2>(pair_max_bits(am, hf));
  const float scale = mx_scale_f32(e);
  uint32_t h[4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) h[rg] = mx4_codes4_bf16(w[rg], scale);
  // a = (h0, h1), b = (h2, h3); after the swap the low lane holds its own a
  // and the partner's a in b, the high lane the partner's b in a and its own b
  const auto sw = __builtin_amdgcn_permlane32_swap(h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                                   false, false);
  const uint32_t lo = sw[0], hi = sw[1];
  *reinterpret_cast<uint2*>(q_lane) =
      make_uint2((lo & 0xffffu) | (hi << 16), (lo >> 16) | (hi & 0xffff0000u));
  if (hf == 0) *s_byte = mx_scale_code(e);
  return am;
}

// Transposed: column c of the block is one MX block of the transposed copy
// (rows 32 rb .. 32 rb + 31).  The wave stages its 32 x 32 bf16 block in a
// private LDS tile (row pitch kTrPitch), then lane l gathers rows
// 16 (l / 32) .. +15 of column l % 32 with four LDS transpose loads
// (ds_read_b64_tr_b16: the 16 lanes of a group fetch a 4-row x 16-column
// piece, lane s taking row s / 4, columns 4 (s % 4) ..; lane i of the group
// receives column i of it, rows 0 .. 3), so a column's block maximum is one
// partner exchange (lane ^ 32) and its 16 codes are one 16-byte store.  LDS
// operations of one wave complete in order, so no barrier is needed and the
// tile is reused block after block.
constexpr int kTrPitch = 36;   // bf16 per staged row (8-byte aligned rows)
constexpr int kTrTile = 32 * kTrPitch;

// The lane's 16 values of its column: c[t4] holds rows 16 hf + 4 t4 .. + 3
// of column lane % 32 (packed bf16, the first row in the low half).
//
// The four transpose reads are one asm block that waits for them itself.
// The compiler cannot tell the staging tile from the stage buffers that LDS
// DMA loads may be filling at the time (the next z chunk, the next tile's
// first stage), so a read it issued would first wait for those loads, and
// for every store before them.  A wave's LDS operations complete in order,
// so the reads see the staging writes just before them (the memory clobber
// keeps those writes ahead of the block).
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
// REDERIVE: the addresses are re-derived from the lane at every block
// rather than kept live across the epilogue (the MXFP4 dGLU kernel spilled
// them and reloaded them in front of its stores).
template <bool REDERIVE>
MOE_DEV void col_gather(const uint2 (&w)[4], uint16_t* tr, int lane, uint2 (&c)[4]) {
  if constexpr (REDERIVE) lane = opaque(lane);
  const int row = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int rg = 0; rg < 4; ++rg)
    *reinterpret_cast<uint2*>(tr + row * kTrPitch + 8 * rg + 4 * hf) = w[rg];
  const int g = lane >> 4, s = lane & 15;
  const uint16_t* src = tr + (16 * (g >> 1) + (s >> 2)) * kTrPitch + 16 * (g & 1) + 4 * (s & 3);
  const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)src));
  static_assert(kTrPitch * 2 * 4 == 288, "row offsets of the reads below");
  u32x2_t r0, r1, r2, r3;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:288\n\t"
      "ds_read_b64_tr_b16 %2, %4 offset:576\n\t"
      "ds_read_b64_tr_b16 %3, %4 offset:864\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(addr)
      : "memory");
  c[0] = make_uint2(r0.x, r0.y);
  c[1] = make_uint2(r1.x, r1.y);
  c[2] = make_uint2(r2.x, r2.y);
  c[3] = make_uint2(r3.x, r3.y);
}

// q_lane: the lane's 16 codes of its column (rows 32 rb + 16 hf ..), s_byte:
// the column's scale.
MOE_DEV void mx_col_block(const uint2 (&w)[4], uint16_t* tr, uint8_t* q_lane, uint8_t* s_byte,
                          int lane) {
  const int hf = lane >> 5;
  uint2 c[4];
  col_gather<false>(w, tr, lane, c);
  const int e = block_exponent<8>(pair_max_bits(bf16_amax_bits(c), hf));
  const float scale = mx_scale_f32(e);
  uint4 q;
  q.x = mx_codes4_bf16(c[0], scale);
  q.y = mx_codes4_bf16(c[1], scale);
  q.z = mx_codes4_bf16(c[2], scale);
  q.w = mx_codes4_bf16(c[3], scale);
  *reinterpret_cast<uint4*>(q_lane) = q;
  if (hf == 0) *s_byte = mx_scale_code(e);
}

// MXFP4 transposed: the lane's 16 E2M1 codes of its column (8 bytes,
// rows 32 rb + 16 hf .., element 2 i in the low nibble of byte i).
MOE_DEV void mx4_col_block(const uint2 (&w)[4], uint16_t* tr, uint8_t* q_lane, uint8_t* s_byte,
                           int lane) {
  const int hf = lane >> 5;
  uint2 c[4];
  col_gather<true>(w, tr, lane, c);
  const int e = block_exponent<2>(pair_max_bits(bf16_amax_bits(c), hf));
  const float scale = mx_scale_f32(e);
  uint2 q;
  q.x = mx4_codes4_bf16(c[0], scale) | (mx4_codes4_bf16(c[1], scale) << 16);
  q.y = mx4_codes4_bf16(c[2], scale) | (mx4_codes4_bf16(c[3], scale) << 16);
  *reinterpret_cast<uint2*>(q_lane) = q;
  if (hf == 0) *s_byte = mx_scale_code(e);
}

// MXFP8: the lane's store addresses of its row block (32 rows starting at
// row block rb, the lane's row `row`) for the block at column 0; the block
// at a column col0 (a multiple of 32) adds wave-uniform offsets only
// (mx_block_out), so no per-lane 64-bit address arithmetic is repeated
// block by block.
struct MxBase {
  uint8_t* q;    // rowwise codes: o.q + row * n + 16 hf
  uint8_t* s;    // rowwise scale of (row, K block 0)
  uint8_t* qT;   // transposed codes of column lane % 32, rows 32 rb + 16 hf ..
  uint8_t* sT;   // transposed scale of (column lane % 32, row block rb)
};

MOE_DEV MxBase mx_base(const MxOut& o, int64_t row, int64_t rb, int lane) {
  const int hf = lane >> 5, c = lane & 31;
  MxBase b;
  b.q = o.q + row * o.n + 16 * hf;
  b.s = o.s + mx_scale_off(row, 0, o.n);
  b.qT = o.qT + static_cast<int64_t>(c) * o.M_cap + rb * 32 + 16 * hf;
  b.sT = o.sT + mx_scale_off(c, rb, o.M_cap);
  return b;
}

// Both MXFP8 copies of the block at columns col0 .. col0 + 31 (col0 % 32 == 0)
// of a row block whose rows all lie before the group's padded end.  With
// col0 a multiple of 32, the tiled scale offsets of (row, col0 / 32) and
// (col0 + lane % 32, rb) are those of block 0 plus terms in col0 alone.
// Returns the lane's maximum of the block (bit pattern).
MOE_DEV uint32_t mx_block_out(const uint2 (&w)[4], const MxOut& o, const MxBase& b,
                              uint16_t* tr, int col0, int lane) {
  uint8_t* const sb = b.s + (col0 >> 6) * 64 + ((col0 >> 5) & 1) * 32;
  const uint32_t am = mx_row_block(w, b.q + col0, sb, lane >> 5);
  if (o.qT)
    mx_col_block(w, tr, b.qT + static_cast<int64_t>(col0) * o.M_cap,
                 b.sT + static_cast<int64_t>(col0 >> 5) * (o.M_cap >> 6) * 64, lane);
  return am;
}

// MXFP4: store addresses of one 32-row block, rows r0b .. r0b + 31 (r0b a
// multiple of 32, wave-uniform; lane l owns row r0b + l % 32 and, in the
// transposed copy, column l % 32 of every 32-column block): the block's
// bases, wave-uniform so they stay in scalar registers, and the lane's
// offsets from them, 32-bit.  Holding no per-lane 64-bit addresses frees
// the vector registers whose spills the MXFP4 dGLU kernel reloaded in front
// of its stores (a reload waits for every store issued before it).  (The
// MXFP8 kernels measured slightly slower this way and keep MxBase.)
struct MxBase4 {
  uint8_t* q;         // rowwise codes of row r0b
  uint8_t* s;         // rowwise scales of row group r0b / 32, K block 0
  uint8_t* qT;        // transposed codes of column 0 at row r0b
  uint8_t* sT;        // transposed scale of (column 0, row block r0b / 32)
  uint32_t q_lane;    // (l % 32) rows + 8 hf bytes
  uint32_t qT_lane;   // (l % 32) columns + 8 hf bytes
};

// The lane offsets span at most 31 rows or columns of a copy: 32 bits for
// M_cap up to 2^27 and I up to 2^26 (checked by the host).
MOE_DEV MxBase4 mx_base4(const MxOut& o, int64_t r0b, int lane) {
  const uint32_t hf = static_cast<uint32_t>(lane) >> 5, c = static_cast<uint32_t>(lane) & 31;
  const int64_t rb = r0b >> 5;
  MxBase4 b;
  b.q = o.q + r0b * (o.n / 2);
  b.s = o.s + rb * (o.n >> 6) * 64;                 // mx_scale_off(r0b + c, 0, n) - c
  b.qT = o.qT + rb * 16;
  b.sT = o.sT + (rb >> 1) * 64 + (rb & 1) * 32;     // mx_scale_off(c, rb, M_cap) - c
  b.q_lane = c * static_cast<uint32_t>(o.n / 2) + 8u * hf;
  b.qT_lane = c * static_cast<uint32_t>(o.M_cap / 2) + 8u * hf;
  return b;
}

// Both MXFP4 copies (rowwise codes [M_cap][n / 2], transposed [n][M_cap / 2])
// of the block at columns col0 .. col0 + 31 (col0 % 32 == 0, wave-uniform);
// returns the lane's maximum as a bf16 magnitude pattern.  TR: the kernel
// writes the transposed copy (o.qT set).
template <bool TR>
MOE_DEV uint32_t mx4_block_out(const uint2 (&w)[4], const MxOut& o, const MxBase4& b,
                               uint16_t* tr, int col0, int lane) {
  const uint32_t c = static_cast<uint32_t>(lane) & 31;
  uint8_t* const sb = b.s + ((col0 >> 6) * 64 + ((col0 >> 5) & 1) * 32) + c;
  const uint32_t am = mx4_row_block(w, b.q + col0 / 2 + b.q_lane, sb, lane >> 5);
  if constexpr (TR)
    mx4_col_block(w, tr, b.qT + static_cast<int64_t>(col0) * (o.M_cap / 2) + b.qT_lane,
                  b.sT + static_cast<int64_t>(col0 >> 5) * (o.M_cap >> 6) * 64 + c, lane);
  return am;
}

// The block bases of either format (MXFP4: r0b is the block's first row).
template <bool F4OUT>
MOE_DEV auto mx_block_base(const MxOut& o, int64_t row, int64_t r0b, int lane) {
  if constexpr (F4OUT) return mx_base4(o, r0b, lane);
  else return mx_base(o, row, r0b >> 5, lane);
}

MOE_DEV void bf16x4_to_f32(uint2 w, float* v) {
  v[0] = __uint_as_float(w.x << 16);
  v[1] = __uint_as_float(w.x & 0xffff0000u);
  v[2] = __uint_as_float(w.y << 16);
  v[3] = __uint_as_float(w.y & 0xffff0000u);
}

// ------------------------------------------------------------ epilogues ---
// Where a tile's outputs sit in a lane.  The MFMA is issued with B as its
// first operand, so each 32x32 block holds C^T: lane l owns output row
// (l % 32) of the block and, in register r, column 8 (r / 4) + 4 (l / 32) +
// r % 4.  A lane thus writes runs of 4 consecutive columns (8 bytes).
struct TileCtx {
  int64_t row0;     // first row of the tile (padded layout)
  int rows_valid;   // rows of the tile that belong to the expert
  int col0;         // first output column
  int cols_valid;   // output columns inside N (multiple of 64)
  int rows_pad;     // rows of the tile before the group's padded end
  int n_t;          // column-tile index
  int m_lane;       // row of this lane inside the tile, block mi = 0
  int n_lane;       // first column of this lane inside the tile, block 0
  int mi_n;         // row blocks per wave: 4, or 2 in a half-height tile
  int wrow;         // rows per wave row: kWaveM, or kWaveM / 2 in a half-height tile
};

// Keeps a block of accumulators in AGPRs up to this point of the epilogue.
// Without it the register allocator copies all 256 accumulators to VGPRs as
// soon as the K loop ends and spills part of them to scratch; a spill reload
// is a vector memory load, so waiting for it also waits for every store the
// epilogue has issued before it.
MOE_DEV void acc_hold(f32x16& v) { asm volatile("" : "+a"(v)); }

// The FC1 bias of four consecutive tile columns from its LDS copy (sb:
// null when the layer has no bias; off: the first column's slot, a multiple
// of 4), and the activation input with the bias added.  Without a bias the
// accumulator is used as is (adding 0 would turn -0 into +0).
MOE_DEV void bias4(const float* sb, int off, float (&b)[4]) {
  if (sb) {
    const float4 v = *reinterpret_cast<const float4*>(sb + off);
    b[0] = v.x; b[1] = v.y; b[2] = v.z; b[3] = v.w;
  } else {
    b[0] = b[1] = b[2] = b[3] = 0.0f;
  }
}
MOE_DEV float with_bias(float v, const float* sb, float b) { return sb ? v + b : v; }

// EPI_STORE: C = bf16(acc)
// HOLD: keep each row block's accumulators in AGPRs until it is stored.
template <bool HOLD>
MOE_DEV void epi_store(f32x16 (&acc)[4][4], uint16_t* __restrict__ C, int64_t ldc,
                       const TileCtx& t) {
  sfor<4>([&](auto mi) {
    if constexpr (HOLD) sfor<4>([&](auto ni) { acc_hold(acc[mi][ni]); });
    const int m = t.m_lane + mi * 32;
    if (mi < t.mi_n && m < t.rows_valid) {
      uint16_t* crow = C + (t.row0 + m) * ldc + t.col0 + t.n_lane;
      sfor<4>([&](auto ni) {
        if (t.n_lane - (t.n_lane & 31) + ni * 32 < t.cols_valid) {
          sfor<4>([&](auto rg) {
            const f32x16& v = acc[mi][ni];
            uint2 w;
            w.x = pack_bf16x2_sw(v[4 * rg], v[4 * rg + 1]);
            w.y = pack_bf16x2_sw(v[4 * rg + 2], v[4 * rg + 3]);
            *reinterpret_cast<uint2*>(crow + ni * 32 + 8 * rg) = w;
          });
        }
      });
    }
    __builtin_amdgcn_sched_barrier(0);  // one 32-row block at a time
  });
}

// The routing probabilities of the lane's four rows (0 for rows past the
// group's data), loaded before the epilogue's first store: vector memory
// operations complete in order, so waiting for a load issued after stores
// would also wait for those stores.
MOE_DEV void row_probs(const float* __restrict__ probs, const TileCtx& t, float (&pr)[4]) {
  sfor<4>([&](auto mi) {
    const int m = t.m_lane + mi * 32;
    pr[mi] = m < t.rows_valid ? probs[t.row0 + m] : 0.0f;
  });
}

// EPI_GLU: z = bf16(acc) (may be null), a = bf16(p * act(gate, up)) with pr
// the probabilities of the lane's four rows (0 past the data); returns
// max |a| over this lane's outputs.  Gated: this wave's 128 packed columns
// [col0 + 128 wn, +128) are gate block q (blocks ni = 0, 1) then up block q
// (ni = 2, 3), so both halves of an output are in the same lane.
// sb: the tile's bias in LDS (null: none), see the kernel's bias staging.
template <int ACT>
MOE_DEV float epi_glu(f32x16 (&acc)[4][4], uint16_t* __restrict__ z, int64_t ldz,
                      uint16_t* __restrict__ a, int64_t lda, const float (&pr)[4],
                      const ActP& act, const TileCtx& t, int wn, int lane,
                      const float* sb) {
  float amax = 0.0f;
  if constexpr (ACT == MOE_ACT_SRELU) {
    sfor<4>([&](auto mi) {
      sfor<4>([&](auto ni) { acc_hold(acc[mi][ni]); });
      const int m = t.m_lane + mi * 32;
      if (mi < t.mi_n && m < t.rows_valid) {
        const int64_t row = t.row0 + m;
        const float p = pr[mi];
        sfor<4>([&](auto ni) { sfor<4>([&](auto rg) {
          const int n = t.n_lane + ni * 32 + 8 * rg;
          if (n < t.cols_valid) {
            if (z) store_bf16x4(z + row * ldz + t.col0 + n, acc[mi][ni], 4 * rg);
            float av[4], b[4];
            bias4(sb, n, b);
            sfor<4>([&](auto i) {
              const float zb = with_bias(acc[mi][ni][4 * rg + i], sb, b[i]);
              const float zc = fminf(fmaxf(zb, act.glo), act.ghi);
              const float rl = fmaxf(zc, 0.0f);
              av[i] = p * rl * rl;
            });
            amax = fmaxf(amax, store_bf16x4_amax(a + row * lda + t.col0 + n, av));
          }
        }); });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  } else if (wn * kWaveN < t.cols_valid) {
    const int q = (t.col0 + wn * kWaveN) / (2 * MOE_INTERLEAVE);
    sfor<4>([&](auto mi) {
      sfor<4>([&](auto ni) { acc_hold(acc[mi][ni]); });
      const int m = t.m_lane + mi * 32;
      if (mi < t.mi_n && m < t.rows_valid) {
        const int64_t row = t.row0 + m;
        const float p = pr[mi];
        sfor<2>([&](auto h) { sfor<4>([&](auto rg) {
          const int c = h * 32 + 8 * rg + 4 * (lane >> 5);  // 0..63 in the block
          if (z) {
            uint16_t* zrow = z + row * ldz + t.col0 + wn * kWaveN + c;
            store_bf16x4(zrow, acc[mi][h], 4 * rg);
            store_bf16x4(zrow + MOE_INTERLEAVE, acc[mi][h + 2], 4 * rg);
          }
          float av[4], bg[4], bu[4];
          bias4(sb, wn * 64 + c, bg);
          bias4(sb, 128 + wn * 64 + c, bu);
          sfor<4>([&](auto i) {
            av[i] = p * glu_eval<ACT>(with_bias(acc[mi][h][4 * rg + i], sb, bg[i]),
                                      with_bias(acc[mi][h + 2][4 * rg + i], sb, bu[i]), act).s;
          });
          amax = fmaxf(amax, store_bf16x4_amax(a + row * lda + q * MOE_INTERLEAVE + c, av));
        }); });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  return amax;
}

// EPI_DGLU, row block MI of the tile: acc = dA over logical columns
// [col0, col0 + BN).  Reads the lane's row of z (both halves) from its
// staged copy (zrow, see ZLoader), writes dz in the layout of z and returns
// this lane's partial sum of dA * s over the block; p is the row's
// probability.
//
// Addresses: the lane's logical columns are col0 + 128 wn + 4 h + 32 ni +
// 8 rg + i (h = lane / 32); with the 64-column interleave their gate
// columns are 2 col0 + 256 wn + 4 h + [128 (ni / 2) + 32 (ni % 2) + 8 rg] + i,
// a lane base plus a compile-time constant, and the up column is 64
// further: staged chunk 32 wn + 16 (ni / 2) + 4 (ni % 2) + rg (up: + 8),
// half h.  Whether a 32-column block lies inside N is uniform across the
// wave.
// sb: the tile's bias in LDS (null: none): gate half at [0, 256), up half
// at [256, 512), by column of the dA tile.
template <int ACT, int MI>
MOE_DEV float dglu_rows(f32x16 (&acc)[4][4], const char* zrow, uint16_t* __restrict__ dz,
                        int64_t lddz, float p, const ActP& act, const TileCtx& t, int wn,
                        int lane, const float* sb) {
  constexpr bool gated = ACT != MOE_ACT_SRELU;
  sfor<4>([&](auto ni) { acc_hold(acc[MI][ni]); });
  const int m = t.m_lane + MI * 32;
  if (m >= t.rows_valid) return 0.0f;
  const int h = lane >> 5, r16 = opaque(lane & 15);
  const int64_t row = t.row0 + m;
  const int lane_col = gated ? 2 * t.col0 + 256 * wn + 4 * h : t.col0 + 128 * wn + 4 * h;
  const char* zb = zrow + (gated ? 512 : 256) * wn + 8 * h;
  uint16_t* db = dz + row * lddz + lane_col;
  float dp = 0.0f;
  sfor<4>([&](auto ni) {
    if (wn * kWaveN + ni * 32 < t.cols_valid) {
      sfor<4>([&](auto rg) {
        float gz[4];
        if constexpr (gated) {
          constexpr int off = 128 * (ni / 2) + 32 * (ni % 2) + 8 * rg;
          constexpr int k = 16 * (ni / 2) + 4 * (ni % 2) + rg;
          float uz[4], bg[4], bu[4];
          bf16x4_to_f32(zread(zb, r16, k), gz);
          bf16x4_to_f32(zread(zb, r16, k + 8), uz);
          bias4(sb, 128 * wn + 32 * ni + 8 * rg + 4 * h, bg);
          bias4(sb, 256 + 128 * wn + 32 * ni + 8 * rg + 4 * h, bu);
          float dg[4], du[4];
          sfor<4>([&](auto i) {
            const float da = acc[MI][ni][4 * rg + i];
            const GluVal v =
                glu_eval<ACT>(with_bias(gz[i], sb, bg[i]), with_bias(uz[i], sb, bu[i]), act);
            const float ds = p * da;
            dg[i] = v.g_in ? ds * v.u * v.df : 0.0f;
            du[i] = v.u_in ? ds * v.f : 0.0f;
            dp += da * v.s;
          });
          store_f32x4_bf16(db + off, dg);
          store_f32x4_bf16(db + off + MOE_INTERLEAVE, du);
        } else {
          constexpr int off = 32 * ni + 8 * rg;
          bf16x4_to_f32(zread(zb, r16, 4 * ni + rg), gz);
          float d[4], b[4];
          bias4(sb, 128 * wn + 32 * ni + 8 * rg + 4 * h, b);
          sfor<4>([&](auto i) {
            const float da = acc[MI][ni][4 * rg + i];
            const float zi = with_bias(gz[i], sb, b[i]);
            const bool in = (zi >= act.glo) && (zi <= act.ghi);
            const float rl = fmaxf(fminf(fmaxf(zi, act.glo), act.ghi), 0.0f);
            d[i] = in ? p * da * 2.0f * rl : 0.0f;
            dp += da * rl * rl;
          });
          store_f32x4_bf16(db + off, d);
        }
      });
    }
  });
  return dp;
}

// EPI_GLU with MXFP8 copies of a (see epi_glu).  Rows of a 32-row block
// past the group's data but before its padded end get zero codes; a block
// past the padded end is not touched (it belongs to the next group).
// F4OUT: MXFP4 copies; TR (MXFP4): with the transposed copy.
template <int ACT, bool F4OUT = false, bool TR = true>
MOE_DEV float epi_glu_mx(f32x16 (&acc)[4][4], uint16_t* __restrict__ z, int64_t ldz,
                         uint16_t* __restrict__ a, int64_t lda, const float (&pr)[4],
                         const ActP& act, const TileCtx& t, int wn, int wm, int lane,
                         const MxOut& mo, uint16_t* tr, const float* sb) {
  constexpr bool gated = ACT != MOE_ACT_SRELU;
  const int hf = lane >> 5;
  if constexpr (F4OUT) {
    // the wave's row and column: uniform, so the block bases stay scalar
    wm = __builtin_amdgcn_readfirstlane(wm);
    wn = __builtin_amdgcn_readfirstlane(wn);
  }
  uint32_t am = 0;   // the lane's max |a| as a bf16 magnitude pattern
  sfor<4>([&](auto mi) {
    sfor<4>([&](auto ni) { acc_hold(acc[mi][ni]); });
    if (mi >= t.mi_n) return;   // a half-height tile's waves own two row blocks
    const int m = t.m_lane + mi * 32;
    const bool row_ok = m < t.rows_valid;
    const int blk = wm * t.wrow + mi * 32;
    const bool blk_ok = blk < t.rows_pad;
    const int64_t row = t.row0 + m;
    const float p = pr[mi];
    const auto mb = mx_block_base<F4OUT>(mo, row, t.row0 + blk, lane);
    if constexpr (gated) {
      if (wn * kWaveN < t.cols_valid) {
        const int q = (t.col0 + wn * kWaveN) / (2 * MOE_INTERLEAVE);
        sfor<2>([&](auto h) {
          uint2 wb[4];
          sfor<4>([&](auto rg) {
            const int c = h * 32 + 8 * rg + 4 * hf;
            if (row_ok && z) {
              uint16_t* zrow = z + row * ldz + t.col0 + wn * kWaveN + c;
              store_bf16x4(zrow, acc[mi][h], 4 * rg);
              store_bf16x4(zrow + MOE_INTERLEAVE, acc[mi][h + 2], 4 * rg);
            }
            float av[4], bg[4], bu[4];
            bias4(sb, wn * 64 + c, bg);
            bias4(sb, 128 + wn * 64 + c, bu);
            sfor<4>([&](auto i) {
              av[i] = p * glu_eval<ACT>(with_bias(acc[mi][h][4 * rg + i], sb, bg[i]),
                                        with_bias(acc[mi][h + 2][4 * rg + i], sb, bu[i]), act).s;
            });
            uint2 w = make_uint2(pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3]));
            if (!row_ok) w = make_uint2(0, 0);
            if (row_ok && a)
              *reinterpret_cast<uint2*>(a + row * lda + q * MOE_INTERLEAVE + c) = w;
            wb[rg] = w;
          });
          // rows past the padded end hold no data (zeros), so skipping
          // them leaves the maximum unchanged
          if (blk_ok) {
            const int cb = q * MOE_INTERLEAVE + h * 32;
            if constexpr (F4OUT) am = max(am, mx4_block_out<TR>(wb, mo, mb, tr, cb, lane));
            else am = max(am, mx_block_out(wb, mo, mb, tr, cb, lane));
          }
        });
      }
    } else {
      sfor<4>([&](auto ni) {
        if (wn * kWaveN + ni * 32 < t.cols_valid) {
          const int cb = t.col0 + wn * kWaveN + ni * 32;
          uint2 wb[4];
          sfor<4>([&](auto rg) {
            const int n = cb + 8 * rg + 4 * hf;
            if (row_ok && z) store_bf16x4(z + row * ldz + n, acc[mi][ni], 4 * rg);
            float av[4], b[4];
            bias4(sb, n - t.col0, b);
            sfor<4>([&](auto i) {
              const float zc =
                  fminf(fmaxf(with_bias(acc[mi][ni][4 * rg + i], sb, b[i]), act.glo), act.ghi);
              const float rl = fmaxf(zc, 0.0f);
              av[i] = p * rl * rl;
            });
            uint2 w = make_uint2(pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3]));
            if (!row_ok) w = make_uint2(0, 0);
            if (row_ok && a) *reinterpret_cast<uint2*>(a + row * lda + n) = w;
            wb[rg] = w;
          });
          if (blk_ok)
            if constexpr (F4OUT) am = max(am, mx4_block_out<TR>(wb, mo, mb, tr, cb, lane));
            else am = max(am, mx_block_out(wb, mo, mb, tr, cb, lane));
        }
      });
    }
    __builtin_amdgcn_sched_barrier(0);
  });
  return __uint_as_float(am << 16);
}

// EPI_DGLU with MXFP8 copies of dz, row block MI (see dglu_rows; pad rows
// as in epi_glu_mx).  With the 64-column interleave a 32-column block of dz
// holds only gate or only up columns.
template <int ACT, int MI, bool F4OUT = false, bool TR = true>
MOE_DEV float dglu_rows_mx(f32x16 (&acc)[4][4], const char* zrow,
                           uint16_t* __restrict__ dz, int64_t lddz, float p, const ActP& act,
                           const TileCtx& t, int wn, int wm, int lane, const MxOut& mo,
                           uint16_t* tr, const float* sb) {
  constexpr bool gated = ACT != MOE_ACT_SRELU;
  sfor<4>([&](auto ni) { acc_hold(acc[MI][ni]); });
  if constexpr (F4OUT) {
    // the wave's row and column: uniform, so the block bases stay scalar
    wm = __builtin_amdgcn_readfirstlane(wm);
    wn = __builtin_amdgcn_readfirstlane(wn);
  }
  const int h = lane >> 5, r16 = opaque(lane & 15);
  const int lane_col = gated ? 2 * t.col0 + 256 * wn + 4 * h : t.col0 + 128 * wn + 4 * h;
  const char* zb = zrow + (gated ? 512 : 256) * wn + 8 * h;
  const int m = t.m_lane + MI * 32;
  const bool row_ok = m < t.rows_valid;
  const int blk = wm * kWaveM + MI * 32;
  const bool blk_ok = blk < t.rows_pad;
  const int64_t row = t.row0 + m;
  const auto mb = mx_block_base<F4OUT>(mo, row, t.row0 + blk, lane);
  float dp = 0.0f;
  sfor<4>([&](auto ni) {
    if (wn * kWaveN + ni * 32 < t.cols_valid) {
      uint2 gw[4], uw[4];
      sfor<4>([&](auto rg) {
        float gz[4];
        if constexpr (gated) {
          constexpr int off = 128 * (ni / 2) + 32 * (ni % 2) + 8 * rg;
          constexpr int k = 16 * (ni / 2) + 4 * (ni % 2) + rg;
          float uz[4], bg[4], bu[4];
          bf16x4_to_f32(zread(zb, r16, k), gz);
          bf16x4_to_f32(zread(zb, r16, k + 8), uz);
          bias4(sb, 128 * wn + 32 * ni + 8 * rg + 4 * h, bg);
          bias4(sb, 256 + 128 * wn + 32 * ni + 8 * rg + 4 * h, bu);
          float dg[4], du[4];
          sfor<4>([&](auto i) {
            const float da = acc[MI][ni][4 * rg + i];
            const GluVal v =
                glu_eval<ACT>(with_bias(gz[i], sb, bg[i]), with_bias(uz[i], sb, bu[i]), act);
            const float ds = p * da;
            dg[i] = v.g_in ? ds * v.u * v.df : 0.0f;
            du[i] = v.u_in ? ds * v.f : 0.0f;
            dp += da * v.s;
          });
          uint2 wg = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
          uint2 wu = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
          if (!row_ok) wg = wu = make_uint2(0, 0);
          if (row_ok && dz) {
            uint16_t* db = dz + row * lddz + lane_col;
            *reinterpret_cast<uint2*>(db + off) = wg;
            *reinterpret_cast<uint2*>(db + off + MOE_INTERLEAVE) = wu;
          }
          gw[rg] = wg;
          uw[rg] = wu;
        } else {
          constexpr int off = 32 * ni + 8 * rg;
          bf16x4_to_f32(zread(zb, r16, 4 * ni + rg), gz);
          float d[4], b[4];
          bias4(sb, 128 * wn + 32 * ni + 8 * rg + 4 * h, b);
          sfor<4>([&](auto i) {
            const float da = acc[MI][ni][4 * rg + i];
            const float zi = with_bias(gz[i], sb, b[i]);
            const bool in = (zi >= act.glo) && (zi <= act.ghi);
            const float rl = fmaxf(fminf(fmaxf(zi, act.glo), act.ghi), 0.0f);
            d[i] = in ? p * da * 2.0f * rl : 0.0f;
            dp += da * rl * rl;
          });
          uint2 w = make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
          if (!row_ok) w = make_uint2(0, 0);
          if (row_ok && dz) *reinterpret_cast<uint2*>(dz + row * lddz + lane_col + off) = w;
          gw[rg] = w;
        }
      });
      if (blk_ok) {
        if constexpr (gated) {
          const int cbg = 2 * t.col0 + 256 * wn + 128 * (ni / 2) + 32 * (ni % 2);
          if constexpr (F4OUT) {
            mx4_block_out<TR>(gw, mo, mb, tr, cbg, lane);
            mx4_block_out<TR>(uw, mo, mb, tr, cbg + MOE_INTERLEAVE, lane);
          } else {
            mx_block_out(gw, mo, mb, tr, cbg, lane);
            mx_block_out(uw, mo, mb, tr, cbg + MOE_INTERLEAVE, lane);
          }
        } else {
          if constexpr (F4OUT) mx4_block_out<TR>(gw, mo, mb, tr, t.col0 + 128 * wn + 32 * ni, lane);
          else mx_block_out(gw, mo, mb, tr, t.col0 + 128 * wn + 32 * ni, lane);
        }
      }
    }
  });
  return dp;
}

// ------------------------------------------------------- block helpers ---
// Exclusive scan of one int per thread over the 256-thread block.
MOE_DEV int block_exclusive_scan(int v, int* s_tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    int t = s_tmp[w];
    if (w < wave) base += t;
    total += t;
  }
  __syncthreads();
  return base + x - v;
}

// ---------------------------------------------------------------- kernel --
// MX: A and B are E4M3 codes with tiled E8M0 scales (a_s, b_s); NN is then
// false.  The GLU / DGLU epilogues also write the MXFP8 copies of their
// output when MX.
// F4 (with MX, plain store only): MXFP4 operands, E2M1 codes packed two per
// byte (element 2 i in the low nibble of byte i) with the same tiled E8M0
// scales; K counts values, so a row holds K / 2 bytes and a 128-byte stage
// four 64-deep steps.
// ACTF: the activation (ACT), plus kActBias when the layer has an FC1 bias
// (g.bias non-null; GLU and DGLU epilogues only) and, in the MXFP4 GLU and
// dGLU kernels, kActTr when the epilogue writes the transposed copy.
template <int EPI, bool NN, int ACTF, bool MX, bool F4 = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_kernel(GemmArgs g) {
  constexpr int ACT = ACTF & ~(kActBias | kActTr);
  constexpr bool kBias = (ACTF & kActBias) != 0 && (EPI == EPI_GLU || EPI == EPI_DGLU);
  // transposed MX copies from the GLU / dGLU epilogue: MXFP8 decides at run
  // time (mx_qT), MXFP4 by instantiation (kActTr)
  constexpr bool kTrOut = !F4 || (ACTF & kActTr) != 0;
  // half-height tiles (an expert's last 128 rows or fewer) in the plain-store
  // and GLU kernels with K-contiguous weights: the dGLU epilogue streams z in
  // 64-row chunks laid out for full tiles, the weight gradient's rows are not
  // routed rows, and with [K][N] weights (the bf16 FC1 dgrad) a half tile
  // measured slower than a full one (its stage time is set by the B loads
  // and transposed reads, which do not shrink)
  constexpr bool kHalfTiles = (EPI == EPI_STORE || EPI == EPI_GLU) && !NN;
  static_assert(!(MX && NN), "MXFP8 operands are always K-contiguous");
  static_assert(!F4 || MX, "MXFP4 operands are microscaled");
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[kStageBytes / 2], sA1[kStageBytes / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t sB0[kStageBytes / 2], sB1[kStageBytes / 2];
  constexpr int kScaleBytes = MX ? (F4 ? 2 * kStageS : kStageS) : 4;
  __shared__ __attribute__((aligned(1024))) uint8_t sS0[kScaleBytes], sS1[kScaleBytes];
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_split[kMaxExperts];
  __shared__ int s_pad[kMaxExperts];
  __shared__ int s_tmp[kThreads / 64];
  __shared__ __attribute__((aligned(16))) float s_red[2 * BM];  // dprobs sums; the tile's bias
  // per-wave staging tiles of the transposed MXFP8 copies (MX epilogues)
  constexpr int kTrWords = (MX && kTrOut && (EPI == EPI_GLU || EPI == EPI_DGLU)) ? 4 * kTrTile : 4;
  __shared__ __attribute__((aligned(16))) uint16_t s_tr[kTrWords];

  const int tid = threadIdx.x;
  // measurement: the workgroup's shader cycles and constant-rate ticks
  int64_t clk_c0 = 0, clk_t0 = 0;
  if (g.clk) {
    clk_c0 = static_cast<int64_t>(__builtin_amdgcn_s_memtime());
    clk_t0 = static_cast<int64_t>(__builtin_amdgcn_s_memrealtime());
  }
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int wm_s = wave_s >> 1;   // wave row, in a scalar register
  const int wm = wave >> 1, wn = wave & 1;
  const int E = g.E;
  const int tiles_n = (g.N + BN - 1) / BN;
  constexpr int kElem = MX ? 1 : 2;  // bytes per operand element

  // ---- tile prefix over the experts (device-resident group sizes) ----
  // row tiles of an expert with n routed rows: ceil(n / BM), or for the
  // weight gradient ceil(P / BM) whatever n (an empty group stores zeros)
  auto tiles_m_of = [&](int n) {
    return EPI == EPI_WGRAD ? (g.wg_rows + BM - 1) / BM : (n + BM - 1) / BM;
  };
  const int per = (E + kThreads - 1) / kThreads;
  int mine = 0;
  for (int i = 0; i < per; ++i) {
    int e = tid * per + i;
    if (e < E) {
      const int n_raw = g.split[e];
      const int n = max(n_raw, 0);
      s_split[e] = n;
      s_pad[e] = g.padded[e];
      mine += tiles_m_of(n) * tiles_n;
      if (g.err && blockIdx.x == 0) {
        // the group [padded[e], padded[e] + n) must start at 0 or later and
        // end before the next group's start and inside M_cap
        const int64_t p0 = g.padded[e], p1 = g.padded[e + 1];
        if (n_raw < 0 || p0 < 0 || p0 + n > p1 || p0 + n > g.M_cap)
          set_err(g.err, MOE_DEVERR_BAD_OFFSETS);
      }
    }
  }
  int total;
  int run = block_exclusive_scan(mine, s_tmp, total);
  for (int i = 0; i < per; ++i) {
    int e = tid * per + i;
    if (e < E) {
      s_start[e] = run;
      run += tiles_m_of(s_split[e]) * tiles_n;
    }
  }
  if (tid == 0) s_start[E] = total;
  __syncthreads();

  // ---- XCD-aware id: give each XCD a contiguous run of tile ids ----
  const int G = gridDim.x;
  int vid = blockIdx.x;
  if (G % kNumXcd == 0) vid = (blockIdx.x % kNumXcd) * (G / kNumXcd) + blockIdx.x / kNumXcd;

  // per-lane LDS byte offsets of the MFMA operands.  K-contiguous image:
  // row base + 16-byte chunk (2 ks + lane / 32) ^ kswz(row) for the
  // 16-deep bf16 sub-step ks (0..3); the swizzle term is the same for rows
  // 32 apart.  [K][N] image (B of the bf16 dgrad GEMMs, read with
  // ds_read_b64_tr_b16): in each 16-lane group g, source lane s = 4 r + q
  // points at 4 consecutive columns nb + 16 (g % 2) + 4 q of row
  // 16 ks + 8 (g / 2) + 4 h + r, h selecting the first or second 4 of the
  // lane's 8 K values.
  const int khalf = lane >> 5;
  const int arow = wm * kWaveM + (lane & 31);
  const int brow = wn * kWaveN + (lane & 31);
  int a_off[4], b_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    a_off[ks] = arow * kRowBytes + ((2 * ks + khalf) ^ kswz(arow)) * 16;
    b_off[ks] = brow * kRowBytes + ((2 * ks + khalf) ^ kswz(brow)) * 16;
  }
  int btr_off[2][4];
  {
    const int gq = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int row = 8 * (gq >> 1) + 4 * h + (sl >> 2);   // + 16 ks
        const int c = wn * 16 + ni * 4 + 2 * (gq & 1) + ((sl & 3) >> 1);
        btr_off[h][ni] = row * 512 + (c ^ (4 * (row & 7))) * 16 + 8 * (sl & 1);
      }
  }
  // the bf16 weight gradient reads A from a [K][M] image too (rows of the
  // routed activations), with the same transpose reads, wave row wm
  constexpr bool kTN = EPI == EPI_WGRAD && !MX;
  int atr_off[2][4];
  if constexpr (kTN) {
    const int gq = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int row = 8 * (gq >> 1) + 4 * h + (sl >> 2);
        const int c = wm * 16 + mi * 4 + 2 * (gq & 1) + ((sl & 3) >> 1);
        atr_off[h][mi] = row * 512 + (c ^ (4 * (row & 7))) * 16 + 8 * (sl & 1);
      }
  }
  // MXFP8 scale byte of this lane's row (row group 4 wm + mi of A, 4 wn + ni
  // of B) for its K block (lane / 32) of 64-deep step j of a scale stage
  const int sa_off = 4 * wm * 128 + lane;
  const int sb_off = 1024 + 4 * wn * 128 + lane;
  // MXFP4: [A | B] x 8 row groups x [step (4)][64 bytes]
  const int sa_off4 = 4 * wm * 256 + lane;
  const int sb_off4 = 2048 + 4 * wn * 256 + lane;

  // ---- per-tile geometry --------------------------------------------
  struct TileInfo {
    int e, m_t, n_t, col0, cols_valid, rows_valid, rows_pad;
    int kbeg, kend;   // K stages of this work item
    int kshift;       // MXFP4 weight gradient: the group's first row (K starts there)
    int kvalid;       // MXFP4 weight gradient: the group's rows, rounded up to 32
    int part, slot;   // split-K part and partial-tile slot (parts > 1)
    int64_t row0;     // first row of A
    int64_t orow0;    // first row of C (row0, or e * P + row0 for EPI_WGRAD)
    bool half;        // half-height tile: an expert's last BM / 2 rows or fewer
  };
  auto tile_info = [&](int tile) {
    // expert owning this tile: last e with s_start[e] <= tile
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (s_start[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    TileInfo ti;
    ti.e = lo;
    const int local = tile - s_start[ti.e];
    const int tm_e = tiles_m_of(s_split[ti.e]);
    const int band = local / (g.group_m * tiles_n);
    const int first_m = band * g.group_m;
    const int gm = min(g.group_m, tm_e - first_m);
    const int rem = local - band * g.group_m * tiles_n;
    const int m_t = first_m + rem % gm;
    ti.m_t = m_t;
    ti.n_t = rem / gm;
    ti.col0 = ti.n_t * BN;
    ti.cols_valid = min(BN, g.N - ti.col0);
    if constexpr (EPI == EPI_WGRAD) {
      // rows of A^T are output rows; K is the group's padded row span of
      // the transposed copies (pad rows there hold zeros), whole stages
      ti.row0 = static_cast<int64_t>(m_t) * BM;
      ti.orow0 = static_cast<int64_t>(ti.e) * g.wg_rows + ti.row0;
      ti.rows_valid = min(BM, g.wg_rows - m_t * BM);
      ti.rows_pad = ti.rows_valid;
      // clamped to the stages of M_cap rows, so inconsistent offsets stay
      // inside the operands (bf16 stages are 64 rows; a last partial one is
      // cut by the row limit, and MXFP8 needs M_cap % 128 == 0)
      ti.half = false;
      if constexpr (F4) {
        // a stage is 256 rows but groups start at multiples of 128: K
        // counts from the group's first row (the loaders' bases move there)
        // and stops at its rows rounded up to a 32-row block, past which
        // the loads fill zeros; offsets are clamped into [0, M_cap]
        const int64_t p0 = min(max(static_cast<int64_t>(s_pad[ti.e]), int64_t{0}), g.M_cap);
        const int64_t n = min(max(static_cast<int64_t>(s_split[ti.e]), int64_t{0}), g.M_cap - p0);
        ti.kshift = static_cast<int>(p0);
        ti.kvalid = static_cast<int>((n + 31) / 32 * 32);
        ti.kbeg = 0;
        ti.kend = static_cast<int>((n + 255) / 256);
        return ti;
      }
      const int nk_all = (g.K * kElem + kRowBytes - 1) / kRowBytes;
      ti.kbeg = min(max(s_pad[ti.e], 0) * kElem / kRowBytes, nk_all);
      ti.kend = min(ti.kbeg + (s_split[ti.e] * kElem + kRowBytes - 1) / kRowBytes, nk_all);
      return ti;
    }
    ti.kshift = ti.kvalid = 0;
    ti.row0 = static_cast<int64_t>(s_pad[ti.e]) + static_cast<int64_t>(m_t) * BM;
    ti.orow0 = ti.row0;
    // rows_valid <= 0 only with inconsistent offsets: the tile then loads
    // zeros (its row range is empty) and stores nothing
    ti.rows_valid = static_cast<int>(
        min(static_cast<int64_t>(min(BM, s_split[ti.e] - m_t * BM)), g.M_cap - ti.row0));
    const int padded_rows =
        (s_split[ti.e] + MOE_GROUP_ALIGN - 1) / MOE_GROUP_ALIGN * MOE_GROUP_ALIGN;
    ti.rows_pad = static_cast<int>(
        min(static_cast<int64_t>(min(BM, padded_rows - m_t * BM)), g.M_cap - ti.row0));
    ti.half = kHalfTiles && g.half_tiles && s_split[ti.e] - m_t * BM <= BM / 2;
    return ti;
  };

  // stages of 128 bytes per row: 64 bf16 or 128 E4M3 K values; an MXFP8 K
  // with K % 128 == 64 ends in a half stage whose second half is zero-filled
  // bytes of an operand row, and between experts of B
  const int k_bytes = F4 ? g.K / 2 : g.K * kElem;
  const int64_t b_stride_bytes = F4 ? g.b_stride / 2 : g.b_stride * kElem;
  const int nk = (k_bytes + kRowBytes - 1) / kRowBytes;
  const int k_steps64 = g.K / 64;  // MXFP8 64-deep MFMA steps
  const char* A = static_cast<const char*>(g.A);
  const char* B = static_cast<const char*>(g.B);
  KLoader la;
  NLoader la_n;     // A of the bf16 weight gradient
  KLoader lb_k;
  NLoader lb_n;
  ScaleLoader<F4> ls;
  int row_end = 0;  // weight gradient: end of the group's rows (bf16 loads stop there)
  // K order of a tile: stages k_rot, k_rot + 1, ..., nk - 1, 0, ..., k_rot - 1
  // with k_rot = stride * (m_t + n_t) mod nk.  Tiles that share an operand
  // panel (same m_t or same n_t; an XCD holds a band of neighbouring tiles
  // at once) then reach a given K slice of it one or more stages apart
  // rather than in lockstep: the first one's L2 miss brings the slice in and
  // the others hit, instead of all of them waiting on the same MALL/HBM fetch.
  int k_rot = 0, k_beg = 0, k_len = nk;
  // bytes per operand row and 64-deep steps the loads stop at (MXFP4 weight
  // gradient: the tile's group, from its first row)
  constexpr bool kF4W = F4 && EPI == EPI_WGRAD;
  int k_lim = k_bytes, steps_lim = k_steps64;
  auto issue_stage = [&](uint16_t* a_st, uint16_t* b_st, uint8_t* s_st, int kt) {
    const bool valid = kt < k_len;
    int kk = kt + k_rot;
    if (kk >= k_len) kk -= k_len;
    kk += k_beg;
    if constexpr (kTN) {
      la_n.issue_lim(a_st, kk * BK * (g.wg_rows * 2), wave_s, valid, kk, row_end, lane);
      lb_n.issue_lim(b_st, kk * BK * (g.N * 2), wave_s, valid, kk, row_end, lane);
    } else {
      la.template issue<MX>(a_st, kk, wave_s, valid, kF4W ? k_lim : k_bytes);
      if constexpr (NN) lb_n.issue(b_st, kk * BK * (g.N * 2), wave_s, valid);
      else lb_k.template issue<MX>(b_st, kk, wave_s, valid, kF4W ? k_lim : k_bytes);
    }
    if constexpr (MX) ls.issue(s_st, kk, wave_s, valid, kF4W ? steps_lim : k_steps64);
  };
  // point the loaders at a tile (its first two stages are issued next)
  const int lane_k = lane, wave_k = wave;
  auto point_tile = [&](const TileInfo& ti) {
    const int nk_item = ti.kend - ti.kbeg;
    k_rot = nk_item > 0 ? (g.k_rot_stride * (ti.m_t + ti.n_t)) % nk_item : 0;
    k_beg = ti.kbeg;
    k_len = nk_item;
    const int64_t a_rows = EPI == EPI_WGRAD ? g.wg_rows : g.M_cap;
    // a half-height tile loads only its BM / 2 rows (the DMA of the other
    // rows falls outside the buffer and fills zeros without a fetch)
    const int64_t rows_all = ti.rows_valid > 0 ? a_rows - ti.row0 : 0;
    const int64_t rows_avail = ti.half ? min(rows_all, static_cast<int64_t>(BM / 2)) : rows_all;
    const int64_t arow0 = ti.rows_valid > 0 ? ti.row0 : 0;
    // the dGLU kernel recomputes the lane offsets per tile (hoisted, they
    // are spilled and reloaded in its epilogue)
    const int lane = EPI == EPI_DGLU ? opaque(lane_k) : lane_k;
    const int wave = EPI == EPI_DGLU ? opaque(wave_k) : wave_k;
    if constexpr (kTN) {
      // A and B are the routed activations [M_cap][P] and [M_cap][Q]; the
      // tile's P columns of A start at row0, its rows (K) are the group's
      row_end = s_pad[ti.e] + s_split[ti.e];
      la_n.init(reinterpret_cast<const uint16_t*>(A),
                static_cast<uint32_t>(static_cast<int64_t>(g.K) * g.wg_rows * 2), g.wg_rows,
                static_cast<int>(ti.row0), wave, lane);
    } else if constexpr (kF4W) {
      // the rows of A^T and B^T are read from the group's first row on
      k_lim = ti.kvalid / 2;
      steps_lim = ti.kvalid / 64 + (ti.kvalid % 64 != 0);
      la.init(A + arow0 * k_bytes + ti.kshift / 2, rows_avail, k_bytes, wave, lane,
              ti.kshift / 2);
    } else {
      la.init(A + arow0 * k_bytes, rows_avail, k_bytes, wave, lane);
    }
    const char* Bexp = B + static_cast<int64_t>(ti.e) * b_stride_bytes;
    if constexpr (NN) {
      lb_n.init(reinterpret_cast<const uint16_t*>(Bexp),
                static_cast<uint32_t>(static_cast<int64_t>(g.K) * g.N * 2), g.N, ti.col0, wave, lane);
    } else if constexpr (kF4W) {
      lb_k.init(Bexp + static_cast<int64_t>(ti.col0) * k_bytes + ti.kshift / 2, g.N - ti.col0,
                k_bytes, wave, lane, ti.kshift / 2);
    } else {
      lb_k.init(Bexp + static_cast<int64_t>(ti.col0) * k_bytes, g.N - ti.col0, k_bytes, wave, lane);
    }
    if constexpr (MX) {
      // waves 0, 1 copy the A scales, waves 2, 3 the B scales (a uniform
      // choice, so the buffer descriptor stays in scalar registers)
      const int64_t per_group = (g.K / 64) * 64;
      const bool a_side = wave_s < 2;
      const uint8_t* sbase =
          a_side ? g.a_s + (arow0 / 32) * per_group
                 : g.b_s + static_cast<int64_t>(ti.e) * g.b_s_stride + (ti.col0 / 32) * per_group;
      // MXFP4 weight gradient: the group's first 32-row block is an even
      // one (groups start at multiples of 128), so its pair of the tiled
      // layout starts kshift / 64 pairs (kshift bytes) into the row group
      const int sshift = kF4W ? ti.kshift : 0;
      ls.init(sbase + sshift, a_side ? rows_avail / 32 : (g.N - ti.col0) / 32, g.K, wave, lane,
              sshift);
    }
  };
  auto start_tile = [&](const TileInfo& ti) {
    point_tile(ti);
    issue_stage(sA0, sB0, sS0, 0);
    issue_stage(sA1, sB1, sS1, 1);
  };

  f32x16 acc[4][4];
  auto bare_barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // ------------------------------------------------------------ K loop ---
  // A stage holds NS MFMA sub-steps: four 16-deep bf16 steps or two 64-deep
  // MXFP8 steps.  Operands are double-buffered in registers across
  // sub-steps; the operands of sub-step j + 1 are read while the MFMAs of
  // sub-step j run.  Before the last sub-step of a stage every wave waits
  // for its reads of the stage and for the next stage's loads (the only
  // ones in flight), a barrier follows, the freed buffer starts loading the
  // stage after next, and the first operands of the next stage are read
  // while the last MFMAs of this one run.  So a stage's loads have a whole
  // stage of MFMA work (2048 cycles at full rate) to land.
  constexpr int NS = (MX && !F4) ? 2 : 4;
  bf16x8 fa[2][4], fb[2][4];   // bf16 operands
  i32x8 qa[2][4], qb[2][4];    // MXFP8 operands
  i32x4 pa[2][4], pb[2][4];    // MXFP4 operands
  int sca[2][4], scb[2][4];    // MXFP8 scales
  // operands of sub-step j of a stage into register set buf
  // half: a half-height tile, whose wave row wm owns rows 64 wm .. 64 wm + 63
  // (row blocks 0 and 1); the swizzle depends on the row modulo 16 only, so
  // its operand addresses are the full tile's moved back by 64 wm rows
  auto read_frags = [&](const uint16_t* a_st, const uint16_t* b_st, const uint8_t* s_st, auto j,
                        auto buf, auto half) {
    constexpr bool HALF = decltype(half)::value;
    static_assert(!HALF || (kHalfTiles && !kTN), "half-height tiles: K-contiguous A only");
    const char* ca = reinterpret_cast<const char*>(a_st) - (HALF ? wm_s * (kWaveM / 2) * kRowBytes : 0);
    const char* cb = reinterpret_cast<const char*>(b_st);
    // A scales: row group 4 wm + mi of the full tile, 2 wm + mi of a half one
    const uint8_t* s_a = s_st - (HALF ? wm_s * 2 * (F4 ? 256 : 128) : 0);
    constexpr int kMiA = HALF ? 2 : 4;   // A row blocks this wave reads
    constexpr int jj = decltype(j)::value;
    if constexpr (F4) {
      // a lane's 16-byte operand of a 64-deep step: 32 values, the whole
      // E8M0 block 2 j + h of the stage row (chunk 2 j + h, as a bf16
      // sub-step reads), scaled by that block's scale
      sfor<4>([&](auto i) {
        if constexpr (i < kMiA)
          pa[buf][i] = *reinterpret_cast<const i32x4*>(ca + a_off[jj] + i * 32 * kRowBytes);
        pb[buf][i] = *reinterpret_cast<const i32x4*>(cb + b_off[jj] + i * 32 * kRowBytes);
      });
      sfor<4>([&](auto i) {
        if constexpr (i < kMiA) sca[buf][i] = s_a[sa_off4 + i * 256 + jj * 64];
        scb[buf][i] = s_st[sb_off4 + i * 256 + jj * 64];
      });
    } else if constexpr (MX) {
      // a lane's 32-byte operand of a 64-deep step: chunks 4 j + h and
      // 4 j + 2 + h, the layout v_mfma_scale_f32_32x32x64_f8f6f4 takes
      sfor<4>([&](auto i) {
        if constexpr (i < kMiA) {
          const i32x4 lo = *reinterpret_cast<const i32x4*>(ca + a_off[2 * jj] + i * 32 * kRowBytes);
          const i32x4 hi =
              *reinterpret_cast<const i32x4*>(ca + a_off[2 * jj + 1] + i * 32 * kRowBytes);
          qa[buf][i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      });
      sfor<4>([&](auto i) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(cb + b_off[2 * jj] + i * 32 * kRowBytes);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(cb + b_off[2 * jj + 1] + i * 32 * kRowBytes);
        qb[buf][i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      });
      sfor<4>([&](auto i) {
        if constexpr (i < kMiA) sca[buf][i] = s_a[sa_off + i * 128 + jj * 64];
        scb[buf][i] = s_st[sb_off + i * 128 + jj * 64];
      });
    } else {
      if constexpr (kTN) {
        sfor<4>([&](auto mi) {
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16_t*)(ca + atr_off[0][mi] + jj * 16 * 512));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16_t*)(ca + atr_off[1][mi] + jj * 16 * 512));
          const v8i16 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          fa[buf][mi] = __builtin_bit_cast(bf16x8, both);
        });
      } else {
        sfor<4>([&](auto i) {
          if constexpr (i < kMiA)
            fa[buf][i] = *reinterpret_cast<const bf16x8*>(ca + a_off[jj] + i * 32 * kRowBytes);
        });
      }
      if constexpr (NN) {
        sfor<4>([&](auto ni) {
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16_t*)(cb + btr_off[0][ni] + jj * 16 * 512));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16_t*)(cb + btr_off[1][ni] + jj * 16 * 512));
          const v8i16 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          fb[buf][ni] = __builtin_bit_cast(bf16x8, both);
        });
      } else {
        sfor<4>([&](auto i) {
          fb[buf][i] = *reinterpret_cast<const bf16x8*>(cb + b_off[jj] + i * 32 * kRowBytes);
        });
      }
    }
  };
  // C^T blocks: B operand first, so a lane owns one output row
  auto mfma_all = [&](auto buf, auto half) {
    constexpr int kMiA = decltype(half)::value ? 2 : 4;
    sfor<kMiA>([&](auto mi) { sfor<4>([&](auto ni) {
      if constexpr (F4)
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            __builtin_shufflevector(pb[buf][ni], pb[buf][ni], 0, 1, 2, 3, -1, -1, -1, -1),
            __builtin_shufflevector(pa[buf][mi], pa[buf][mi], 0, 1, 2, 3, -1, -1, -1, -1),
            acc[mi][ni], 4, 4, 0, scb[buf][ni], 0, sca[buf][mi]);
      else if constexpr (MX)
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            qb[buf][ni], qa[buf][mi], acc[mi][ni], 0, 0, 0, scb[buf][ni], 0, sca[buf][mi]);
      else
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][ni], fa[buf][mi],
                                                              acc[mi][ni], 0, 0, 0);
    }); });
  };
  // LDS reads per sub-step and DMA loads per stage (per wave); a half-height
  // tile reads two A row blocks instead of four (and their scales)
  constexpr int kReads = F4 ? 16 : (MX ? 24 : (kTN ? 16 : (NN ? 12 : 8)));
  constexpr int kReadsHalf = F4 ? 12 : (MX ? 18 : (NN ? 10 : 6));
  constexpr int kLoads = 16 + (MX ? ScaleLoader<F4>::kInstr : 0);
  // issue order: reads spread between the 16 MFMAs of a sub-step (8 in a
  // half-height tile); in the last sub-step of a stage the next stage's DMA
  // loads go in between too (a DMA load blocks the wave until the address
  // unit takes it)
  auto pin = [&](auto half) {
    constexpr bool HALF = decltype(half)::value;
    constexpr int kR = HALF ? kReadsHalf : kReads;
    sfor<8>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(0x100, (kR + 7) / 8, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, HALF ? 1 : 2, 0);  // MFMA
    });
    __builtin_amdgcn_sched_barrier(0);
  };
  auto pin_load = [&](auto half) {
    constexpr bool HALF = decltype(half)::value;
    constexpr int kR = HALF ? kReadsHalf : kReads;
    if constexpr (kLoads > 16) __builtin_amdgcn_sched_group_barrier(0x020, kLoads - 16, 0);
    sfor<8>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);           // VMEM (DMA)
      __builtin_amdgcn_sched_group_barrier(0x100, (kR + 7) / 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, HALF ? 1 : 2, 0);
    });
    __builtin_amdgcn_sched_barrier(0);
  };
  // One stage (kt): cur = its buffers, nxt = the next stage's; the freed
  // cur buffers take stage kt + 2.
  auto stage = [&](const uint16_t* a_cur, const uint16_t* b_cur, const uint8_t* s_cur,
                   uint16_t* a_nxt, uint16_t* b_nxt, uint8_t* s_nxt, int kt, auto half) {
    sfor<NS - 1>([&](auto j) {
      __builtin_amdgcn_sched_barrier(0);
      constexpr int jj = decltype(j)::value;
      read_frags(a_cur, b_cur, s_cur, std::integral_constant<int, jj + 1>{},
                 std::integral_constant<int, (jj + 1) % 2>{}, half);
      mfma_all(std::integral_constant<int, jj % 2>{}, half);
      pin(half);
    });
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    bare_barrier();
    issue_stage(const_cast<uint16_t*>(a_cur), const_cast<uint16_t*>(b_cur),
                const_cast<uint8_t*>(s_cur), kt + 2);
    read_frags(a_nxt, b_nxt, s_nxt, std::integral_constant<int, 0>{},
               std::integral_constant<int, NS % 2>{}, half);
    mfma_all(std::integral_constant<int, (NS - 1) % 2>{}, half);
    pin_load(half);
  };
  // the K loop of one tile (its stages 0 and 1 issued already)
  auto k_loop = [&](auto half) {
    read_frags(sA0, sB0, sS0, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{},
               half);
    for (int kt = 0; kt < k_len; kt += 2) {
      stage(sA0, sB0, sS0, sA1, sB1, sS1, kt, half);
      stage(sA1, sB1, sS1, sA0, sB0, sS0, kt + 1, half);
    }
  };
  static_assert(NS % 2 == 0, "sub-step register sets alternate 0, 1 across stages");

  // ---- persistent tile loop -------------------------------------------
  // Work items.  Tiles fill `full` = floor(total / G) whole rounds; when the
  // remaining tail tiles would leave at least half the grid idle in a last
  // round, each tail tile is split along K into S parts (bf16 plain-store
  // GEMMs with a workspace only: for MXFP8 the split measured no faster and
  // its code made the allocator spill accumulators in the epilogue).  Every
  // workgroup derives the same split from the device-computed tile count,
  // so the host never needs it.
  const int full = (total / G) * G;
  const int tail = total - full;
  int S = 1;
  if constexpr (EPI == EPI_STORE && !MX) {
    if (g.split_ws && tail > 0 && 2 * tail <= G) {
      S = min(min(G / tail, g.split_max), max(1, nk / max(1, g.split_min_k)));
      if (tail * S > g.split_slots) S = max(1, g.split_slots / tail);
    }
  }
  const int items = full + tail * S;
  auto item_info = [&](int w) {
    int tile = w, part = 0;
    if (w >= full) {
      tile = full + (w - full) / S;
      part = (w - full) % S;
    }
    TileInfo ti = tile_info(tile);
    const int parts = w >= full ? S : 1;
    ti.part = part;
    ti.slot = tile - full;
    if constexpr (EPI != EPI_WGRAD) {   // the weight gradient's range is the group's
      ti.kbeg = part * nk / parts;
      ti.kend = (part + 1) * nk / parts;
    }
    return ti;
  };

  // GLU: a tile's row probabilities are loaded just before its first stages,
  // so the wait for stage 0 covers them and the epilogue, which runs with
  // its stores in flight, never waits on a load
  //
  // FC1 bias (instantiations with kActBias): the epilogue reads the tile's
  // bias from LDS (s_red).  GLU: thread t holds one value, loaded with the
  // row probabilities, for slot t: gated, the gate (t < 128) or up
  // (t >= 128) bias of logical column col0 / 2 + t % 128; sReLU, column
  // col0 + t.
  constexpr bool kGatedAct = ACT != MOE_ACT_SRELU;
  float pr_next[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float bias_next = 0.0f;
  auto load_probs = [&](const TileInfo& ti) {
    if constexpr (EPI == EPI_GLU) {
      const int ml = wm * (ti.half ? kWaveM / 2 : kWaveM) + (lane & 31);
      sfor<4>([&](auto mi) {
        const int m = ml + mi * 32;
        pr_next[mi] = m < ti.rows_valid ? g.probs[ti.row0 + m] : 0.0f;
      });
      if constexpr (kBias) {
        const float* be = g.bias + static_cast<int64_t>(ti.e) * g.N;
        if constexpr (kGatedAct) {
          const int half = g.N / 2, j = ti.col0 / 2 + (tid & 127);
          bias_next = j < half ? be[(tid < 128 ? 0 : half) + j] : 0.0f;
        } else {
          const int j = ti.col0 + tid;
          bias_next = j < g.N ? be[j] : 0.0f;
        }
      }
    }
  };

  // Dynamic scheduling (g.tile_ctr set and G a multiple of the XCD count):
  // the first round is static (item vid), later items come from work
  // counters, one per XCD, so a workgroup that starts late (its CU busy with
  // another kernel) leaves its share to the others.  XCD x's counter hands
  // out, in order, the items the static order gives XCD x (slot j of round
  // r >= 1: r G + x (G / 8) + j), keeping the XCD's band of tiles together
  // in its L2; once they are exhausted the workgroup takes from the other
  // XCDs' counters in turn.  Each item is handed out once.  Thread 0 fetches
  // the next item while the current one's K loop runs (the atomic is older
  // than the loop's last wait) and passes it on through LDS.
  const bool dyn = g.tile_ctr != nullptr && G % kNumXcd == 0;
  const int per_x = G / kNumXcd;
  const int my_x = blockIdx.x % kNumXcd;
  __shared__ int s_wnext;
  int fetched = 0;   // thread 0: the last counter value it took
  auto slot_item = [&](int x, int i) { return (1 + i / per_x) * G + x * per_x + i % per_x; };
  auto next_item = [&](int i) {
    int id = slot_item(my_x, i);
    for (int d = 1; d < kNumXcd && id >= items; ++d) {
      const int x = (my_x + d) % kNumXcd;
      id = slot_item(x, atomicAdd(g.tile_ctr + 16 * x, 1));
    }
    return id;
  };

  int w = vid;
  TileInfo cur{};
  if (w < items) {
    cur = item_info(w);
    load_probs(cur);
    start_tile(cur);
  }
  while (w < items) {
    float pr_tile[4];
    sfor<4>([&](auto mi) { pr_tile[mi] = pr_next[mi]; });
    const float bias_tile = bias_next;
    sfor<4>([&](auto mi) { sfor<4>([&](auto ni) { acc[mi][ni] = f32x16{}; }); });
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(kLoads));   // stage 0 landed
    bare_barrier();
    if (dyn && tid == 0) fetched = atomicAdd(g.tile_ctr + 16 * my_x, 1);
    if constexpr (kHalfTiles) {
      if (cur.half) k_loop(std::true_type{});
      else k_loop(std::false_type{});
    } else {
      k_loop(std::false_type{});
    }
    // the loads still in flight are zero fills; then every wave is done
    // with the stages and the next item may start loading
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    if (dyn && tid == 0) s_wnext = next_item(fetched);
    __syncthreads();
    const TileInfo t0 = cur;
    const bool split = w >= full && S > 1;
    w = dyn ? s_wnext : w + G;
    const bool more = w < items;
    if (more) {
      cur = item_info(w);
      // the dGLU epilogue stages z in the stage buffers first and starts
      // the next tile's loads itself
      if constexpr (EPI != EPI_DGLU) {
        load_probs(cur);
        start_tile(cur);
      }
    }

    // ------------------------------------------------------ epilogues ---
    TileCtx t;
    t.row0 = t0.orow0;
    t.rows_valid = t0.rows_valid;
    t.rows_pad = t0.rows_pad;
    t.col0 = t0.col0;
    t.cols_valid = t0.cols_valid;
    t.n_t = t0.n_t;
    t.mi_n = t0.half ? 2 : 4;
    t.wrow = t0.half ? kWaveM / 2 : kWaveM;
    t.m_lane = wm * t.wrow + (lane & 31);
    t.n_lane = wn * kWaveN + 4 * (lane >> 5);
    MxOut mo{g.mx_q, g.mx_s, g.mx_qT, g.mx_sT, g.mx_n, g.M_cap};
    if constexpr (EPI == EPI_STORE || EPI == EPI_WGRAD) {
      if (!MX && split) {
        // partial tile to slot (t0.slot, part); the part that arrives last
        // sums all S partials in part order (deterministic) and stores
        float4* ws = reinterpret_cast<float4*>(g.split_ws) +
                     static_cast<int64_t>(t0.slot * S + t0.part) * (64 * kThreads);
        sfor<4>([&](auto mi) { sfor<4>([&](auto ni) {
          acc_hold(acc[mi][ni]);
          sfor<4>([&](auto q) {
            const f32x16& a = acc[mi][ni];
            ws[((mi * 4 + ni) * 4 + q) * kThreads + tid] =
                make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
          });
        }); });
        // release: the partials reach memory before this part is counted
        // (another XCD's L2 may hold the tile that reads them)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (tid == 0) s_tmp[0] = atomicAdd(&g.split_cnt[t0.slot], 1);
        __syncthreads();
        if (s_tmp[0] == S - 1) {
          // acquire: drop stale cached copies before reading the partials
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          const float4* base = reinterpret_cast<const float4*>(g.split_ws) +
                               static_cast<int64_t>(t0.slot * S) * (64 * kThreads);
          sfor<4>([&](auto mi) { sfor<4>([&](auto ni) { acc[mi][ni] = f32x16{}; }); });
          for (int p = 0; p < S; ++p) {
            const float4* src = base + static_cast<int64_t>(p) * (64 * kThreads);
            sfor<4>([&](auto mi) { sfor<4>([&](auto ni) { sfor<4>([&](auto q) {
              const float4 v = src[((mi * 4 + ni) * 4 + q) * kThreads + tid];
              acc[mi][ni][4 * q] += v.x;
              acc[mi][ni][4 * q + 1] += v.y;
              acc[mi][ni][4 * q + 2] += v.z;
              acc[mi][ni][4 * q + 3] += v.w;
            }); }); });
          }
          epi_store<true>(acc, g.C, g.ldc, t);
        }
        __syncthreads();   // s_tmp is read by every thread above
      } else {
        epi_store<true>(acc, g.C, g.ldc, t);
      }
    } else if constexpr (EPI == EPI_GLU) {
      float amax;
      const float* sb = kBias ? s_red : nullptr;   // the tile's bias in LDS
      if constexpr (kBias) {
        s_red[tid] = bias_tile;
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        bare_barrier();
      }
      if constexpr (MX) {
        // lane values re-derived here, not kept live (and spilled) across
        // the K loop: a spill reload would wait on the next tile's loads
        const int lane_e = opaque(lane), wave_e = opaque(wave);
        TileCtx te = t;
        te.m_lane = (wave_e >> 1) * t.wrow + (lane_e & 31);
        te.n_lane = (wave_e & 1) * kWaveN + 4 * (lane_e >> 5);
        amax = epi_glu_mx<ACT, F4, kTrOut>(acc, g.C, g.ldc, g.act_out, g.ld_act, pr_tile, g.act, te,
                               wave_e & 1, wave_e >> 1, lane_e, mo, s_tr + wave_e * kTrTile,
                               sb);
      } else
        amax = epi_glu<ACT>(acc, g.C, g.ldc, g.act_out, g.ld_act, pr_tile, g.act, t, wn, lane,
                            sb);
      if (g.amax) {
        amax = wave_max_imm(amax);
        if (lane == 0) atomic_max_nonneg(g.amax, amax);
      }
    } else {
      // z of the tile's rows, 64 rows (row block mi of both wave rows) per
      // chunk, streams through the two stage buffers: chunks mi + 1 (and
      // from mi = 0 to 1 also mi + 2) load while block mi is computed; the
      // buffers then take the next tile's first two stages during the last
      // two blocks.
      constexpr bool kGated = ACT != MOE_ACT_SRELU;
      constexpr int kZRow = kGated ? 1024 : 512;
      using ZL = ZLoader<kZRow>;
      // the row probabilities first: a load issued after the chunks would
      // wait for them (vector memory operations complete in order)
      // lane-derived values are re-derived here rather than kept live (and
      // spilled) across the K loop
      const int lane_e = opaque(lane), wave_e = opaque(wave);
      const int wm_e = wave_e >> 1, wn_e = wave_e & 1;
      TileCtx te = t;
      te.m_lane = wm_e * kWaveM + (lane_e & 31);
      te.n_lane = wn_e * kWaveN + 4 * (lane_e >> 5);
      float pr[4];
      row_probs(g.probs, te, pr);
      // the tile's bias (before the chunks, like the probabilities): thread t
      // holds the gate (or sReLU) bias of dA column col0 + t and the up bias
      // of the same column, for LDS slots t and 256 + t
      float bz[2] = {0.0f, 0.0f};
      if constexpr (kBias) {
        const int tid_e = lane_e + 64 * wave_e;
        const int j = t.col0 + tid_e;
        const float* be = g.bias + static_cast<int64_t>(t0.e) * (kGated ? 2 * g.N : g.N);
        if (j < g.N) {
          bz[0] = be[j];
          if constexpr (kGated) bz[1] = be[g.N + j];
        }
      }
      const float* sb = kBias ? s_red : nullptr;
      ZL zl;
      zl.init(g.zin, g.ldz, t.row0, t.rows_valid, kGated ? 2 * t.col0 : t.col0);
      zl.issue(sA0, sB0, 0, wave_s, lane_e);
      zl.issue(sA1, sB1, 1, wave_s, lane_e);
      float dp[4];
      sfor<4>([&](auto mi) {
        constexpr int MI = decltype(mi)::value;
        uint16_t* za = MI % 2 ? sA1 : sA0;
        uint16_t* zb = MI % 2 ? sB1 : sB0;
        // chunk MI has landed once at most the loads issued after it are
        // outstanding: chunk MI + 1 (MI < 3), or stage 0 of the next tile
        // (issued after block 2), which may be in flight
        if constexpr (MI < 3) {
          __builtin_amdgcn_s_waitcnt(wait_vmcnt(ZL::kInstr));
        } else {
          if (more) __builtin_amdgcn_s_waitcnt(wait_vmcnt(kLoads));
          else __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
        }
        if constexpr (kBias && MI == 0) {
          // the bias loads are older than chunk 0's, so they have landed;
          // the previous tile's last reads of s_red were before its final
          // barrier
          const int tid_e = lane_e + 64 * wave_e;
          s_red[tid_e] = bz[0];
          if constexpr (kGated) s_red[256 + tid_e] = bz[1];
          __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        }
        bare_barrier();
        const char* zrow =
            reinterpret_cast<const char*>(wm_e ? zb : za) + (lane_e & 31) * kZRow;
        if constexpr (MX)
          dp[MI] = dglu_rows_mx<ACT, MI, F4, kTrOut>(acc, zrow, g.C, g.ldc, pr[MI], g.act, te, wn_e, wm_e,
                                         lane_e, mo, s_tr + (F4 ? __builtin_amdgcn_readfirstlane(wave_e) : wave_e) * kTrTile, sb);
        else
          dp[MI] = dglu_rows<ACT, MI>(acc, zrow, g.C, g.ldc, pr[MI], g.act, te, wn_e, lane_e,
                                      sb);
        __builtin_amdgcn_sched_barrier(0);
        // every wave is done reading the chunk before its buffer is reused
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        bare_barrier();
        if constexpr (MI < 2) {
          zl.issue(za, zb, MI + 2, wave_s, lane_e);
        } else if constexpr (MI == 2) {
          // stage 0 of the next tile goes out before the last row block
          if (more) {
            point_tile(cur);
            issue_stage(sA0, sB0, sS0, 0);
          }
        } else {
          if (more) issue_stage(sA1, sB1, sS1, 1);
        }
      });
      sfor<4>([&](auto mi) {
        // lanes l and l ^ 32 hold the same row: fixed-order pair sum
        const float v = dp[mi] + partner32(dp[mi], lane_e >> 5);
        if (lane_e < 32) s_red[wn_e * BM + te.m_lane + mi * 32] = v;
      });
      // LDS-only handoff: no fence, so the next tile's loads keep flying
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      bare_barrier();
      {
        const int m = lane_e + 64 * wave_e;  // the thread's id; BM == kThreads
        if (m < t.rows_valid)
          g.dp_part[(t.row0 + m) * g.n_part + t.n_t] = s_red[m] + s_red[BM + m];
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      bare_barrier();  // s_red is reused by the next tile
    }
  }
  if (g.clk && tid == 0) {
    const int64_t c1 = static_cast<int64_t>(__builtin_amdgcn_s_memtime());
    const int64_t t1 = static_cast<int64_t>(__builtin_amdgcn_s_memrealtime());
    g.clk[2 * blockIdx.x] = c1 - clk_c0;
    g.clk[2 * blockIdx.x + 1] = t1 - clk_t0;
  }
}


// Launch of one kernel family for the activation in g.act (SwiGLU with no
// clamp and no linear offset takes its own instantiation when there is no
// bias; a bias takes the instantiations flagged kActBias).
template <int EPI, bool NN, bool MX, int BIAS, bool F4 = false>
hipError_t launch_act_b(const GemmArgs& g, int grid, hipStream_t s) {
  dim3 blk(kThreads), grd(grid);
  switch (g.act.act) {
    case MOE_ACT_SWIGLU:
      if (!(BIAS & kActBias) && act_unclamped(g.act))
        grouped_gemm_kernel<EPI, NN, kActSwigluFree | BIAS, MX, F4><<<grd, blk, 0, s>>>(g);
      else
        grouped_gemm_kernel<EPI, NN, MOE_ACT_SWIGLU | BIAS, MX, F4><<<grd, blk, 0, s>>>(g);
      break;
    case MOE_ACT_GEGLU:
      grouped_gemm_kernel<EPI, NN, MOE_ACT_GEGLU | BIAS, MX, F4><<<grd, blk, 0, s>>>(g);
      break;
    case MOE_ACT_SRELU:
      grouped_gemm_kernel<EPI, NN, MOE_ACT_SRELU | BIAS, MX, F4><<<grd, blk, 0, s>>>(g);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int EPI, bool NN, bool MX>
hipError_t launch_act(const GemmArgs& g, int grid, hipStream_t s) {
  return g.bias ? launch_act_b<EPI, NN, MX, kActBias>(g, grid, s)
                : launch_act_b<EPI, NN, MX, 0>(g, grid, s);
}

// MXFP4 operands with an activation epilogue (no bias)
template <int EPI>
hipError_t launch_act_f4(const GemmArgs& g_in, int grid, hipStream_t s) {
  if (g_in.bias) return hipErrorInvalidValue;
  GemmArgs g = g_in;
  g.clk = gemm_clock_slot(grid);
  return g.mx_qT ? launch_act_b<EPI, false, true, kActTr, true>(g, grid, s)
                 : launch_act_b<EPI, false, true, 0, true>(g, grid, s);
}

}  // namespace

// One launcher per kernel family, each instantiated in a source file of its
// own (gemm_store.hip, gemm_glu_*.hip, gemm_dglu_*.hip, gemm_wgrad.hip) so the families
// compile in parallel.
hipError_t launch_gemm_store(const GemmArgs& g, bool b_nn, bool mx, int grid, hipStream_t s);
hipError_t launch_gemm_glu_bf16(const GemmArgs& g, int grid, hipStream_t s);
hipError_t launch_gemm_glu_mx(const GemmArgs& g, int grid, hipStream_t s);
hipError_t launch_gemm_dglu_bf16(const GemmArgs& g, int grid, hipStream_t s);
hipError_t launch_gemm_dglu_mx(const GemmArgs& g, int grid, hipStream_t s);
hipError_t launch_gemm_wgrad(const GemmArgs& g, bool mx, int grid, hipStream_t s);

}  // namespace moe
