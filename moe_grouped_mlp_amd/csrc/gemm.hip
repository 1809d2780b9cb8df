// Persistent grouped GEMM for gfx950 (CDNA4) with fused MoE epilogues.
//
// One launch covers every expert: C_e = A_e . B_e for the row group of each
// local expert, with the per-group row counts (split sizes) and padded group
// starts read from device memory, so the host never learns the shapes
// ("Boosting MoE Training Throughput with Advanced Fusion Kernels",
// § "Eliminating host-device synchronization and CPU launch overhead").
//
// Work decomposition
//   * Tile 256 x 256 x 64 (BM x BN x BK), 4 waves of 64 lanes in a 2 x 2
//     layout, each wave owning a 128 x 128 sub-tile as 4 x 4 blocks of the
//     v_mfma_f32_32x32x16_bf16 instruction (fp32 accumulators, 256 per lane).
//   * A (activations, [M][K] K-contiguous) and B (weights) are staged through
//     registers into a double-buffered LDS tile (2 x 64 KB); one barrier per
//     K step; the global loads of step k+1 are in flight while step k runs.
//   * B comes either as [N][K] ("NT": forward GEMMs, W1 and W2 as stored) or
//     as [K][N] ("NN": the dgrad GEMMs read the same weights along their
//     other axis).  NN tiles are transposed in registers (8 x 8 blocks of
//     bf16 with v_perm_b32) before the LDS store, so both layouts feed the
//     MFMA from the same K-contiguous LDS image.
//   * LDS rows are 128 B (64 bf16); the 16-byte chunk c of row r is stored
//     at chunk c ^ ((r ^ r >> 3) & 7), which keeps the MFMA operand reads
//     (8 consecutive rows, same chunk) and the transposed NN stores (rows
//     8 apart) free of bank conflicts.
//   * Persistent scheduling: every workgroup first builds, in LDS, the tile
//     prefix over the experts (ceil(M_e / BM) * ceil(N / BN) tiles each),
//     then walks tile ids with stride gridDim.  Consecutive workgroup ids
//     are dispatched round-robin over the 8 XCDs, so ids are remapped to give
//     each XCD a contiguous run of tiles; inside an expert tiles are ordered
//     in bands of `group_m` row tiles so that the tiles an XCD holds at one
//     time share their weight panels in that XCD's L2.
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
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kWaveM = 128;  // rows of a wave's sub-tile
constexpr int kWaveN = 128;  // cols of a wave's sub-tile

MOE_DEV int swz(int row) { return (row ^ (row >> 3)) & 7; }

// -------------------------------------------------------- activations ---
MOE_DEV float sigmoid_f(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Unscaled gated activation s and its partial derivatives.
struct GluVal {
  float s;     // act(g) * u
  float f;     // act(g)
  float df;    // act'(g)
  float u;     // clamped linear half (+ offset)
  bool g_in, u_in;
};

MOE_DEV GluVal glu_eval(float g_pre, float u_pre, const ActP& p) {
  GluVal r;
  float g = fminf(fmaxf(g_pre, p.glo), p.ghi);
  r.u = fminf(fmaxf(u_pre, p.llo), p.lhi) + p.loff;
  r.g_in = (g_pre >= p.glo) && (g_pre <= p.ghi);
  r.u_in = (u_pre >= p.llo) && (u_pre <= p.lhi);
  if (p.act == MOE_ACT_GEGLU) {
    const float kInvSqrt2 = 0.70710678118654752f;
    const float kInvSqrt2Pi = 0.39894228040143268f;
    float cdf = 0.5f * (1.0f + erff(g * kInvSqrt2));
    r.f = g * cdf;
    r.df = cdf + g * kInvSqrt2Pi * __expf(-0.5f * g * g);
  } else {
    float sg = sigmoid_f(p.beta * g);
    r.f = g * sg;
    r.df = sg * (1.0f + p.beta * g * (1.0f - sg));
  }
  r.s = r.f * r.u;
  return r;
}

// ------------------------------------------------------------ loaders ---
// Buffer resource over `bytes` bytes at `base`.  Raw (untyped) loads whose
// VGPR offset reaches num_records return zero without touching memory; row
// indices therefore always go into the VGPR offset (the scalar offset only
// carries the K position, which stays inside a row), so partial tiles need
// no clamping.
MOE_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

MOE_DEV i32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

// K-contiguous [ROWS][BK] tile -> LDS, 16-byte chunks.  Thread t moves the
// chunk (row t/8 + 32 i, k-chunk t%8) for i < ROWS/32.
template <int ROWS>
struct NTLoader {
  static constexpr int kIters = ROWS * BK / 8 / kThreads;
  __amdgpu_buffer_rsrc_t rsrc;
  int voff;       // bytes, chunk i = 0
  int row_step;   // bytes between chunk rows i and i+1 (32 rows)
  int l0, l1;     // LDS chunk index for even / odd i (swizzle flips bit 2)
  i32x4 reg[kIters];

  MOE_DEV void init(const uint16_t* base, int64_t rows_avail, int ld, int tid) {
    const int64_t rows = rows_avail < ROWS ? rows_avail : ROWS;
    rsrc = make_rsrc(base, static_cast<uint32_t>(rows * ld * 2));
    const int row = tid >> 3, kc = tid & 7;
    voff = (row * ld + kc * 8) * 2;
    row_step = 32 * ld * 2;
    l0 = row * 8 + (kc ^ swz(row));
    l1 = row * 8 + (kc ^ swz(row) ^ 4);
  }
  MOE_DEV void load(int k0) {
#pragma unroll
    for (int i = 0; i < kIters; ++i) reg[i] = buf_load16(rsrc, voff + i * row_step, k0 * 2);
  }
  MOE_DEV void store(uint16_t* s) {
#pragma unroll
    for (int i = 0; i < kIters; ++i)
      *reinterpret_cast<i32x4*>(s + ((i & 1 ? l1 : l0) + 256 * i) * 8) = reg[i];
  }
};

// N-contiguous [BK][BN] tile of a [K][N] matrix -> transposed LDS [BN][BK].
// Each thread moves one 8 (k) x 8 (n) block: 8 row loads of 16 bytes, an
// in-register 8x8 transpose of bf16 pairs (v_perm_b32), 8 LDS stores.
// Column blocks past N are clamped to the last block (their results are
// discarded by the epilogue), so every address lies inside the matrix.
struct NNLoader {
  static_assert(BN / 8 * (BK / 8) == kThreads, "one 8x8 block per thread");
  __amdgpu_buffer_rsrc_t rsrc;
  int voff;      // bytes
  int ld2;       // row pitch in bytes
  int nb, kb;
  i32x4 reg[8];

  MOE_DEV void init(const uint16_t* mat, uint32_t mat_bytes, int ld, int col0, int tid) {
    rsrc = make_rsrc(mat, mat_bytes);
    kb = tid / (BN / 8);
    nb = tid % (BN / 8);
    ld2 = ld * 2;
    const int n = min(col0 + 8 * nb, ld - 8);
    voff = (8 * kb * ld + n) * 2;
  }
  MOE_DEV void load(int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) reg[i] = buf_load16(rsrc, voff + (k0 + i) * ld2, 0);
  }
  MOE_DEV void store(uint16_t* s) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      i32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = static_cast<int>(__builtin_amdgcn_perm(
            static_cast<uint32_t>(reg[2 * q + 1][c >> 1]),
            static_cast<uint32_t>(reg[2 * q][c >> 1]), sel));
      const int n = 8 * nb + c;
      *reinterpret_cast<i32x4*>(s + (n * 8 + (kb ^ swz(n))) * 8) = o;
    }
  }
};

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
template <int EPI, bool NN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_split[kMaxExperts];
  __shared__ int s_pad[kMaxExperts];
  __shared__ int s_tmp[kThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int E = g.E;
  const int tiles_n = (g.N + BN - 1) / BN;

  // ---- tile prefix over the experts (device-resident group sizes) ----
  const int per = (E + kThreads - 1) / kThreads;
  int mine = 0;
  for (int i = 0; i < per; ++i) {
    int e = tid * per + i;
    if (e < E) {
      int n = max(g.split[e], 0);
      s_split[e] = n;
      s_pad[e] = g.padded[e];
      mine += ((n + BM - 1) / BM) * tiles_n;
    }
  }
  int total;
  int run = block_exclusive_scan(mine, s_tmp, total);
  for (int i = 0; i < per; ++i) {
    int e = tid * per + i;
    if (e < E) {
      s_start[e] = run;
      run += ((s_split[e] + BM - 1) / BM) * tiles_n;
    }
  }
  if (tid == 0) s_start[E] = total;
  __syncthreads();

  // ---- XCD-aware id: give each XCD a contiguous run of tile ids ----
  const int G = gridDim.x;
  int vid = blockIdx.x;
  if (G % kNumXcd == 0) vid = (blockIdx.x % kNumXcd) * (G / kNumXcd) + blockIdx.x / kNumXcd;

  for (int tile = vid; tile < total; tile += G) {
    // expert owning this tile: last e with s_start[e] <= tile
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (s_start[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int local = tile - s_start[e];
    const int tm_e = (s_split[e] + BM - 1) / BM;
    const int band = local / (g.group_m * tiles_n);
    const int first_m = band * g.group_m;
    const int gm = min(g.group_m, tm_e - first_m);
    const int rem = local - band * g.group_m * tiles_n;
    const int m_t = first_m + rem % gm;
    const int n_t = rem / gm;

    const int64_t row0 = static_cast<int64_t>(s_pad[e]) + static_cast<int64_t>(m_t) * BM;
    const int rows_valid = static_cast<int>(
        min(static_cast<int64_t>(min(BM, s_split[e] - m_t * BM)), g.M_cap - row0));
    const int col0 = n_t * BN;
    const int cols_valid = min(BN, g.N - col0);
    if (rows_valid <= 0) continue;  // only with inconsistent offsets; stays in bounds

    const uint16_t* Bexp = g.B + static_cast<int64_t>(e) * g.b_stride;
    NTLoader<BM> la;
    la.init(g.A + row0 * g.K, g.M_cap - row0, g.K, tid);
    NTLoader<BN> lb_nt;
    NNLoader lb_nn;
    if constexpr (NN) {
      lb_nn.init(Bexp, static_cast<uint32_t>(static_cast<int64_t>(g.K) * g.N * 2), g.N, col0, tid);
    } else {
      lb_nt.init(Bexp + static_cast<int64_t>(col0) * g.K, g.N - col0, g.K, tid);
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = g.K / BK;
    la.load(0);
    if constexpr (NN) lb_nn.load(0); else lb_nt.load(0);
    la.store(sA[0]);
    if constexpr (NN) lb_nn.store(sB[0]); else lb_nt.store(sB[0]);
    __syncthreads();

    // per-lane LDS chunk coordinates of the MFMA operands
    const int arow = wm * kWaveM + (lane & 31);
    const int brow = wn * kWaveN + (lane & 31);
    const int khalf = lane >> 5;

    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        la.load((kt + 1) * BK);
        if constexpr (NN) lb_nn.load((kt + 1) * BK); else lb_nt.load((kt + 1) * BK);
      }
      const uint16_t* a_s = sA[cur];
      const uint16_t* b_s = sB[cur];
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int ch = ks * 2 + khalf;
        bf16x8 af[4], bfr[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const int r = arow + mi * 32;
          af[mi] = *reinterpret_cast<const bf16x8*>(a_s + (r * 8 + (ch ^ swz(r))) * 8);
        }
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int r = brow + ni * 32;
          bfr[ni] = *reinterpret_cast<const bf16x8*>(b_s + (r * 8 + (ch ^ swz(r))) * 8);
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
      }
      if (more) {
        la.store(sA[cur ^ 1]);
        if constexpr (NN) lb_nn.store(sB[cur ^ 1]); else lb_nt.store(sB[cur ^ 1]);
      }
      __syncthreads();
    }

    // ------------------------------------------------------ epilogues ---
    // The MFMA is issued with B as its first operand, so each 32x32 block
    // holds C^T: lane l owns output row (l % 32) of the block and, in
    // register r, column 8 * (r / 4) + 4 * (l / 32) + r % 4.  A lane thus
    // writes runs of 4 consecutive columns (8 bytes of bf16).
    const int m_lane = wm * kWaveM + (lane & 31);
    const int n_lane = wn * kWaveN + 4 * (lane >> 5);

    if constexpr (EPI == EPI_STORE) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int m = m_lane + mi * 32;
        if (m >= rows_valid) continue;
        uint16_t* crow = g.C + (row0 + m) * g.ldc + col0;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int n = n_lane + ni * 32 + 8 * rg;
            if (n < cols_valid) store_bf16x4(crow + n, acc[mi][ni], 4 * rg);
          }
      }
    } else if constexpr (EPI == EPI_GLU) {
      float amax = 0.0f;
      if (g.act.act == MOE_ACT_SRELU) {
        // not gated: each output column is independent, FC1 width = I
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const int m = m_lane + mi * 32;
          if (m >= rows_valid) continue;
          const int64_t row = row0 + m;
          const float p = g.probs[row];
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
              const int n = n_lane + ni * 32 + 8 * rg;
              if (n >= cols_valid) continue;
              if (g.C) store_bf16x4(g.C + row * g.ldc + col0 + n, acc[mi][ni], 4 * rg);
              float av[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float zc = fminf(fmaxf(acc[mi][ni][4 * rg + i], g.act.glo), g.act.ghi);
                const float rl = fmaxf(zc, 0.0f);
                av[i] = p * rl * rl;
              }
              amax = fmaxf(amax, store_bf16x4_amax(g.act_out + row * g.ld_act + col0 + n, av));
            }
        }
      } else if (wn * kWaveN < cols_valid) {
        // This wave's packed columns [col0 + 128 wn, +128) are gate block q
        // (blocks ni = 0, 1) followed by up block q (ni = 2, 3).
        const int q = (col0 + wn * kWaveN) / (2 * MOE_INTERLEAVE);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const int m = m_lane + mi * 32;
          if (m >= rows_valid) continue;
          const int64_t row = row0 + m;
          const float p = g.probs[row];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
              const int c = h * 32 + 8 * rg + 4 * (lane >> 5);  // 0..63 in the block
              if (g.C) {
                uint16_t* zrow = g.C + row * g.ldc + col0 + wn * kWaveN + c;
                store_bf16x4(zrow, acc[mi][h], 4 * rg);
                store_bf16x4(zrow + MOE_INTERLEAVE, acc[mi][h + 2], 4 * rg);
              }
              float av[4];
#pragma unroll
              for (int i = 0; i < 4; ++i)
                av[i] = p * glu_eval(acc[mi][h][4 * rg + i], acc[mi][h + 2][4 * rg + i], g.act).s;
              amax = fmaxf(amax, store_bf16x4_amax(
                                     g.act_out + row * g.ld_act + q * MOE_INTERLEAVE + c, av));
            }
        }
      }
      if (g.amax) {
        amax = wave_max(amax);
        if (lane == 0) atomic_max_nonneg(g.amax, amax);
      }
    } else {  // EPI_DGLU: acc = dA over logical columns [col0, col0 + BN)
      const bool gated = g.act.act != MOE_ACT_SRELU;
      float* red = reinterpret_cast<float*>(&sA[0][0]);  // [2][BM], free after the loop
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int m = m_lane + mi * 32;
        const bool row_ok = m < rows_valid;
        const int64_t row = row0 + (row_ok ? m : 0);
        const float p = row_ok ? g.probs[row] : 0.0f;
        float dp = 0.0f;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int n = n_lane + ni * 32 + 8 * rg;
            if (!row_ok || n >= cols_valid) continue;
            const int j = col0 + n;  // logical column of dA (4 consecutive)
            if (gated) {
              const int pg = (j / MOE_INTERLEAVE) * 2 * MOE_INTERLEAVE + (j % MOE_INTERLEAVE);
              float gz[4], uz[4], dg[4], du[4];
              load_bf16x4(g.zin + row * g.ldz + pg, gz);
              load_bf16x4(g.zin + row * g.ldz + pg + MOE_INTERLEAVE, uz);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float da = acc[mi][ni][4 * rg + i];
                const GluVal v = glu_eval(gz[i], uz[i], g.act);
                const float ds = p * da;
                dg[i] = v.g_in ? ds * v.u * v.df : 0.0f;
                du[i] = v.u_in ? ds * v.f : 0.0f;
                dp += da * v.s;
              }
              store_f32x4_bf16(g.C + row * g.ldc + pg, dg);
              store_f32x4_bf16(g.C + row * g.ldc + pg + MOE_INTERLEAVE, du);
            } else {
              float zv[4], dz[4];
              load_bf16x4(g.zin + row * g.ldz + j, zv);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float da = acc[mi][ni][4 * rg + i];
                const bool in = (zv[i] >= g.act.glo) && (zv[i] <= g.act.ghi);
                const float rl = fmaxf(fminf(fmaxf(zv[i], g.act.glo), g.act.ghi), 0.0f);
                dz[i] = in ? p * da * 2.0f * rl : 0.0f;
                dp += da * rl * rl;
              }
              store_f32x4_bf16(g.C + row * g.ldc + j, dz);
            }
          }
        // lanes l and l ^ 32 hold the same row: fixed-order pair sum
        dp += __shfl_xor(dp, 32, kWave);
        if (lane < 32) red[wn * BM + m] = dp;
      }
      __syncthreads();
      {
        const int m = tid;  // BM == kThreads
        if (m < rows_valid) g.dp_part[(row0 + m) * g.n_part + n_t] = red[m] + red[BM + m];
      }
      __syncthreads();
    }
  }
}

// dprobs_p[r] = sum_n part[r][n] for valid rows (fixed order), 0 for pad rows.
__global__ __launch_bounds__(256) void dprobs_reduce_kernel(
    const float* __restrict__ part, int n_part, const int32_t* __restrict__ split,
    const int32_t* __restrict__ padded, int E, int64_t M_cap, float* __restrict__ out) {
  __shared__ int s_pad[kMaxExperts + 1];
  __shared__ int s_split[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    s_pad[e] = padded[e];
    s_split[e] = split[e];
  }
  if (threadIdx.x == 0) s_pad[E] = padded[E];
  __syncthreads();
  const int64_t total = min(static_cast<int64_t>(s_pad[E]), M_cap);
  for (int64_t r = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; r < total;
       r += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (s_pad[mid] <= r) lo = mid; else hi = mid - 1;
    }
    float s = 0.0f;
    if (r < s_pad[lo] + s_split[lo]) {
      const float* p = part + r * n_part;
      for (int n = 0; n < n_part; ++n) s += p[n];
    }
    out[r] = s;
  }
}

}  // namespace

int grouped_gemm_tile_n() { return BN; }
int grouped_gemm_tile_m() { return BM; }

hipError_t launch_grouped_gemm(const GemmArgs& g, int epi, bool b_nn, int grid, hipStream_t s) {
  dim3 blk(kThreads), grd(grid);
  if (b_nn) {
    if (epi == EPI_STORE) grouped_gemm_kernel<EPI_STORE, true><<<grd, blk, 0, s>>>(g);
    else if (epi == EPI_DGLU) grouped_gemm_kernel<EPI_DGLU, true><<<grd, blk, 0, s>>>(g);
    else return hipErrorInvalidValue;
  } else {
    if (epi == EPI_STORE) grouped_gemm_kernel<EPI_STORE, false><<<grd, blk, 0, s>>>(g);
    else if (epi == EPI_GLU) grouped_gemm_kernel<EPI_GLU, false><<<grd, blk, 0, s>>>(g);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dprobs_reduce(const float* part, int n_part, const int32_t* split,
                                const int32_t* padded, int E, int64_t M_cap, float* dprobs_p,
                                hipStream_t s) {
  int64_t blocks = (M_cap + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  dprobs_reduce_kernel<<<static_cast<int>(blocks), 256, 0, s>>>(part, n_part, split, padded, E,
                                                              M_cap, dprobs_p);
  return hipGetLastError();
}

}  // namespace moe
