// Internal launcher interface between the C ABI (api.cpp) and the gfx950
// kernels.  All launchers enqueue on `stream` and return hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_gmlp.h"

namespace moe {

constexpr int kMaxExperts = 1024;  // per-call local experts (LDS tables)
constexpr int kMaxTopK = 8;
constexpr int kRouteChunk = 256;   // tokens per routing workgroup

// Activation parameters as the kernels see them.
struct ActP {
  int act;
  float beta, glo, ghi, llo, lhi, loff;
};

inline ActP to_actp(const moe_act_params& a) {
  return ActP{a.act, a.beta, a.gate_lo, a.gate_hi, a.lin_lo, a.lin_hi, a.lin_offset};
}

// ---- routing / data movement --------------------------------------------
hipError_t launch_route(const moe_permute_args& a, hipStream_t s);
hipError_t launch_gather(const moe_permute_args& a, hipStream_t s);
hipError_t launch_unpermute(const moe_unpermute_args& a, hipStream_t s);
hipError_t launch_repack_interleave(const void* src, void* dst, int E, int I,
                                    int H, int block, int inverse, hipStream_t s);
hipError_t launch_fill_f32(float* p, float v, int64_t n, hipStream_t s);
hipError_t launch_quantize_mxfp8(const moe_quant_args& a, hipStream_t s);
hipError_t launch_quantize_mxfp4(const moe_quant_args& a, hipStream_t s);  // ROW only
// direction 0: a = bf16(p * act(z)) (+ amax); 1: dz, dprobs from dA and z
hipError_t launch_glu_unfused(int direction, const int32_t* split, const int32_t* padded, int E,
                              int I, int64_t rows, const ActP& act, const float* probs,
                              const void* z, void* a, float* amax, const void* da, void* dz,
                              float* dprobs, hipStream_t s);
hipError_t launch_router_topk(const float* logits, int T, int E, int k, int32_t* idx,
                              float* probs, hipStream_t s);
// router + routing metadata in one launch (router_route.hip)
hipError_t launch_router_route(const moe_router_route_args& a, hipStream_t s);
int router_route_chunks(int T, int E_total);     // workgroups of the launch
size_t router_route_workspace_bytes(int T, int E_total, int E);

// ---- grouped GEMM --------------------------------------------------------
// EPI_WGRAD: weight gradient C_e [P][Q] = sum over expert e's routed rows m
// of A[m][p] B[m][q], C [E][P][Q] stored as in EPI_STORE.  bf16: A and B are
// the routed activations [M_cap][P], [M_cap][Q] (rows past the group's data
// read as zero); MXFP8: their transposed copies [P][M_cap], [Q][M_cap],
// blocked along M, over the group's padded span (pad rows hold zeros).
enum Epi { EPI_STORE = 0, EPI_GLU = 1, EPI_DGLU = 2, EPI_WGRAD = 3 };

struct GemmArgs {
  int E, N, K;
  int64_t M_cap;
  const int32_t* split;
  const int32_t* padded;
  const void* A;         // [M_cap][K] bf16, or E4M3 codes (MXFP8)
  const void* B;         // per expert: B_NT [N][K], B_NN [K][N] (bf16 only)
  int64_t b_stride;      // elements between experts of B
  const uint8_t* a_s;    // MXFP8: tiled scales of A (R = M_cap)
  const uint8_t* b_s;    // MXFP8: tiled scales of B per expert (R = N)
  int64_t b_s_stride;    // bytes between experts of b_s
  int wg_rows;           // EPI_WGRAD: P, rows of A and of each expert's C
  int group_m;           // m-tiles per band of the tile order
  int k_rot_stride;      // K-order rotation per (m_t + n_t) step (0: none)
  // epilogue
  uint16_t* C;           // STORE: out [M_cap][N]; GLU: z (nullable); DGLU: dz (nullable with MX)
  int64_t ldc;
  uint16_t* act_out;     // GLU: a [M_cap][ld_act] (nullable with MX)
  int64_t ld_act;
  const float* probs;    // GLU, DGLU: probs_p [M_cap]
  float* amax;           // GLU (nullable)
  const uint16_t* zin;   // DGLU: z [M_cap][ldz]
  int64_t ldz;
  float* dp_part;        // DGLU: [M_cap][n_part]
  int n_part;
  ActP act;
  // GLU, DGLU (nullable): FC1 bias [E][N1] fp32 in logical column order
  // (gated: gate half, then up half), added to the activation's input
  const float* bias;
  // split-K of the last, partial round of tiles (plain-store epilogue only):
  // fp32 partial tiles and one arrival counter per split tile (zeroed before
  // the launch); null disables splitting
  float* split_ws;
  int* split_cnt;
  int split_slots;       // partial tiles split_ws holds
  int split_max;         // K parts per split tile (<= grouped_gemm_split_limit())
  int split_min_k;       // K steps each part keeps at least
  // MXFP8 copies of the GLU / DGLU output ([M_cap][mx_n])
  uint8_t* mx_q;
  uint8_t* mx_s;
  uint8_t* mx_qT;        // nullable
  uint8_t* mx_sT;
  int mx_n;
  int32_t* err;          // nullable: MOE_DEVERR_BAD_OFFSETS when the offsets are inconsistent
  // half-height tiles for an expert's last 128 rows or fewer (plain-store
  // and GLU kernels; 0: every tile is 256 rows)
  int half_tiles;
  // dynamic tile scheduling (nullable: static): one work counter per XCD,
  // tile_ctr[16 x] (64 bytes apart), zero before the launch
  int* tile_ctr;
  // measurement (nullable): workgroup i writes clk[2 i] = shader cycles and
  // clk[2 i + 1] = constant-rate ticks between its start and its end
  int64_t* clk;
};

hipError_t launch_grouped_gemm(const GemmArgs& g, int epi, bool b_nn, bool mx,
                               int grid, hipStream_t s);
// the record area of the next grouped-GEMM launch while a clock trace is set
// (moe_gemm_clock_trace), else null
int64_t* gemm_clock_slot(int grid);
// MXFP4 operands (A, B: packed E2M1 codes, K / 2 bytes per row; b_stride
// in values), plain store, no split-K
hipError_t launch_gemm_store_f4(const GemmArgs& g, int grid, hipStream_t s);
// MXFP4 operands with the GLU / dGLU epilogue, whose MX copies are then
// MXFP4: rowwise (mx_q, mx_s: [M_cap][mx_n / 2] codes) and, when mx_qT is
// set, transposed (mx_qT, mx_sT: [mx_n][M_cap / 2]); no bias
hipError_t launch_gemm_glu_f4(const GemmArgs& g, int grid, hipStream_t s);
hipError_t launch_gemm_dglu_f4(const GemmArgs& g, int grid, hipStream_t s);
// MXFP4 weight-gradient GEMM (transposed copies, K along the routed rows)
hipError_t launch_gemm_wgrad_f4(const GemmArgs& g, int grid, hipStream_t s);
int grouped_gemm_tile_n();  // BN of the launched configuration
// bytes of split_ws + split_cnt for a grid of `grid` workgroups
size_t grouped_gemm_split_bytes(int grid);
// bytes of one launch's dynamic-scheduling counters (GemmArgs::tile_ctr)
constexpr size_t kTileCtrBytes = 8 * 64;
int grouped_gemm_split_limit();  // largest split_max the kernel accepts
int grouped_gemm_tile_m();  // BM
hipError_t launch_dprobs_reduce(const float* part, int n_part, const int32_t* split,
                                const int32_t* padded, int E, int64_t M_cap,
                                float* dprobs_p, hipStream_t s);

// ---- entry-point bodies shared between C-ABI variants (api.cpp) ---------
// moe_grouped_mlp_bwd with the workspace given apart from the arguments
moe_status grouped_mlp_bwd_impl(const moe_bwd_args* a, void* ws, size_t ws_bytes,
                                void* stream);
moe_status grouped_mlp_bwd_check(const moe_bwd_args* a);  // host-side checks only
int64_t grouped_mlp_dprobs_parts(int I);  // fp32 dprobs partials per row

}  // namespace moe
