// C ABI of the fused grouped-MLP expert block: argument validation, launch
// configuration and launch order.  Nothing here allocates device memory,
// copies to the host or synchronises; every call only enqueues kernels on
// the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/moe_gmlp.h"
#include "kernels.h"

namespace {

using moe::kMaxExperts;
using moe::kMaxTopK;

constexpr int kMaxDevices = 64;

struct DeviceInfo {
  std::atomic<int> state{0};  // 0 unknown, 1 ok, -1 unusable
  int cu_count = 0;
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

// Attributes of the current device, looked up once per device.
moe_status device_info(int* cu_count) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
  DeviceInfo& d = g_dev[dev];
  int st = d.state.load(std::memory_order_acquire);
  if (st == 0) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    st = d.state.load(std::memory_order_relaxed);
    if (st == 0) {
      hipDeviceProp_t prop;
      st = -1;
      if (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
          std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) {
        d.cu_count = prop.multiProcessorCount;
        st = 1;
      }
      d.state.store(st, std::memory_order_release);
    }
  }
  if (st != 1) return MOE_ERR_DEVICE;
  *cu_count = d.cu_count;
  return MOE_OK;
}

moe_status launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

// Tile-order parameters of the grouped GEMM (performance only; results
// differ at most in fp32 summation order): m-tiles per band, and the K-order
// rotation stride.  Read once from MOE_GEMM_GROUP_M / MOE_GEMM_KROT.
struct GemmTuning {
  // bands of 4 row tiles: as fast as 8-16 or faster on every layer measured
  // (bf16, MXFP8, MXFP4), with a third fewer L2 misses in FC1 (Mixtral)
  int group_m = 4;
  int k_rot = 1;
  int split_max = 4;    // K parts of a split tail tile (1: no split-K); 3-4 measured best
  int split_min_k = 2;  // K steps each part keeps at least
  bool dynamic = true;  // work counters when the workspace holds them (MOE_GEMM_DYNAMIC=0: off)
  bool half_tiles = true;  // half-height last tiles of an expert (MOE_GEMM_HALF=0: off)
};
const GemmTuning& tuning() {
  static const GemmTuning t = [] {
    GemmTuning v;
    if (const char* e = std::getenv("MOE_GEMM_GROUP_M")) v.group_m = std::max(1, std::atoi(e));
    if (const char* e = std::getenv("MOE_GEMM_KROT")) v.k_rot = std::max(0, std::atoi(e));
    if (const char* e = std::getenv("MOE_GEMM_SPLIT_MAX"))
      v.split_max = std::min(std::max(1, std::atoi(e)), moe::grouped_gemm_split_limit());
    if (const char* e = std::getenv("MOE_GEMM_SPLIT_MIN_K"))
      v.split_min_k = std::max(1, std::atoi(e));
    if (const char* e = std::getenv("MOE_GEMM_DYNAMIC")) v.dynamic = std::atoi(e) != 0;
    if (const char* e = std::getenv("MOE_GEMM_HALF")) v.half_tiles = std::atoi(e) != 0;
    return v;
  }();
  return t;
}

bool act_ok(const moe_act_params& a) {
  if (a.act != MOE_ACT_SWIGLU && a.act != MOE_ACT_GEGLU && a.act != MOE_ACT_SRELU) return false;
  if (std::isnan(a.beta) || std::isnan(a.gate_lo) || std::isnan(a.gate_hi) ||
      std::isnan(a.lin_lo) || std::isnan(a.lin_hi) || !std::isfinite(a.lin_offset))
    return false;
  return a.gate_lo <= a.gate_hi && a.lin_lo <= a.lin_hi;
}

void record(void* ev, hipStream_t s) {
  if (ev) (void)hipEventRecord(static_cast<hipEvent_t>(ev), s);
}

// Persistent grid: all CUs but the margin, a multiple of the XCD count so
// the tile-id remap applies, no more than the tiles that can exist.
int gemm_grid(int cu_count, int cu_margin, int64_t M_cap, int E, int N) {
  int g = cu_count - cu_margin;
  if (g >= 8) g -= g % 8;
  const int bm = moe::grouped_gemm_tile_m(), bn = moe::grouped_gemm_tile_n();
  const int64_t ub = ((M_cap + bm - 1) / bm + E) * ((N + bn - 1) / bn);
  if (ub < g) g = static_cast<int>(ub);
  return g < 1 ? 1 : g;
}

int64_t dgrad_parts(int I) {
  const int bn = moe::grouped_gemm_tile_n();
  return (I + bn - 1) / bn;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_DEVICE: return "no usable gfx950 device";
  }
  return "unknown status";
}

int moe_gmlp_version(void) { return 100; }

moe_status moe_weight_repack_interleave(const void* w1, void* w1i, int E, int I, int H,
                                        int block, int inverse, void* stream) {
  if (!w1 || !w1i || w1 == w1i || E < 1 || I < 1 || H < 8 || H % 8 != 0 ||
      block != MOE_INTERLEAVE || I % block != 0)
    return MOE_ERR_INVALID_ARG;
  int cu = 0;
  if (moe_status st = device_info(&cu)) return st;
  return launched(moe::launch_repack_interleave(w1, w1i, E, I, H, block, inverse,
                                                static_cast<hipStream_t>(stream)));
}

size_t moe_permute_workspace_size(int T, int E) {
  if (T < 0 || E < 1) return 0;
  const int64_t chunks = (static_cast<int64_t>(T) + moe::kRouteChunk - 1) / moe::kRouteChunk;
  return static_cast<size_t>(chunks * E * sizeof(int32_t));
}

moe_status moe_permute(const moe_permute_args* a, void* stream) {
  if (!a) return MOE_ERR_INVALID_ARG;
  const int known = MOE_PERMUTE_BUILD_MAP | MOE_PERMUTE_GATHER | MOE_PERMUTE_WRITE_MX |
                    MOE_PERMUTE_WRITE_MX4;
  if (a->flags == 0 || (a->flags & ~known)) return MOE_ERR_INVALID_ARG;
  if ((a->flags & MOE_PERMUTE_WRITE_MX) && (a->flags & MOE_PERMUTE_WRITE_MX4))
    return MOE_ERR_INVALID_ARG;
  if (a->T < 0 || a->k < 1 || a->k > kMaxTopK || a->E < 1 || a->E > kMaxExperts ||
      a->M_cap < 0 || a->M_cap > INT32_MAX)
    return MOE_ERR_INVALID_ARG;
  if (!a->split_sizes || !a->padded_offsets || !a->row_id_map) return MOE_ERR_INVALID_ARG;
  const bool build = a->flags & MOE_PERMUTE_BUILD_MAP;
  const bool gather = a->flags & MOE_PERMUTE_GATHER;
  const bool write_mx = a->flags & (MOE_PERMUTE_WRITE_MX | MOE_PERMUTE_WRITE_MX4);
  if (write_mx && (!gather || !a->xp_q || !a->xp_s || a->H % 64 != 0 || a->M_cap % 128 != 0))
    return MOE_ERR_INVALID_ARG;
  if (build) {
    if (!a->expert_idx || !a->probs || !a->row_src || !a->probs_p) return MOE_ERR_INVALID_ARG;
    if (!a->workspace || a->workspace_bytes < moe_permute_workspace_size(a->T, a->E))
      return MOE_ERR_WORKSPACE;
  }
  if (gather && (!a->x || (!a->xp && !write_mx) || a->H < 8 || a->H % 8 != 0))
    return MOE_ERR_INVALID_ARG;
  int cu = 0;
  if (moe_status st = device_info(&cu)) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (build) {
    if (moe_status st = launched(moe::launch_route(*a, s))) return st;
  }
  if (gather) {
    if (moe_status st = launched(moe::launch_gather(*a, s))) return st;
  }
  return MOE_OK;
}

moe_status moe_unpermute(const moe_unpermute_args* a, void* stream) {
  if (!a || a->T < 0 || a->k < 1 || a->k > kMaxTopK || a->H < 8 || a->H % 8 != 0 ||
      a->M_cap < 0 || !a->row_id_map || !a->yp || !a->out)
    return MOE_ERR_INVALID_ARG;
  if ((a->dprobs != nullptr) != (a->dprobs_p != nullptr)) return MOE_ERR_INVALID_ARG;
  int cu = 0;
  if (moe_status st = device_info(&cu)) return st;
  if (a->T == 0) return MOE_OK;
  return launched(moe::launch_unpermute(*a, static_cast<hipStream_t>(stream)));
}

int64_t moe_mx_scale_offset(int64_t r, int64_t b, int64_t K) {
  return ((r / 32) * (K / 64) + b / 2) * 64 + (b % 2) * 32 + r % 32;
}

moe_status moe_quantize_mxfp8(const moe_quant_args* a, void* stream) {
  if (!a || a->mode < MOE_QUANT_ROW || a->mode > MOE_QUANT_BOTH || a->batch < 0 ||
      a->rows < 64 || a->cols < 64 || a->rows % 64 != 0 || a->cols % 64 != 0 || !a->x || !a->q ||
      !a->s || (a->mode == MOE_QUANT_BOTH && (!a->qT || !a->sT)))
    return MOE_ERR_INVALID_ARG;
  const int64_t n = static_cast<int64_t>(a->rows) * a->cols;
  if (a->x_stride != 0 && (a->x_stride < n || a->x_stride % 8 != 0)) return MOE_ERR_INVALID_ARG;
  int cu = 0;
  if (moe_status st = device_info(&cu)) return st;
  if (a->batch == 0) return MOE_OK;
  moe_quant_args b = *a;
  if (b.x_stride == 0) b.x_stride = n;
  return launched(moe::launch_quantize_mxfp8(b, static_cast<hipStream_t>(stream)));
}

moe_status moe_quantize_mxfp4(const moe_quant_args* a, void* stream) {
  if (!a || a->mode < MOE_QUANT_ROW || a->mode > MOE_QUANT_BOTH || a->batch < 0 ||
      a->rows < 32 || a->cols < 64 || a->rows % 32 != 0 || a->cols % 64 != 0 || !a->x || !a->q ||
      !a->s || a->amax || (a->mode == MOE_QUANT_BOTH && (!a->qT || !a->sT)))
    return MOE_ERR_INVALID_ARG;
  if (a->mode != MOE_QUANT_ROW && a->rows % 64 != 0) return MOE_ERR_INVALID_ARG;
  const int64_t n = static_cast<int64_t>(a->rows) * a->cols;
  if (a->x_stride != 0 && (a->x_stride < n || a->x_stride % 8 != 0)) return MOE_ERR_INVALID_ARG;
  int cu = 0;
  if (moe_status st = device_info(&cu)) return st;
  if (a->batch == 0) return MOE_OK;
  moe_quant_args b = *a;
  if (b.x_stride == 0) b.x_stride = n;
  return launched(moe::launch_quantize_mxfp4(b, static_cast<hipStream_t>(stream)));
}

// Workspace layout: [dprobs partials, fp32 M_cap x ceil(I / 256)] then, at a
// 256-byte boundary, the split-K area of the plain-store GEMMs (partial tiles
// and arrival counters for a grid of one workgroup per CU).
static size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }
static int ws_grid() {
  int cu = 0;
  return device_info(&cu) == MOE_OK ? cu : 256;
}

static size_t dprobs_bytes(int I, int64_t M_cap) {
  return align256(static_cast<size_t>(M_cap * dgrad_parts(I) * sizeof(float)));
}

size_t moe_grouped_mlp_workspace_size(int E, int H, int I, int64_t M_cap, int prec, int act) {
  (void)E;
  (void)H;
  (void)prec;
  (void)act;
  if (I < 1 || M_cap < 0) return 0;
  return dprobs_bytes(I, M_cap) + align256(moe::grouped_gemm_split_bytes(ws_grid())) +
         2 * moe::kTileCtrBytes;
}

size_t moe_grouped_gemm_workspace_size(int dynamic) {
  return align256(moe::grouped_gemm_split_bytes(ws_grid())) + (dynamic ? moe::kTileCtrBytes : 0);
}

// The dynamic-scheduling counters of `launches` GEMM launches: the last
// launches x kTileCtrBytes of the workspace layout, after the split-K area
// sized for a full grid, at `offset` + that area.  Zeroed here (a fill
// kernel, so graph capture records no memset).  Null (static scheduling)
// when the workspace is smaller or the knob is off.
static int* tile_counters(void* ws, size_t ws_bytes, size_t offset, int launches,
                          hipStream_t s, moe_status* st) {
  *st = MOE_OK;
  if (!ws || !tuning().dynamic) return nullptr;
  const size_t at = offset + align256(moe::grouped_gemm_split_bytes(ws_grid()));
  const size_t need = static_cast<size_t>(launches) * moe::kTileCtrBytes;
  if (ws_bytes < at + need) return nullptr;
  int* c = reinterpret_cast<int*>(static_cast<char*>(ws) + at);
  *st = launched(moe::launch_fill_f32(reinterpret_cast<float*>(c), 0.0f,
                                      static_cast<int64_t>(need / sizeof(float)), s));
  return c;
}

// Point a plain-store GEMM at the split-K area of the workspace (if it is
// large enough for `grid`) and zero its counters; returns the launch status.
static moe_status attach_split(moe::GemmArgs& f, void* ws, size_t ws_bytes, size_t offset,
                               int grid, hipStream_t s) {
  f.split_ws = nullptr;
  f.split_cnt = nullptr;
  f.split_slots = 0;
  const size_t need = moe::grouped_gemm_split_bytes(grid);
  if (!ws || ws_bytes < offset + need) return MOE_OK;
  char* base = static_cast<char*>(ws) + offset;
  f.split_ws = reinterpret_cast<float*>(base);
  f.split_slots = grid;
  f.split_max = tuning().split_max;
  f.split_min_k = tuning().split_min_k;
  f.split_cnt = reinterpret_cast<int*>(base + static_cast<size_t>(grid) * 256 * 256 * sizeof(float));
  // 0.0f has the bit pattern of int 0
  return launched(moe::launch_fill_f32(reinterpret_cast<float*>(f.split_cnt), 0.0f, grid, s));
}

// Host-side checks shared by the forward and the backward (no HIP calls, so
// they answer without a device).
static moe_status check_common(int E, int H, int I, int64_t M_cap, int prec,
                               const moe_act_params& act, int cu_margin,
                               const int32_t* split, const int32_t* padded,
                               const float* probs_p) {
  if (E < 1 || E > kMaxExperts || H < 64 || I < 64 || H % 64 != 0 || I % 64 != 0 ||
      M_cap < 1 || M_cap > INT32_MAX || !act_ok(act) || cu_margin < 0)
    return MOE_ERR_INVALID_ARG;
  if (!split || !padded || !probs_p) return MOE_ERR_INVALID_ARG;
  if (prec != MOE_PREC_BF16 && prec != MOE_PREC_MXFP8 && prec != MOE_PREC_MXFP4)
    return MOE_ERR_INVALID_ARG;
  if (prec != MOE_PREC_BF16 && M_cap % 128 != 0) return MOE_ERR_INVALID_ARG;
  // MXFP4 epilogues address 31 rows or columns of a copy with 32-bit lane
  // offsets
  if (prec == MOE_PREC_MXFP4 && (M_cap > (int64_t(1) << 27) || I > (1 << 26)))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status moe_grouped_mlp_fwd(const moe_fwd_args* a, void* stream) {
  if (!a) return MOE_ERR_INVALID_ARG;
  if (moe_status st = check_common(a->E, a->H, a->I, a->M_cap, a->prec, a->act, a->cu_margin,
                                   a->split_sizes, a->padded_offsets, a->probs_p))
    return st;
  const bool f4 = a->prec == MOE_PREC_MXFP4;
  const bool mx = a->prec == MOE_PREC_MXFP8 || f4;
  const bool gated = a->act.act != MOE_ACT_SRELU;
  const int N1 = gated ? 2 * a->I : a->I;
  if (mx) {
    if (!a->xp_q || !a->xp_s || !a->w1_q || !a->w1_s || !a->w2_q || !a->w2_s || !a->a_q ||
        !a->a_s || !a->yp || ((a->aT_q != nullptr) != (a->aT_s != nullptr)))
      return MOE_ERR_INVALID_ARG;
    // MXFP4: no bias
    if (f4 && a->bias1) return MOE_ERR_INVALID_ARG;
  } else {
    if (!a->xp || !a->w1i || !a->w2 || !a->a || !a->yp) return MOE_ERR_INVALID_ARG;
    if (a->w1_stride != 0 && a->w1_stride < static_cast<int64_t>(N1) * a->H)
      return MOE_ERR_INVALID_ARG;
    if (a->w2_stride != 0 && a->w2_stride < static_cast<int64_t>(a->H) * a->I)
      return MOE_ERR_INVALID_ARG;
  }
  int cu = 0;
  if (moe_status st = device_info(&cu)) return st;
  if (a->cu_margin >= cu) return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (a->amax) {
    if (moe_status st = launched(moe::launch_fill_f32(a->amax, 0.0f, 1, s))) return st;
  }
  moe::GemmArgs g{};
  g.E = a->E;
  g.M_cap = a->M_cap;
  g.split = a->split_sizes;
  g.padded = a->padded_offsets;
  g.group_m = tuning().group_m;
  g.half_tiles = tuning().half_tiles;
  g.k_rot_stride = tuning().k_rot;
  g.probs = a->probs_p;
  g.act = moe::to_actp(a->act);
  g.bias = a->bias1;
  g.err = a->err_flag;
  moe_status cst;
  int* ctr = tile_counters(a->workspace, a->workspace_bytes, dprobs_bytes(a->I, a->M_cap), 2,
                           s, &cst);
  if (cst) return cst;
  g.tile_ctr = ctr;

  // FC1: z = xp . W1i^T with the activation epilogue
  g.N = N1;
  g.K = a->H;
  if (mx) {
    g.A = a->xp_q;
    g.a_s = a->xp_s;
    g.B = a->w1_q;
    g.b_stride = static_cast<int64_t>(N1) * a->H;
    g.b_s = a->w1_s;
    g.b_s_stride = g.b_stride / 32;
    g.mx_q = a->a_q;
    g.mx_s = a->a_s;
    g.mx_qT = a->aT_q;
    g.mx_sT = a->aT_s;
    g.mx_n = a->I;
  } else {
    g.A = a->xp;
    g.B = a->w1i;
    g.b_stride = a->w1_stride ? a->w1_stride : static_cast<int64_t>(N1) * a->H;
  }
  g.C = static_cast<uint16_t*>(a->z);
  g.ldc = N1;
  g.act_out = static_cast<uint16_t*>(a->a);
  g.ld_act = a->I;
  g.amax = a->amax;
  record(a->timing_events[0], s);
  const int grid1 = gemm_grid(cu, a->cu_margin, a->M_cap, a->E, g.N);
  if (moe_status st = launched(f4 ? moe::launch_gemm_glu_f4(g, grid1, s)
                                  : moe::launch_grouped_gemm(g, moe::EPI_GLU, false, mx, grid1,
                                                             s)))
    return st;
  record(a->timing_events[1], s);

  // FC2: yp = a . W2^T
  moe::GemmArgs f = g;
  f.N = a->H;
  f.K = a->I;
  if (mx) {
    f.A = a->a_q;
    f.a_s = a->a_s;
    f.B = a->w2_q;
    f.b_stride = static_cast<int64_t>(a->H) * a->I;
    f.b_s = a->w2_s;
    f.b_s_stride = f.b_stride / 32;
    f.mx_q = f.mx_s = f.mx_qT = f.mx_sT = nullptr;
  } else {
    f.A = a->a;
    f.B = a->w2;
    f.b_stride = a->w2_stride ? a->w2_stride : static_cast<int64_t>(a->H) * a->I;
  }
  f.C = static_cast<uint16_t*>(a->yp);
  f.ldc = a->H;
  f.act_out = nullptr;
  f.amax = nullptr;
  f.bias = nullptr;
  f.tile_ctr = ctr ? ctr + moe::kTileCtrBytes / sizeof(int) : nullptr;
  const int grid2 = gemm_grid(cu, a->cu_margin, a->M_cap, a->E, f.N);
  if (f4) {   // the MXFP4 plain-store GEMM runs its last round unsplit
    if (moe_status st = launched(moe::launch_gemm_store_f4(f, grid2, s))) return st;
  } else {
    if (moe_status st = attach_split(f, a->workspace, a->workspace_bytes, 0, grid2, s)) return st;
    if (moe_status st = launched(moe::launch_grouped_gemm(f, moe::EPI_STORE, false, mx, grid2, s)))
      return st;
  }
  record(a->timing_events[2], s);
  return MOE_OK;
}

// The backward with its workspace given separately: the caller's
// (moe_grouped_mlp_bwd) or the library's fixed scratch array
// (moe_grouped_mlp_bwd_noalloc).
// Host-side checks of the backward's arguments (no HIP call).
static moe_status bwd_check(const moe_bwd_args* a) {
  if (!a) return MOE_ERR_INVALID_ARG;
  if (moe_status st = check_common(a->E, a->H, a->I, a->M_cap, a->prec, a->act, a->cu_margin,
                                   a->split_sizes, a->padded_offsets, a->probs_p))
    return st;
  const bool f4 = a->prec == MOE_PREC_MXFP4;
  const bool mx = a->prec == MOE_PREC_MXFP8 || f4;
  const int N1 = a->act.act != MOE_ACT_SRELU ? 2 * a->I : a->I;
  if (!a->z || !a->dprobs_p || !a->dxp) return MOE_ERR_INVALID_ARG;
  if (mx) {
    if (!a->dyp_q || !a->dyp_s || !a->w2t_q || !a->w2t_s || !a->w1t_q || !a->w1t_s ||
        !a->dz_q || !a->dz_s || ((a->dzT_q != nullptr) != (a->dzT_s != nullptr)))
      return MOE_ERR_INVALID_ARG;
    if (f4 && a->bias1) return MOE_ERR_INVALID_ARG;
  } else {
    if (!a->dyp || !a->w2 || !a->w1i || !a->dz) return MOE_ERR_INVALID_ARG;
    if (a->w1_stride != 0 && a->w1_stride < static_cast<int64_t>(N1) * a->H)
      return MOE_ERR_INVALID_ARG;
    if (a->w2_stride != 0 && a->w2_stride < static_cast<int64_t>(a->H) * a->I)
      return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

static moe_status bwd_impl(const moe_bwd_args* a, void* ws, size_t ws_bytes, void* stream) {
  if (moe_status st = bwd_check(a)) return st;
  const bool f4 = a->prec == MOE_PREC_MXFP4;
  const bool mx = a->prec == MOE_PREC_MXFP8 || f4;
  const bool gated = a->act.act != MOE_ACT_SRELU;
  const int N1 = gated ? 2 * a->I : a->I;
  // the dprobs partials are required; the split-K area is used when present
  const size_t need = static_cast<size_t>(a->M_cap * dgrad_parts(a->I) * sizeof(float));
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  int cu = 0;
  if (moe_status st = device_info(&cu)) return st;
  if (a->cu_margin >= cu) return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);

  moe::GemmArgs g{};
  g.E = a->E;
  g.M_cap = a->M_cap;
  g.split = a->split_sizes;
  g.padded = a->padded_offsets;
  g.group_m = tuning().group_m;
  g.half_tiles = tuning().half_tiles;
  g.k_rot_stride = tuning().k_rot;
  g.probs = a->probs_p;
  g.act = moe::to_actp(a->act);
  g.bias = a->bias1;
  g.err = a->err_flag;
  moe_status cst;
  int* ctr = tile_counters(ws, ws_bytes, dprobs_bytes(a->I, a->M_cap), 2, s, &cst);
  if (cst) return cst;
  g.tile_ctr = ctr;

  // FC2 dgrad: dA = dyp . W2 (contracting over H) + dActivation.  bf16 reads
  // W2 [H][I] as [K=H][N=I]; MXFP8 reads its copy quantized along H, [I][H].
  const int n_part = static_cast<int>(dgrad_parts(a->I));
  g.N = a->I;
  g.K = a->H;
  if (mx) {
    g.A = a->dyp_q;
    g.a_s = a->dyp_s;
    g.B = a->w2t_q;
    g.b_stride = static_cast<int64_t>(a->I) * a->H;
    g.b_s = a->w2t_s;
    g.b_s_stride = g.b_stride / 32;
    g.mx_q = a->dz_q;
    g.mx_s = a->dz_s;
    g.mx_qT = a->dzT_q;
    g.mx_sT = a->dzT_s;
    g.mx_n = N1;
  } else {
    g.A = a->dyp;
    g.B = a->w2;
    g.b_stride = a->w2_stride ? a->w2_stride : static_cast<int64_t>(a->H) * a->I;
  }
  g.C = static_cast<uint16_t*>(a->dz);
  g.ldc = N1;
  g.zin = static_cast<const uint16_t*>(a->z);
  g.ldz = N1;
  g.dp_part = static_cast<float*>(ws);
  g.n_part = n_part;
  record(a->timing_events[0], s);
  const int grid1 = gemm_grid(cu, a->cu_margin, a->M_cap, a->E, g.N);
  if (moe_status st = launched(f4 ? moe::launch_gemm_dglu_f4(g, grid1, s)
                                  : moe::launch_grouped_gemm(g, moe::EPI_DGLU, !mx, mx, grid1, s)))
    return st;
  if (moe_status st = launched(moe::launch_dprobs_reduce(g.dp_part, n_part, a->split_sizes,
                                                         a->padded_offsets, a->E, a->M_cap,
                                                         a->dprobs_p, s)))
    return st;
  record(a->timing_events[1], s);

  // FC1 dgrad: dxp = dz . W1i (contracting over N1).  bf16 reads W1i [N1][H]
  // as [K=N1][N=H]; MXFP8 reads its copy quantized along N1, [H][N1].
  moe::GemmArgs f{};
  f.E = a->E;
  f.M_cap = a->M_cap;
  f.split = a->split_sizes;
  f.padded = a->padded_offsets;
  f.group_m = tuning().group_m;
  f.half_tiles = tuning().half_tiles;
  f.k_rot_stride = tuning().k_rot;
  f.act = g.act;
  f.err = a->err_flag;
  f.tile_ctr = ctr ? ctr + moe::kTileCtrBytes / sizeof(int) : nullptr;
  f.N = a->H;
  f.K = N1;
  if (mx) {
    f.A = a->dz_q;
    f.a_s = a->dz_s;
    f.B = a->w1t_q;
    f.b_stride = static_cast<int64_t>(a->H) * N1;
    f.b_s = a->w1t_s;
    f.b_s_stride = f.b_stride / 32;
  } else {
    f.A = a->dz;
    f.B = a->w1i;
    f.b_stride = a->w1_stride ? a->w1_stride : static_cast<int64_t>(N1) * a->H;
  }
  f.C = static_cast<uint16_t*>(a->dxp);
  f.ldc = a->H;
  const int grid2 = gemm_grid(cu, a->cu_margin, a->M_cap, a->E, f.N);
  const size_t dp_bytes =
      align256(static_cast<size_t>(a->M_cap * dgrad_parts(a->I) * sizeof(float)));
  if (f4) {   // the MXFP4 plain-store GEMM runs its last round unsplit
    if (moe_status st = launched(moe::launch_gemm_store_f4(f, grid2, s))) return st;
  } else {
    if (moe_status st = attach_split(f, ws, ws_bytes, dp_bytes, grid2, s)) return st;
    if (moe_status st = launched(moe::launch_grouped_gemm(f, moe::EPI_STORE, !mx, mx, grid2, s)))
      return st;
  }
  record(a->timing_events[2], s);
  return MOE_OK;
}

moe_status moe_grouped_mlp_bwd(const moe_bwd_args* a, void* stream) {
  if (!a) return MOE_ERR_INVALID_ARG;
  return bwd_impl(a, a->workspace, a->workspace_bytes, stream);
}

moe_status moe_grouped_gemm(const moe_gemm_args* a, void* stream) {
  if (!a) return MOE_ERR_INVALID_ARG;
  if (a->E < 1 || a->E > kMaxExperts || a->N < 64 || a->K < 64 || a->N % 64 != 0 ||
      a->K % 64 != 0 || a->M_cap < 1 || a->M_cap > INT32_MAX || a->cu_margin < 0 ||
      (a->b_kn != 0 && a->b_kn != 1) || !a->split_sizes || !a->padded_offsets || !a->a ||
      !a->b || !a->c)
    return MOE_ERR_INVALID_ARG;
  if (a->b_stride != 0 && a->b_stride < static_cast<int64_t>(a->N) * a->K)
    return MOE_ERR_INVALID_ARG;
  if (a->prec != MOE_PREC_BF16 && a->prec != MOE_PREC_MXFP8 && a->prec != MOE_PREC_MXFP4)
    return MOE_ERR_INVALID_ARG;
  const bool f4 = a->prec == MOE_PREC_MXFP4;
  const bool mx = a->prec == MOE_PREC_MXFP8 || f4;
  if (mx && (a->b_kn != 0 || !a->a_s || !a->b_s || a->M_cap % 128 != 0 ||
             (a->b_s_stride != 0 && a->b_s_stride < static_cast<int64_t>(a->N) * a->K / 32)))
    return MOE_ERR_INVALID_ARG;
  if (f4 && a->b_stride % 2 != 0) return MOE_ERR_INVALID_ARG;
  int cu = 0;
  if (moe_status st = device_info(&cu)) return st;
  if (a->cu_margin >= cu) return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  moe::GemmArgs g{};
  if (mx) {
    g.a_s = a->a_s;
    g.b_s = a->b_s;
    g.b_s_stride = a->b_s_stride ? a->b_s_stride : static_cast<int64_t>(a->N) * a->K / 32;
  }
  g.E = a->E;
  g.N = a->N;
  g.K = a->K;
  g.M_cap = a->M_cap;
  g.split = a->split_sizes;
  g.padded = a->padded_offsets;
  g.A = a->a;
  g.B = a->b;
  g.b_stride = a->b_stride ? a->b_stride : static_cast<int64_t>(a->N) * a->K;
  g.group_m = tuning().group_m;
  g.half_tiles = tuning().half_tiles;
  g.k_rot_stride = tuning().k_rot;
  g.C = static_cast<uint16_t*>(a->c);
  g.ldc = a->N;
  g.err = a->err_flag;
  moe_status cst;
  g.tile_ctr = tile_counters(a->workspace, a->workspace_bytes, 0, 1, s, &cst);
  if (cst) return cst;
  const int grid = gemm_grid(cu, a->cu_margin, a->M_cap, a->E, a->N);
  if (f4) return launched(moe::launch_gemm_store_f4(g, grid, s));
  if (moe_status st = attach_split(g, a->workspace, a->workspace_bytes, 0, grid, s)) return st;
  return launched(moe::launch_grouped_gemm(g, moe::EPI_STORE, a->b_kn != 0, mx, grid, s));
}

moe_status moe_glu_unfused(const moe_glu_args* a, void* stream) {
  if (!a) return MOE_ERR_INVALID_ARG;
  if ((a->direction != 0 && a->direction != 1) || a->E < 1 || a->E > kMaxExperts ||
      a->I < 64 || a->I % 64 != 0 || a->M_cap < 1 || a->M_cap > INT32_MAX || !act_ok(a->act) ||
      !a->split_sizes || !a->padded_offsets || !a->probs_p || !a->z)
    return MOE_ERR_INVALID_ARG;
  if (a->direction == 0 && !a->a) return MOE_ERR_INVALID_ARG;
  if (a->direction == 1 && (!a->da || !a->dz || !a->dprobs_p)) return MOE_ERR_INVALID_ARG;
  int cu = 0;
  if (moe_status st = device_info(&cu)) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a->direction == 0 && a->amax) {
    if (moe_status st = launched(moe::launch_fill_f32(a->amax, 0.0f, 1, s))) return st;
  }
  return launched(moe::launch_glu_unfused(a->direction, a->split_sizes, a->padded_offsets, a->E,
                                          a->I, a->M_cap, moe::to_actp(a->act), a->probs_p,
                                          a->z, a->a, a->amax, a->da, a->dz, a->dprobs_p, s));
}

moe_status moe_router_topk(const moe_router_args* a, void* stream) {
  if (!a) return MOE_ERR_INVALID_ARG;
  if (a->T < 1 || a->E < 1 || a->E > kMaxExperts || a->k < 1 || a->k > kMaxTopK ||
      a->k > a->E || !a->logits || !a->expert_idx || !a->probs)
    return MOE_ERR_INVALID_ARG;
  int cu = 0;
  if (moe_status st = device_info(&cu)) return st;
  return launched(moe::launch_router_topk(a->logits, a->T, a->E, a->k, a->expert_idx, a->probs,
                                          static_cast<hipStream_t>(stream)));
}

size_t moe_router_route_workspace_size(int T, int E_total, int E) {
  if (T < 1 || E_total < 1 || E < 1) return 0;
  return moe::router_route_workspace_bytes(T, E_total, E);
}

moe_status moe_router_route(const moe_router_route_args* a, void* stream) {
  if (!a) return MOE_ERR_INVALID_ARG;
  if (a->T < 1 || a->E_total < 1 || a->E_total > kMaxExperts || a->k < 1 || a->k > kMaxTopK ||
      a->k > a->E_total || a->E < 1 || a->E > kMaxExperts || a->first_expert < 0 ||
      a->M_cap < 1 || a->M_cap > INT32_MAX || !a->logits || !a->expert_idx || !a->probs ||
      !a->split_sizes || !a->padded_offsets || !a->row_id_map || !a->row_src || !a->probs_p)
    return MOE_ERR_INVALID_ARG;
  if (!a->workspace ||
      a->workspace_bytes < moe::router_route_workspace_bytes(a->T, a->E_total, a->E))
    return MOE_ERR_WORKSPACE;
  int cu = 0;
  if (moe_status st = device_info(&cu)) return st;
  // every workgroup must be resident at once (grid-wide barriers): a
  // workgroup takes 256 threads and at most 53 KB of LDS, so a CU holds at
  // least three; allow two per CU, and at most 512 (a column of chunk
  // counts is scanned by one wave, eight chunks a lane)
  const int64_t G = moe::router_route_chunks(a->T, a->E_total);
  if (G > 2 * cu || G > 512) return MOE_ERR_UNSUPPORTED;
  return launched(moe::launch_router_route(*a, static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_mlp_wgrad(const moe_wgrad_args* a, void* stream) {
  if (!a) return MOE_ERR_INVALID_ARG;
  if (a->E < 1 || a->E > kMaxExperts || a->H < 64 || a->I < 64 || a->H % 64 != 0 ||
      a->I % 64 != 0 || (a->gated != 0 && a->gated != 1) || a->M_cap < 1 ||
      a->M_cap > (int64_t{1} << 22) || a->cu_margin < 0)
    return MOE_ERR_INVALID_ARG;
  if (a->prec != MOE_PREC_BF16 && a->M_cap % 128 != 0) return MOE_ERR_INVALID_ARG;
  if (!a->split_sizes || !a->padded_offsets) return MOE_ERR_INVALID_ARG;
  if (a->prec != MOE_PREC_BF16 && a->prec != MOE_PREC_MXFP8 && a->prec != MOE_PREC_MXFP4)
    return MOE_ERR_INVALID_ARG;
  const bool f4 = a->prec == MOE_PREC_MXFP4;
  const bool mx = a->prec == MOE_PREC_MXFP8 || f4;
  const int N1 = a->gated ? 2 * a->I : a->I;
  if (mx) {
    if (a->dw1 && (!a->dzT_q || !a->dzT_s || !a->xpT_q || !a->xpT_s)) return MOE_ERR_INVALID_ARG;
    if (a->dw2 && (!a->dypT_q || !a->dypT_s || !a->aT_q || !a->aT_s)) return MOE_ERR_INVALID_ARG;
  } else {
    if (a->dw1 && (!a->dz || !a->xp)) return MOE_ERR_INVALID_ARG;
    if (a->dw2 && (!a->dyp || !a->a)) return MOE_ERR_INVALID_ARG;
    // the loaders address a whole [M_cap][n] activation with 31-bit offsets
    // (0x7fffffff, the offset of a masked lane, must lie past its end)
    const int64_t widest = std::max(std::max(N1, a->H), a->I);
    if (a->M_cap * widest * 2 > int64_t{INT32_MAX}) return MOE_ERR_INVALID_ARG;
  }
  int cu = 0;
  if (moe_status st = device_info(&cu)) return st;
  if (a->cu_margin >= cu) return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);

  // C_e [P][Q] = sum over e's rows m of A[m][p] B[m][q]: bf16 A [M_cap][P],
  // B [M_cap][Q]; MX their transposed copies
  auto run = [&](const void* A, const uint8_t* As, int P, const void* Bm, const uint8_t* Bs,
                 int Q, void* C) -> moe_status {
    moe::GemmArgs g{};
    g.err = a->err_flag;
    g.E = a->E;
    g.N = Q;
    g.K = static_cast<int>(a->M_cap);
    g.M_cap = a->M_cap;
    g.split = a->split_sizes;
    g.padded = a->padded_offsets;
    g.A = A;
    g.a_s = As;
    g.B = Bm;
    g.b_stride = 0;
    g.b_s = Bs;
    g.b_s_stride = 0;
    g.wg_rows = P;
    g.group_m = tuning().group_m;
    g.half_tiles = tuning().half_tiles;
    g.k_rot_stride = tuning().k_rot;
    g.C = static_cast<uint16_t*>(C);
    g.ldc = Q;
    const int bm = moe::grouped_gemm_tile_m(), bn = moe::grouped_gemm_tile_n();
    const int64_t tiles = static_cast<int64_t>(a->E) * ((P + bm - 1) / bm) * ((Q + bn - 1) / bn);
    int grid = cu - a->cu_margin;
    if (grid >= 8) grid -= grid % 8;
    if (tiles < grid) grid = static_cast<int>(tiles);
    if (f4) return launched(moe::launch_gemm_wgrad_f4(g, grid, s));
    return launched(moe::launch_grouped_gemm(g, moe::EPI_WGRAD, false, mx, grid, s));
  };
  record(a->timing_events[0], s);
  if (a->dw1) {
    if (moe_status st = mx ? run(a->dzT_q, a->dzT_s, N1, a->xpT_q, a->xpT_s, a->H, a->dw1)
                           : run(a->dz, nullptr, N1, a->xp, nullptr, a->H, a->dw1))
      return st;
  }
  record(a->timing_events[1], s);
  if (a->dw2) {
    if (moe_status st = mx ? run(a->dypT_q, a->dypT_s, a->H, a->aT_q, a->aT_s, a->I, a->dw2)
                           : run(a->dyp, nullptr, a->H, a->a, nullptr, a->I, a->dw2))
      return st;
  }
  record(a->timing_events[2], s);
  return MOE_OK;
}

}  // extern "C"

namespace moe {
moe_status grouped_mlp_bwd_impl(const moe_bwd_args* a, void* ws, size_t ws_bytes,
                                void* stream) {
  if (!a) return MOE_ERR_INVALID_ARG;
  return bwd_impl(a, ws, ws_bytes, stream);
}
moe_status grouped_mlp_bwd_check(const moe_bwd_args* a) { return bwd_check(a); }
int64_t grouped_mlp_dprobs_parts(int I) { return dgrad_parts(I); }
}  // namespace moe
