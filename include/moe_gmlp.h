/*
 * moe_gmlp.h -- C ABI of the fused grouped-MLP MoE expert block for AMD
 * Instinct MI355X (gfx950).
 *
 * Pages cited (by title and section):
 *   [FK] "Boosting MoE Training Throughput with Advanced Fusion Kernels",
 *        NVIDIA technical blog (zh-cn translation).
 *   [TE] "NVIDIA Transformer Engine 优化 MoE 生物基础模型训练", the
 *        Transformer Engine + BioNeMo Mixtral tutorial.
 *
 * The block computes, for T tokens routed to k of E local experts:
 *   forward   Xp = permute(X);  Z_e = Xp_e W1_e^T;  A = p * GLU(Z);
 *             Yp_e = A_e W2_e^T;  out = unpermute(Yp)
 *   backward  dYp = permute(dOut);  dA_e = dYp_e W2_e;  dZ, dp = dGLU(...);
 *             dXp_e = dZ_e W1_e;  dX = unpermute(dXp);  dprobs = gather(dp)
 * with one grouped-GEMM launch per GEMM whose per-group row counts are read
 * from device memory ([FK] § "Eliminating host-device synchronization and
 * CPU launch overhead"), so no call below ever synchronises with the host.
 *
 * Conventions shared by every entry point
 *   - Pointers named as device buffers are device addresses owned by the
 *     caller; the library never allocates, frees, copies to the host or
 *     synchronises.  Every call only enqueues kernels on `stream` (a
 *     hipStream_t passed as void*; NULL = the null stream), so every call is
 *     legal inside hipStreamBeginCapture in global mode.
 *   - bf16 means IEEE bfloat16 (1-8-7 bits); tensors are row-major with the
 *     last index contiguous.
 *   - Host-checkable problems (NULL pointers, unsupported sizes, small
 *     workspace) return a negative moe_status before anything is launched.
 *     Problems only visible on the device (padded rows exceeding M_cap,
 *     duplicate experts in a token's top-k list, inconsistent group offsets
 *     handed to a grouped GEMM) OR a bit into the optional device int32
 *     *err_flag (MOE_DEVERR_*); kernels then clamp so that no access leaves
 *     the caller's buffers.
 *   - Calls are re-entrant; a per-device attribute cache is filled once.
 */
#ifndef MOE_GMLP_H
#define MOE_GMLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,   /* NULL pointer, bad size or flag          */
  MOE_ERR_UNSUPPORTED = -2,   /* valid request this build does not serve */
  MOE_ERR_WORKSPACE = -3,     /* workspace NULL or smaller than required */
  MOE_ERR_LAUNCH = -4,        /* a kernel launch failed (hipGetLastError) */
  MOE_ERR_DEVICE = -5         /* no usable gfx950 device                 */
} moe_status;

/* Bits OR-ed into *err_flag by kernels (never read back by the library). */
#define MOE_DEVERR_MCAP_OVERFLOW 0x1  /* padded row count > M_cap          */
#define MOE_DEVERR_DUP_EXPERT 0x2     /* a token lists one expert twice    */
#define MOE_DEVERR_SYNC_TIMEOUT 0x4   /* a grid-wide wait of moe_router_route
                                         ran out (the grid was not resident
                                         at once); no rows were written     */
#define MOE_DEVERR_BAD_OFFSETS 0x8    /* a grouped GEMM found split_sizes /
                                         padded_offsets inconsistent: a
                                         negative size or start, or a group
                                         running past the next group's start
                                         or past M_cap (its rows there are
                                         not computed)                       */

/* Group-start alignment of the padded row layout (rows).  Every group of
 * the permuted layout starts at a multiple of it, so MXFP8 blocks of 32
 * rows never straddle two experts. */
#define MOE_GROUP_ALIGN 128
/* Gate/up interleave block of the repacked FC1 weight (rows). */
#define MOE_INTERLEAVE 64
/* MXFP8 block length ([TE] § "Challenge 2", Fig. 3). */
#define MOE_MX_BLOCK 32

/* MXFP8 tensors ([TE] § "Challenge 2", Fig. 3: E4M3 values sharing one
 * E8M0 scale per 32 consecutive values).  The MXFP8 copy of an [R][K]
 * operand, blocked along its contraction axis K, is two device buffers:
 *   codes   u8 [R][K], E4M3 (bias 7, largest finite 448, no infinities)
 *   scales  u8, R*K/32 bytes, E8M0 (value 2^(code - 127)), in the tiled
 *           order the grouped GEMM reads: the scale of row r, block b
 *           (columns [32b, 32b + 32)) is byte moe_mx_scale_offset(r, b, K)
 *             = ((r / 32) * (K / 64) + b / 2) * 64 + (b % 2) * 32 + r % 32,
 *           so one 64-byte run holds what a 32-row slice needs for a 64-deep
 *           K step.  Needs R % 32 == 0 and K % 64 == 0.
 * Encoding of a block v[0..31] (the bf16 values as stored):
 *   e = clamp(floor(log2 max|v|) - 8, -127, 127), e = -127 for an all-zero
 *   block; scale code e + 127; code_i = E4M3 round-to-nearest-even of
 *   v_i / 2^e, saturated to +-448, sign kept (-0 gives 0x80). */
int64_t moe_mx_scale_offset(int64_t r, int64_t b, int64_t K);

typedef enum moe_act {
  MOE_ACT_SWIGLU = 0, /* Swish_beta(g) * u   ([FK] § GLU epilogue, eq. SwiGLU) */
  MOE_ACT_GEGLU = 1,  /* GELU(g) * u, exact erf form                           */
  MOE_ACT_SRELU = 2   /* max(z, 0)^2, not gated: FC1 width I, no interleave    */
} moe_act;

typedef enum moe_prec {
  MOE_PREC_BF16 = 0,  /* bf16 operands, fp32 accumulation                  */
  MOE_PREC_MXFP8 = 1, /* E4M3 operands with E8M0 scales per 32 along K     */
  MOE_PREC_MXFP4 = 2  /* E2M1 operands with E8M0 scales per 32 along K;
                         moe_grouped_gemm and moe_quantize_mxfp4 only      */
} moe_prec;

/* Activation options: the supported GLU family with clamping and scaling
 * ([FK] § "Overcoming training bottlenecks in MoE blocks", list of supported
 * activations; § "Optimizing GLU activations with fused GEMM epilogues").
 *   gated:  g = clamp(z_gate, gate_lo, gate_hi)
 *           u = clamp(z_up, lin_lo, lin_hi) + lin_offset
 *           s = act(g) * u,   act = Swish_beta or GELU
 *   sReLU:  s = max(clamp(z, gate_lo, gate_hi), 0)^2
 * Gradients pass through a clamp only where lo <= pre-clamp value <= hi.
 * Use -INFINITY / +INFINITY for no clamp.  The output of the activation is
 * multiplied by the row's routing probability (ScaledSwiGLU, [TE] §
 * "Challenge 3"). */
typedef struct moe_act_params {
  int32_t act;        /* moe_act */
  float beta;         /* Swish_beta slope; 1 = SiLU */
  float gate_lo, gate_hi;
  float lin_lo, lin_hi;
  float lin_offset;
} moe_act_params;

/* ------------------------------------------------------------------------
 * moe_weight_repack_interleave
 *   Row permutation of the FC1 weight so that one output tile holds matching
 *   halves of gate and up columns ([FK] § "Optimizing GLU activations with
 *   fused GEMM epilogues", Fig. 2).  Done once, e.g. at checkpoint load.
 *   w1   bf16 [E][2I][H], rows [0,I) gate, [I,2I) up   (inverse: w1i layout)
 *   w1i  bf16 [E][2I][H], packed row 2b*floor(j/b) + j%b holds gate row j and
 *        packed row 2b*floor(j/b) + b + j%b holds up row j (b = block)
 *   block must be MOE_INTERLEAVE; I % block == 0.  inverse != 0 undoes it.
 *   w1 and w1i must not overlap.  Bit-exact copy.
 * ---------------------------------------------------------------------- */
moe_status moe_weight_repack_interleave(const void* w1, void* w1i, int E,
                                        int I, int H, int block, int inverse,
                                        void* stream);

/* ------------------------------------------------------------------------
 * moe_permute -- routing metadata and token gather.
 *   The per-expert token counts (GroupedLinear's split_sizes, [TE] §
 *   "Challenge 1") and the expert-major row layout are built on the device
 *   ([FK] § "Eliminating host-device synchronization").
 *
 *   MOE_PERMUTE_BUILD_MAP: from expert_idx[T][k] (global ids; local expert e
 *     is id first_expert+e, any other id is not local) and probs[T][k]:
 *       split_sizes[E]       rows of each local expert
 *       offsets[E+1]         exclusive scan of split_sizes
 *       padded_offsets[E+1]  exclusive scan of split_sizes rounded up to
 *                            MOE_GROUP_ALIGN (group starts)
 *       row_id_map[T][k]     row of (t, slot), -1 if the slot is not local;
 *                            inside a group rows follow ascending t
 *       row_src[M_cap]       token of each row, -1 for pad rows
 *       probs_p[M_cap]       probs[t][slot] of each row, 0 for pad rows
 *     Needs workspace of moe_permute_workspace_size(T, E) bytes.
 *   MOE_PERMUTE_GATHER: xp[r] = x[row_src[r]] (bf16 [T][H] -> [M_cap][H]) for
 *     r < padded_offsets[E]; pad rows are zero; rows past padded_offsets[E]
 *     are not written.  Reads the map built by this or an earlier call.
 *     Used for X in the forward and for dOut in the backward.
 *   MOE_PERMUTE_WRITE_MX: also (or, with xp == NULL, only) write the MXFP8
 *     copy of the gathered rows blocked along H (codes xp_q u8 [M_cap][H],
 *     tiled scales xp_s of M_cap*H/32 bytes, see MOE_MX_BLOCK); pad rows
 *     get zero codes and scale code 0.  Needs H % 64 == 0, M_cap % 128 == 0.
 *   MOE_PERMUTE_WRITE_MX4: the same with an MXFP4 copy instead ([FK] §
 *     "Fused MXFP8 and NVFP4 quantization": the 4-bit recipe's operands,
 *     read here as E2M1 with E8M0 scales per 32 along H): codes xp_q u8
 *     [M_cap][H / 2] (two a byte, element 2 i in the low nibble of byte i),
 *     scales as for WRITE_MX with the MXFP4 block rule (see
 *     moe_quantize_mxfp4).  Not together with WRITE_MX.
 *   Requires H % 32 == 0 for GATHER, M_cap >= T*k + E*(MOE_GROUP_ALIGN-1)
 *   unless the caller knows the padded total fits (else MOE_DEVERR_MCAP_
 *   OVERFLOW is raised and rows past M_cap are dropped).
 * ---------------------------------------------------------------------- */
#define MOE_PERMUTE_BUILD_MAP 0x1
#define MOE_PERMUTE_GATHER 0x2
#define MOE_PERMUTE_WRITE_MX 0x4
#define MOE_PERMUTE_WRITE_MX4 0x8

typedef struct moe_permute_args {
  int32_t flags;
  int32_t T, k, E, first_expert, H;
  int64_t M_cap;
  const int32_t* expert_idx;   /* [T][k]  device */
  const float* probs;          /* [T][k]  device */
  int32_t* split_sizes;        /* [E]     device */
  int32_t* offsets;            /* [E+1]   device (may be NULL) */
  int32_t* padded_offsets;     /* [E+1]   device */
  int32_t* row_id_map;         /* [T][k]  device */
  int32_t* row_src;            /* [M_cap] device */
  float* probs_p;              /* [M_cap] device */
  const void* x;               /* bf16 [T][H]     device (GATHER) */
  void* xp;                    /* bf16 [M_cap][H] device (GATHER) */
  uint8_t* xp_q;               /* u8 [M_cap][H]          (WRITE_MX) */
  uint8_t* xp_s;               /* u8 M_cap*H/32, tiled   (WRITE_MX) */
  int32_t* err_flag;           /* optional device int32 */
  void* workspace;             /* device, BUILD_MAP only */
  size_t workspace_bytes;
} moe_permute_args;

size_t moe_permute_workspace_size(int T, int E);
moe_status moe_permute(const moe_permute_args* args, void* stream);

/* ------------------------------------------------------------------------
 * moe_unpermute -- combine of the expert outputs (the index-add of [TE] §
 *   "Challenge 1"), in gather form so that no atomics are needed:
 *     out[t] = bf16( sum_{s < k, row_id_map[t][s] >= 0} yp[row_id_map[t][s]] )
 *   summed in fp32 in slot order; a token with no local slot gets zeros.
 *   The same call combines dXp into dX in the backward.  If dprobs_p and
 *   dprobs are both non-NULL it also writes
 *     dprobs[t][s] = row_id_map[t][s] >= 0 ? dprobs_p[row_id_map[t][s]] : 0.
 *   yp bf16 [M_cap][H]; out bf16 [T][H]; H % 8 == 0.
 * ---------------------------------------------------------------------- */
typedef struct moe_unpermute_args {
  int32_t T, k, H;
  int64_t M_cap;
  const int32_t* row_id_map;   /* [T][k]     device */
  const void* yp;              /* bf16 [M_cap][H] device */
  void* out;                   /* bf16 [T][H] device */
  const float* dprobs_p;       /* [M_cap] device, optional */
  float* dprobs;               /* [T][k]  device, optional */
} moe_unpermute_args;

moe_status moe_unpermute(const moe_unpermute_args* args, void* stream);

/* ------------------------------------------------------------------------
 * moe_quantize_mxfp8 -- bf16 -> MXFP8 ([TE] § "Challenge 2", Fig. 3;
 *   § "Challenge 3": bf16 master weights are quantized before the
 *   low-precision GEMM).  Encoding and scale layout as under MOE_MX_BLOCK.
 *   x bf16 [batch][rows][cols], x_stride elements between batch entries
 *   (0: rows*cols; a multiple of 8).
 *   MOE_QUANT_ROW: blocks along cols (K = cols): q [batch][rows][cols],
 *     scales rows*cols/32 bytes per batch entry, tiled with R = rows.
 *   MOE_QUANT_COL: blocks along rows, written transposed so that the
 *     consumer's K = rows is contiguous: q [batch][cols][rows], scales
 *     tiled with R = cols, K = rows.
 *   MOE_QUANT_BOTH: ROW into q / s and COL into qT / sT in one pass that
 *     reads x once ([TE] § "Challenge 3": the master weights are cast for
 *     every step, so the two copies of a weight are made together).
 *   The weight copies the MXFP8 forward and backward read are
 *     ROW of w1i (K = H), ROW of w2 (K = I), COL of w2 (K = H) and COL of
 *     w1i (K = N1): BOTH of w1i and BOTH of w2.
 *   rows and cols must be multiples of 64.  If amax != NULL, *amax is raised
 *   to max|x| (the caller zeroes it first).  Memory-bound: reads 2 bytes and
 *   writes 33/32 bytes per element and copy.  qT and sT are read only in
 *   the BOTH mode.  With live (say the split sizes, batch = E), the batch
 *   entries of experts with no routed rows are skipped: a step's GEMMs read
 *   no weight of such an expert.
 * ---------------------------------------------------------------------- */
#define MOE_QUANT_ROW 0
#define MOE_QUANT_COL 1
#define MOE_QUANT_BOTH 2

typedef struct moe_quant_args {
  int32_t mode;
  int32_t batch, rows, cols;
  int64_t x_stride;            /* elements between batch entries of x */
  const void* x;               /* bf16 device */
  uint8_t* q;                  /* device */
  uint8_t* s;                  /* device */
  float* amax;                 /* optional device float */
  uint8_t* qT;                 /* device, MOE_QUANT_BOTH: the COL codes */
  uint8_t* sT;                 /* device, MOE_QUANT_BOTH: the COL scales */
  const int32_t* live;         /* optional device int32 [batch]: entries with
                                  live[b] == 0 are skipped (their codes and
                                  scales keep what they held) */
} moe_quant_args;

moe_status moe_quantize_mxfp8(const moe_quant_args* args, void* stream);

/* ------------------------------------------------------------------------
 * moe_quantize_mxfp4 -- bf16 -> MXFP4, the 4-bit microscaling format of
 *   gfx950's scaled MFMA, standing where [FK] § "Fused MXFP8 and NVFP4
 *   quantization" names a 4-bit recipe (NVFP4's E4M3 scales per 16 values
 *   have no MFMA form; MXFP4 keeps E8M0 scales per 32).
 *   Elements E2M1 (exponent bias 1, one mantissa bit, values 0, 0.5, 1,
 *   1.5, 2, 3, 4, 6 and their negatives); block scale 2^e with
 *   e = clamp(floor(log2 max|v|) - 2, -127, 127) (-127 for an all-zero
 *   block), code e + 127; element code = E2M1 round-to-nearest-even of
 *   v / 2^e, magnitudes past 6 saturated, sign kept (-0 -> 0x8).
 *   x bf16 [batch][rows][cols]; codes two a byte, element 2 i in the low
 *   nibble of byte i; scales rows*cols/32 bytes per batch entry in the tiled
 *   layout of MOE_MX_BLOCK.
 *   MOE_QUANT_ROW: blocks along cols: q [batch][rows][cols / 2], scales
 *     tiled with R = rows, K = cols.
 *   MOE_QUANT_COL: blocks along rows, written transposed: q
 *     [batch][cols][rows / 2], scales tiled with R = cols, K = rows
 *     (rows % 64 == 0).
 *   MOE_QUANT_BOTH: ROW into q / s and COL into qT / sT, one pass
 *     (rows % 64 == 0).
 *   rows % 32 == 0, cols % 64 == 0; amax must be NULL.  Memory-bound: reads
 *   2 bytes, writes 17/32 bytes per element.
 * ---------------------------------------------------------------------- */
moe_status moe_quantize_mxfp4(const moe_quant_args* args, void* stream);

/* ------------------------------------------------------------------------
 * moe_grouped_mlp_fwd -- FC1 grouped GEMM with the fused activation epilogue,
 *   then the FC2 grouped GEMM: two persistent launches whose tile schedulers
 *   walk split_sizes / padded_offsets on the device.
 *   ([FK] § "Overcoming training bottlenecks", kernel families 1 and 2,
 *   Fig. 1; § "Optimizing GLU activations with fused GEMM epilogues";
 *   [TE] § "Challenge 3": GroupedLinear -> ScaledSwiGLU -> GroupedLinear.)
 *
 *   For every local expert e and row r in [padded_offsets[e],
 *   padded_offsets[e] + split_sizes[e]):
 *     z[r]  = xp[r] . W1i_e^T                 (fp32 accumulate, stored bf16)
 *     a[r]  = bf16( probs_p[r] * act(z[r] + b_e) )  (act on the fp32 accumulator)
 *     yp[r] = bf16( a[r] . W2_e^T )
 *   Rows outside those ranges are not written.
 *   b_e is the optional FC1 bias ([FK] § "Optimizing GLU activations with
 *   fused GEMM epilogues": the epilogue also folds in a bias-vector add):
 *   bias1 fp32 [E][N1] in LOGICAL column order (gated: the gate half, then
 *   the up half; not interleaved), added to the fp32 accumulator before the
 *   activation; z is stored without it.  NULL: no bias.
 *   Shapes: N1 = 2I (gated) or I (sReLU).
 *     xp   bf16 [M_cap][H]
 *     w1i  bf16 [E][N1][H], gated: interleaved by moe_weight_repack_interleave
 *     w2   bf16 [E][H][I]
 *     z    bf16 [M_cap][N1] in the same (interleaved) column order as w1i rows;
 *          may be NULL when no backward follows, or when the backward
 *          rebuilds it (activation recompute, see moe_grouped_gemm)
 *     a    bf16 [M_cap][I] logical column order
 *     yp   bf16 [M_cap][H]
 *     amax optional device float: raised to max|a| over written rows (the
 *          call zeroes it first, so it holds this call's value)
 *   Requires H % 64 == 0, I % 64 == 0, E >= 1.
 *   timing_events: optional hipEvent_t handles; non-NULL entries are recorded
 *   on `stream` before FC1, between FC1 and FC2, and after FC2.
 *
 *   prec == MOE_PREC_MXFP8 ([TE] § "Challenge 2"/"Challenge 3"; [FK] §
 *   "Fused MXFP8 and NVFP4 quantization"): both GEMMs take MXFP8 operands
 *   (E4M3 x E4M3 with E8M0 scales per 32 along K, fp32 accumulation):
 *     FC1: xp_q/xp_s (moe_permute WRITE_MX) x w1_q/w1_s (ROW of w1i)
 *     FC2: a_q/a_s x w2_q/w2_s (ROW of w2)
 *   xp, w1i and w2 are not read.  The FC1 epilogue writes z and a as in
 *   bf16 (a may be NULL), amax, and the MXFP8 copies of a, quantized from the
 *   stored bf16 a: a_q/a_s blocked along I (the FC2 operand) and, if aT_q
 *   and aT_s are both set, the transposed copy aT_q [I][M_cap] blocked along
 *   M inside each group (scales tiled with R = I, K = M_cap).  Pad rows of a
 *   group (up to the next multiple of MOE_GROUP_ALIGN) get zero codes and
 *   scale code 0 in both copies.  Weights are contiguous per expert
 *   (w1_stride / w2_stride are ignored).  Needs M_cap % 128 == 0.
 *
 *   prec == MOE_PREC_MXFP4 ([FK] § "Fused MXFP8 and NVFP4 quantization":
 *   the 4-bit recipe; E2M1 codes with E8M0 scales per 32 along K on MI355X,
 *   the format of moe_quantize_mxfp4): the same fields as MXFP8, every
 *   operand MXFP4 -- codes two a byte (element 2 i in the low nibble of
 *   byte i), [rows][K / 2] -- and scales in the tiled layout with the
 *   MXFP4 block rule: xp_q/xp_s (moe_permute WRITE_MX4), w1_q/w1_s and
 *   w2_q/w2_s (moe_quantize_mxfp4 ROW of w1i and w2).  The FC1 epilogue
 *   writes a_q/a_s, the MXFP4 copy of the stored bf16 a blocked along I
 *   (codes [M_cap][I / 2]) and, when aT_q is set, aT_q/aT_s, its MXFP4
 *   transposed copy blocked along M (codes [I][M_cap / 2], pad rows as
 *   zeros), the operand of the MXFP4 weight gradient.  No bias (bias1
 *   NULL), else MOE_ERR_INVALID_ARG.  MXFP4 serves M_cap up to 2^27 and I
 *   up to 2^26 (forward and backward), else MOE_ERR_UNSUPPORTED.
 * ---------------------------------------------------------------------- */
typedef struct moe_fwd_args {
  int32_t E, H, I;
  int64_t M_cap;
  int32_t prec;                /* moe_prec */
  moe_act_params act;
  int32_t cu_margin;           /* CUs to leave free for concurrent kernels */
  const int32_t* split_sizes;     /* [E]     device */
  const int32_t* padded_offsets;  /* [E+1]   device */
  const float* probs_p;           /* [M_cap] device */
  const void* xp;
  const void* w1i;
  const void* w2;
  int64_t w1_stride;           /* elements between experts of w1i (0: N1*H) */
  int64_t w2_stride;           /* elements between experts of w2  (0: H*I)  */
  void* z;
  void* a;
  float* amax;
  void* yp;
  int32_t* err_flag;
  void* timing_events[3];
  /* MXFP8 operands and outputs (prec == MOE_PREC_MXFP8 only) */
  const uint8_t* xp_q;  const uint8_t* xp_s;   /* [M_cap][H]            */
  const uint8_t* w1_q;  const uint8_t* w1_s;   /* [E][N1][H], along H   */
  const uint8_t* w2_q;  const uint8_t* w2_s;   /* [E][H][I],  along I   */
  uint8_t* a_q;   uint8_t* a_s;                /* [M_cap][I], along I   */
  uint8_t* aT_q;  uint8_t* aT_s;               /* [I][M_cap], along M (optional) */
  /* optional workspace (moe_grouped_mlp_workspace_size bytes): lets FC2
   * split its last, partial round of tiles along K; NULL disables that */
  void* workspace;
  size_t workspace_bytes;
  const float* bias1;          /* optional [E][N1] fp32, logical order (see above) */
} moe_fwd_args;

moe_status moe_grouped_mlp_fwd(const moe_fwd_args* args, void* stream);

/* ------------------------------------------------------------------------
 * moe_grouped_mlp_bwd -- FC2 dgrad grouped GEMM with the fused
 *   dActivation epilogue, then the FC1 dgrad grouped GEMM
 *   ([FK] § "Overcoming training bottlenecks", kernel family 3, Fig. 1;
 *   § "Optimizing GLU activations": the backward epilogue reads the GEMM
 *   output, applies dSwiGLU and writes the result).
 *
 *   For every valid row r of expert e:
 *     dA[r]       = dyp[r] . W2_e                   (fp32, not stored)
 *     s[r]        = act(z[r] + b_e)                 (recomputed from bf16 z)
 *     dprobs_p[r] = sum_j dA[r][j] * s[r][j]        (fixed-order, deterministic)
 *     dz[r]       = bf16( dact(z[r] + b_e, probs_p[r] * dA[r]) )  (layout of z)
 *   with b_e the forward's optional bias1 (NULL: none); dz is also the
 *   gradient of b_e's summands (sum dz over an expert's rows, in logical
 *   order, is dL/db_e).
 *     dxp[r]      = bf16( dz[r] . W1i_e )           (contracts over N1)
 *   Shapes as in moe_grouped_mlp_fwd; dyp bf16 [M_cap][H]; dz bf16
 *   [M_cap][N1]; dprobs_p float [M_cap]; dxp bf16 [M_cap][H].
 *   Needs workspace of moe_grouped_mlp_workspace_size(...) bytes (partial
 *   sums of dprobs_p).  timing_events as in the forward (before FC2 dgrad,
 *   between, after FC1 dgrad).
 *
 *   prec == MOE_PREC_MXFP8: both GEMMs take MXFP8 operands blocked along
 *   their K:
 *     FC2 dgrad: dyp_q/dyp_s (moe_permute WRITE_MX of dOut, along H) x
 *                w2t_q/w2t_s (COL of w2: [E][I][H], along H)
 *     FC1 dgrad: dz_q/dz_s x w1t_q/w1t_s (COL of w1i: [E][H][N1], along N1)
 *   dyp, w2 and w1i are not read; z is read (bf16).  The dActivation
 *   epilogue writes dz (bf16, may be NULL), dprobs_p, and the MXFP8 copies
 *   of the stored bf16 dz: dz_q/dz_s [M_cap][N1] blocked along N1 (in the
 *   interleaved column order; with the 64-row interleave every block holds
 *   only gate or only up columns) and, if dzT_q and dzT_s are both set, the
 *   transposed dzT_q [N1][M_cap] blocked along M inside each group.  Pad
 *   rows as in the forward.  Needs M_cap % 128 == 0.
 *
 *   prec == MOE_PREC_MXFP4: as MXFP8 with MXFP4 operands (see the forward):
 *   dyp_q/dyp_s (moe_permute WRITE_MX4 of dOut), w2t_q/w2t_s and
 *   w1t_q/w1t_s (moe_quantize_mxfp4 COL of w2 and w1i), and the epilogue's
 *   dz_q/dz_s, the MXFP4 copy of the stored bf16 dz blocked along N1, and
 *   optionally dzT_q/dzT_s, its transposed MXFP4 copy [N1][M_cap / 2]
 *   blocked along M.  No bias.
 * ---------------------------------------------------------------------- */
typedef struct moe_bwd_args {
  int32_t E, H, I;
  int64_t M_cap;
  int32_t prec;
  moe_act_params act;
  int32_t cu_margin;
  const int32_t* split_sizes;
  const int32_t* padded_offsets;
  const float* probs_p;
  const void* dyp;
  const void* w2;
  const void* z;
  const void* w1i;
  int64_t w1_stride;
  int64_t w2_stride;
  void* dz;
  float* dprobs_p;
  void* dxp;
  int32_t* err_flag;
  void* workspace;
  size_t workspace_bytes;
  void* timing_events[3];
  /* MXFP8 operands and outputs (prec == MOE_PREC_MXFP8 only) */
  const uint8_t* dyp_q; const uint8_t* dyp_s;  /* [M_cap][H]            */
  const uint8_t* w2t_q; const uint8_t* w2t_s;  /* [E][I][H],  along H   */
  const uint8_t* w1t_q; const uint8_t* w1t_s;  /* [E][H][N1], along N1  */
  uint8_t* dz_q;  uint8_t* dz_s;               /* [M_cap][N1], along N1 */
  uint8_t* dzT_q; uint8_t* dzT_s;              /* [N1][M_cap], along M (optional) */
  const float* bias1;          /* optional [E][N1] fp32, as in the forward */
} moe_bwd_args;

moe_status moe_grouped_mlp_bwd(const moe_bwd_args* args, void* stream);

/* ------------------------------------------------------------------------
 * moe_grouped_mlp_bwd_noalloc -- moe_grouped_mlp_bwd for callers that cannot
 *   allocate device memory (code under stream capture, tight training loops,
 *   harnesses that forbid hipMalloc): the same computation and arguments,
 *   but the workspace fields of *args are ignored.  The workspace comes
 *   instead from a fixed array of MOE_NOALLOC_SCRATCH_BYTES that the library
 *   holds on every device it runs on, until the process ends.
 *   Limit: M_cap * ceil(I / 256) * 4 <= MOE_NOALLOC_SCRATCH_BYTES (the fp32
 *   dprobs partial sums), else MOE_ERR_UNSUPPORTED before any launch; the
 *   FC1 dgrad splits its last round of tiles along K only when that area
 *   also fits in the array.  Nothing in the array needs clearing between
 *   calls (every partial read is written first in the same call).
 *   All calls on one device share that device's array: calls that overlap
 *   in time on one device (two streams, two threads) race and give wrong
 *   results; order them on one stream.  The array's address is looked up on
 *   the first call on each device (with that device current); make that
 *   first call outside stream capture.  No hipMalloc, hipFree or host sync.
 * ---------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)

moe_status moe_grouped_mlp_bwd_noalloc(const moe_bwd_args* args, void* stream);

/* ------------------------------------------------------------------------
 * moe_grouped_mlp_wgrad -- the weight-gradient grouped GEMMs of the backward
 *   ([FK] § "Overcoming training bottlenecks", Fig. 1: the weight gradients
 *   stay in separate blocks outside the fused kernels; § "Fused MXFP8 and
 *   NVFP4 quantization": the transposed copies the epilogues write are the
 *   MXFP8 operands).
 *
 *   For every local expert e, over its rows r in [padded_offsets[e],
 *   padded_offsets[e] + split_sizes[e]):
 *     dw1[e] = bf16( sum_r dz[r]^T xp[r] )   [N1][H], rows in the column
 *                                            order of dz (that of w1i)
 *     dw2[e] = bf16( sum_r dyp[r]^T a[r] )   [H][I]
 *   fp32 accumulation, one rounding; an expert with no rows gets zeros.
 *     prec == MOE_PREC_BF16: dz [M_cap][N1], xp [M_cap][H], dyp [M_cap][H]
 *       and a [M_cap][I] as the forward and backward store them (bf16,
 *       row-major).  Only the rows of the groups' data are read, so pad rows
 *       may hold anything.  Needs M_cap * max(N1, H, I) * 2 < 2^31.
 *     prec == MOE_PREC_MXFP8: their transposed copies [n][M_cap], E4M3
 *       codes blocked along M with scales tiled (R = n, K = M_cap): aT_q from
 *       moe_grouped_mlp_fwd, dzT_q from moe_grouped_mlp_bwd, xpT_q and
 *       dypT_q from moe_quantize_mxfp8 (MOE_QUANT_COL of xp and dyp, rows =
 *       M_cap).  Columns [padded_offsets[e], padded_offsets[e + 1]) belong to
 *       expert e and are read whole, so the pad rows there must encode zero
 *       (as the producers above write them).
 *     prec == MOE_PREC_MXFP4: the same transposed copies in MXFP4, E2M1
 *       codes two a byte ([n][M_cap / 2], element 2 i in the low nibble of
 *       byte i) blocked along M with the MXFP4 block rule: aT_q / dzT_q
 *       from the MXFP4 forward / backward, xpT_q and dypT_q from
 *       moe_quantize_mxfp4 (MOE_QUANT_COL).  Expert e's codes are read from
 *       its first row on, up to its split_sizes[e] rows rounded up to 32.
 *   dw1 or dw2 may be NULL to skip that GEMM; the caller owns every buffer.
 *   Needs M_cap <= 4194304 (MX: M_cap % 128 == 0); H, I multiples of 64.
 *   Invalid arguments return MOE_ERR_INVALID_ARG before any launch.
 *   timing_events: optional hipEvent_t handles recorded before dw1, between,
 *   and after dw2.
 * ---------------------------------------------------------------------- */
typedef struct moe_wgrad_args {
  int32_t E, H, I;
  int32_t gated;                  /* 1: N1 = 2 I (GLU), 0: N1 = I (sReLU) */
  int64_t M_cap;
  int32_t prec;
  int32_t cu_margin;
  const int32_t* split_sizes;     /* [E]   device */
  const int32_t* padded_offsets;  /* [E+1] device */
  const void* dz;  const void* xp;  const void* dyp;  const void* a;   /* bf16 */
  const uint8_t* dzT_q;  const uint8_t* dzT_s;    /* MX [N1][M_cap] (MXFP4: M_cap / 2 bytes a row) */
  const uint8_t* xpT_q;  const uint8_t* xpT_s;    /* MX [H][M_cap]  */
  const uint8_t* dypT_q; const uint8_t* dypT_s;   /* MX [H][M_cap]  */
  const uint8_t* aT_q;   const uint8_t* aT_s;     /* MX [I][M_cap]  */
  void* dw1;                      /* bf16 [E][N1][H] or NULL */
  void* dw2;                      /* bf16 [E][H][I] or NULL  */
  void* timing_events[3];
  int32_t* err_flag;              /* optional device int32 (MOE_DEVERR_BAD_OFFSETS) */
} moe_wgrad_args;

moe_status moe_grouped_mlp_wgrad(const moe_wgrad_args* args, void* stream);

/* ------------------------------------------------------------------------
 * The unfused baseline: a plain grouped GEMM and separate activation passes,
 * the layer as it runs without the fused epilogues ([FK] § "Overcoming
 * training bottlenecks": unfused, activation and quantization are separate
 * memory-bound kernels; Fig. 3 compares fused with unfused kernels).  The
 * fused entry points above are the product; these measure what fusion buys.
 *
 * moe_grouped_gemm -- C[r] = bf16(A[r] . B_e^T) for every routed row r of
 *   expert e (fp32 accumulation): A [M_cap][K], C [M_cap][N] bf16; B_e at
 *   b + e * b_stride, [N][K] (b_kn = 0) or [K][N] (b_kn = 1); pad rows of C
 *   are not written.  Needs N, K multiples of 64.  workspace (optional, the
 *   size moe_grouped_mlp_workspace_size gives) enables the K split of a
 *   partial last round (bf16).
 *   prec == MOE_PREC_MXFP8: A and B are E4M3 codes with tiled E8M0 scales
 *   blocked along K (a_s: R = M_cap; b_s per expert: R = N, b_s_stride bytes
 *   apart, 0 = N * K / 32); b_kn must be 0 and M_cap % 128 == 0.
 *   prec == MOE_PREC_MXFP4: A and B are packed E2M1 codes (K / 2 bytes a
 *   row, moe_quantize_mxfp4's layout) with tiled E8M0 scales as for MXFP8;
 *   b_stride counts values (even); no split-K.  Same limits as MXFP8.
 *   Activation recompute ([FK] § "What's next" names it as planned work):
 *   with workspace NULL, A = xp (or xp_q/xp_s), B = w1i (or w1_q/w1_s),
 *   N = N1, K = H, every tile sums K in the order moe_grouped_mlp_fwd's FC1
 *   uses, so C is bit for bit the z FC1 stores; a forward called with z NULL
 *   can then be followed by moe_grouped_mlp_bwd on this rebuilt z.
 * ---------------------------------------------------------------------- */
typedef struct moe_gemm_args {
  int32_t E, N, K;
  int64_t M_cap;
  int32_t b_kn;
  int32_t cu_margin;
  const int32_t* split_sizes;
  const int32_t* padded_offsets;
  const void* a;
  const void* b;
  int64_t b_stride;               /* elements; 0: N * K */
  void* c;
  void* workspace;
  size_t workspace_bytes;
  int32_t prec;                   /* MOE_PREC_BF16 or MOE_PREC_MXFP8 */
  const uint8_t* a_s;
  const uint8_t* b_s;
  int64_t b_s_stride;             /* bytes; 0: N * K / 32 */
  int32_t* err_flag;              /* optional device int32 (MOE_DEVERR_BAD_OFFSETS) */
} moe_gemm_args;

moe_status moe_grouped_gemm(const moe_gemm_args* args, void* stream);

/* Workspace bytes for moe_grouped_gemm: with dynamic == 0 the K split of
 * the last round only; otherwise also the per-XCD work counters of dynamic
 * tile scheduling ([FK] § "From kernel-level to pre-training speedups":
 * dynamic scheduling, for efficient overlap with other kernels).  With the
 * counters, workgroups take tiles from them after a static first round, so
 * a workgroup that starts late (its CU busy with another kernel) leaves its
 * share to the others; without them every workgroup walks a fixed list.
 * Results do not depend on the scheduling (each tile's sum runs in one
 * fixed order).  The fused forward and backward use the counters when
 * their workspace has moe_grouped_mlp_workspace_size bytes. */
size_t moe_grouped_gemm_workspace_size(int dynamic);

/* moe_glu_unfused -- the activation of the FC1 output as its own pass.
 *   direction 0: a[r] = bf16(probs_p[r] * act(z[r])) and amax = max |a|
 *     (amax optional; it is reset by the call);
 *   direction 1: with dA = da[r]: dz[r] = bf16(dact(z[r], probs_p[r] dA))
 *     and dprobs_p[r] = sum_j dA[j] s[j] (fixed order); pad rows get
 *     dprobs_p 0.
 *   Same meaning as the fused epilogues of moe_grouped_mlp_fwd / _bwd: z, dz
 *   bf16 [M_cap][N1] in the interleaved column order (N1 = 2 I gated, I for
 *   sReLU); a, da bf16 [M_cap][I].  Rows holding data are written as
 *   above; pad rows inside the groups' padded spans get zeros (so column
 *   blocks of 32 rows quantized from them encode zeros there).
 * ---------------------------------------------------------------------- */
typedef struct moe_glu_args {
  int32_t direction;
  int32_t E, I;
  int64_t M_cap;
  moe_act_params act;
  const int32_t* split_sizes;
  const int32_t* padded_offsets;
  const float* probs_p;
  const void* z;
  void* a;
  float* amax;
  const void* da;
  void* dz;
  float* dprobs_p;
} moe_glu_args;

moe_status moe_glu_unfused(const moe_glu_args* args, void* stream);

/* ------------------------------------------------------------------------
 * moe_router_topk -- the top-k router of the sparse MoE block ([TE] Fig. 1:
 *   a top-2 router sends each token to two of eight experts, whose outputs
 *   are combined as a weighted sum; the layer's configs route by "softmax
 *   then top-k").
 *
 *   For every token t: p = softmax(logits[t]) over all E experts (fp32);
 *   expert_idx[t][0..k-1] = the experts of the k largest logits, in
 *   descending order, ties to the lower id; probs[t][j] = p[expert_idx[t][j]]
 *   (not renormalised).  The selection compares the logits themselves, so
 *   it is exact.  These are the expert_idx / probs moe_permute takes.
 *   logits float [T][E], expert_idx int32 [T][k], probs float [T][k], all
 *   device memory owned by the caller; logits must be finite.
 *   Needs T >= 1, 1 <= E <= 1024, 1 <= k <= min(E, 8); invalid arguments
 *   return MOE_ERR_INVALID_ARG before any launch.
 * ---------------------------------------------------------------------- */
typedef struct moe_router_args {
  int32_t T, E, k;
  const float* logits;
  int32_t* expert_idx;
  float* probs;
} moe_router_args;

moe_status moe_router_topk(const moe_router_args* args, void* stream);

/* ------------------------------------------------------------------------
 * moe_router_route -- the router and the routing metadata in one launch
 *   ([FK] § "Eliminating host-device synchronization and CPU launch
 *   overhead": per-group counts stay on the device, no host round trip;
 *   the AI-digest summary of the same work lists gating, top-k and routing
 *   fused into one launch).
 *
 *   Computes exactly what moe_router_topk followed by moe_permute with
 *   MOE_PERMUTE_BUILD_MAP computes, with the same router arithmetic (the
 *   same bits):
 *     expert_idx[T][k], probs[T][k]     as moe_router_topk, from
 *                                       logits [T][E_total]
 *     split_sizes, offsets (nullable), padded_offsets, row_id_map,
 *     row_src, probs_p                  as moe_permute BUILD_MAP, for the
 *                                       local experts first_expert ..
 *                                       first_expert + E - 1
 *   One workgroup per 256 tokens (64 when E_total > 32), all resident at
 *   once, with two grid-wide barriers inside the launch (bounded waits; see
 *   MOE_DEVERR_SYNC_TIMEOUT).
 *   workspace: moe_router_route_workspace_size(T, E_total, E) bytes whose
 *   first 4096 bytes (barrier counters) must be zero before the first call;
 *   every call leaves them as the next call expects, so one buffer serves any
 *   number of calls, of any sizes, and graph replays.  Calls that share a
 *   workspace must not overlap in time.
 *   Needs 1 <= T and at most min(512, 2 x the device's CU count) workgroups
 *   (T <= 131072 for E_total <= 32, T <= 32768 beyond, on MI355X), else
 *   MOE_ERR_UNSUPPORTED (moe_router_topk + moe_permute serve any size);
 *   1 <= E_total <= 1024,
 *   1 <= k <= min(E_total, 8), 1 <= E <= 1024, 0 <= first_expert, M_cap >= 1.
 *   Device problems as in moe_permute (MOE_DEVERR_MCAP_OVERFLOW).
 * ---------------------------------------------------------------------- */
typedef struct moe_router_route_args {
  int32_t T, E_total, k;          /* router: T tokens, top-k of E_total */
  int32_t E, first_expert;        /* local experts */
  int64_t M_cap;
  const float* logits;            /* [T][E_total] device, finite */
  int32_t* expert_idx;            /* [T][k]  device, out */
  float* probs;                   /* [T][k]  device, out */
  int32_t* split_sizes;           /* [E]     device, out */
  int32_t* offsets;               /* [E+1]   device, out (may be NULL) */
  int32_t* padded_offsets;        /* [E+1]   device, out */
  int32_t* row_id_map;            /* [T][k]  device, out */
  int32_t* row_src;               /* [M_cap] device, out */
  float* probs_p;                 /* [M_cap] device, out */
  int32_t* err_flag;              /* optional device int32 */
  void* workspace;                /* device, see above */
  size_t workspace_bytes;
} moe_router_route_args;

size_t moe_router_route_workspace_size(int T, int E_total, int E);
moe_status moe_router_route(const moe_router_route_args* args, void* stream);

/* Workspace bytes for these sizes: the backward needs at least the dprobs
 * partials (fp32 M_cap x ceil(I / 256)); the full size adds the area where
 * the plain-store GEMMs (FC2, FC1 dgrad) split their last, partial round of
 * tiles along K (partial tiles reduced in a fixed order, so results stay
 * deterministic).  One buffer may serve the forward and the backward. */
size_t moe_grouped_mlp_workspace_size(int E, int H, int I, int64_t M_cap,
                                      int prec, int act);

/* ------------------------------------------------------------------------
 * Measurement: the shader clock the grouped GEMMs ran at.
 *
 * The dense MFMA peak is quoted at the 2.4 GHz maximum shader clock; under
 * a sustained GEMM load the power manager runs the clock lower, so
 * throughput is also judged against the peak at the clock the work ran at.
 *
 * Clock trace of the grouped GEMMs.  While set, every
 * grouped-GEMM launch that follows (inside moe_grouped_mlp_fwd, _bwd,
 * _bwd_noalloc, _wgrad and moe_grouped_gemm) takes the next of `slots`
 * record areas in turn, and its workgroup i writes, as it ends,
 * area[2 i] = shader cycles and area[2 i + 1] = constant-rate ticks
 * (moe_clock_tick_rate_hz) since it started; area j starts at
 * records + j x 2 x MOE_CLOCK_MAX_WORKGROUPS.  Workgroups live for the
 * whole launch (persistent), so cycles / ticks x the tick rate is the clock
 * the GEMM ran at, on that workgroup's compute unit.  Launches with more
 * workgroups than MOE_CLOCK_MAX_WORKGROUPS record nothing.
 *   records: device int64 [slots][MOE_CLOCK_MAX_WORKGROUPS][2], caller-owned,
 *   kept until the trace is cleared; NULL clears the trace (slots ignored).
 *   1 <= slots <= 64, else MOE_ERR_INVALID_ARG.  Launches captured into a
 *   graph keep the area they were captured with.  The setting is global to
 *   the process; the slot counter restarts at 0 on every call. */
#define MOE_CLOCK_MAX_WORKGROUPS 1024
moe_status moe_gemm_clock_trace(int64_t* records, int slots);

/* Frequency of the constant-rate counter on the current device (Hz), 0 if
 * it cannot be read. */
int64_t moe_clock_tick_rate_hz(void);

/* Measurement: keeps `workgroups` compute units busy (one workgroup per CU,
 * holding 96 KB of LDS so that no grouped-GEMM workgroup fits beside it)
 * for `ticks` of the constant-rate counter, as a stand-in for a concurrent
 * kernel (expert- or data-parallel communication) when measuring how the
 * grouped GEMMs overlap with other work.  1 <= workgroups <= 1024 and
 * 1 <= ticks <= 1e8, else MOE_ERR_INVALID_ARG. */
moe_status moe_bench_occupy(int workgroups, int64_t ticks, void* stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status status);

/* Library version, e.g. 100 = 0.1.0. */
int moe_gmlp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_GMLP_H */
