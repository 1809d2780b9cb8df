"""Plain CPU oracle of the fused grouped-MLP MoE expert block.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  The product path
(moe_grouped_mlp_amd) never imports, links or runs it, and it imports
nothing from the product path.

Pages followed (cited by title and section):
  [FK] "Boosting MoE Training Throughput with Advanced Fusion Kernels",
       NVIDIA technical blog (zh-cn translation).
  [TE] "NVIDIA Transformer Engine 优化 MoE 生物基础模型训练", the TE +
       BioNeMo Mixtral tutorial.

What it computes, in float64, storing bf16 (round-to-nearest-even) or MXFP8
exactly where the GPU path stores such a tensor and computing exactly in
between:

  route      [TE § Challenge 1, the per-expert Python loop and GroupedLinear's
             split_sizes]; [FK § Eliminating host-device sync: per-group token
             counts live on the device]
  permute    gather of token rows into expert-contiguous order [TE § Challenge 1]
  repack     interleaving of the gate/up weight rows [FK § Optimizing GLU
             activations with fused GEMM epilogues, Fig. 2]
  fc1 / fc2  per-expert linear layers (GroupedLinear) [TE § Challenge 1]
  glu        SwiGLU(x,W,V,b,c,beta) = Swish_beta(xW+b) * (xV+c) [FK § Optimizing
             GLU activations, eq. SwiGLU]; GeGLU / sReLU and the clamp option
             [FK § Overcoming training bottlenecks, list of supported
             activations]; routing-probability scaling (ScaledSwiGLU)
             [TE § Challenge 3]
  unpermute  weighted combine by index-add [TE § Challenge 1]
  router     softmax over the experts, top-k [TE § dense vs sparse MoE block, Fig. 1]
  wgrad      per-expert weight gradients dW1 = dZ^T Xp, dW2 = dYp^T a
             [FK § Overcoming training bottlenecks, Fig. 1]
  backward   FC2 dgrad + dActivation [FK § Overcoming training bottlenecks,
             Fig. 1; § Optimizing GLU activations, backward epilogue], FC1
             dgrad, and the gradient of the routing probabilities
  MXFP8      [TE § Challenge 2, Fig. 3]; [FK § Fused MXFP8 and NVFP4
             quantization] (rowwise output plus a transposed copy)

Readings where the pages are silent (the same list is kept in the design
notes): gate half first (columns [0, I) get Swish), beta = 1 unless given,
clamp applied to both halves with an inclusive pass-through gradient, the
linear-half offset added after its clamp, probabilities multiplied into the
activation output (before FC2), rows inside a group in ascending token order,
group starts padded to 128 rows with zero pad rows, exact sums with one bf16
rounding per stored tensor.

Parity status: every function here is pinned by tests in tests/test_oracle_*.py
(closed forms, brute force on tiny inputs, library special cases, finite
differences, exhaustive format checks).  The blocking axis of every MX
operand (forward, backward, weight gradients; MXFP8 and MXFP4) is pinned by
data that MX blocks carry exactly along that axis and not along any other
(tests/test_oracle_mx_axes.py).  The grouped GEMMs at sizes beyond the
brute-force cases are pinned only through the E=1 dense special case and the
exact-arithmetic invariants.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
from scipy.special import erf

from .numerics import bf16_to_f64, mx_quantize, mx_dequantize, mxfp4_round, round_bf16

ALIGN = 128          # group-start alignment of the padded row layout
INTERLEAVE = 64      # gate/up interleave block of the repacked FC1 weight


# =============================================================== routing ===
@dataclasses.dataclass
class Routing:
    split_sizes: np.ndarray      # int32 [E]   rows per local expert
    offsets: np.ndarray          # int32 [E+1] exclusive scan of split_sizes
    padded_offsets: np.ndarray   # int32 [E+1] scan of sizes rounded to ALIGN
    row_id_map: np.ndarray       # int32 [T][k] row of (t, slot), -1 if none
    row_src: np.ndarray          # int32 [M_cap] token of a row, -1 for pad
    probs_p: np.ndarray          # float32 [M_cap] prob of a row, 0 for pad
    #                              (float64 when the caller passes float64)


def route(expert_idx: np.ndarray, probs: np.ndarray, E: int,
          first_expert: int = 0, M_cap: Optional[int] = None,
          align: int = ALIGN) -> Routing:
    """Expert-major row layout of the (token, slot) pairs that pick a local
    expert.

    For local expert e (global id first_expert + e) the rows are the tokens
    that picked it, in ascending token order -- the order in which the
    per-expert loop of [TE § Challenge 1] finds them.  Group e starts at row
    padded_offsets[e], a multiple of `align`.
    """
    expert_idx = np.asarray(expert_idx)
    T, k = expert_idx.shape
    local = expert_idx.astype(np.int64) - first_expert
    split = np.zeros(E, dtype=np.int64)
    members = []
    for e in range(E):
        t_idx, s_idx = np.nonzero(local == e)   # row-major: token ascending
        members.append((t_idx, s_idx))
        split[e] = len(t_idx)
    offsets = np.concatenate([[0], np.cumsum(split)])
    padded = np.concatenate([[0], np.cumsum(-(-split // align) * align)])
    if M_cap is None:
        M_cap = int(padded[-1])
    if padded[-1] > M_cap:
        raise ValueError("padded row count exceeds M_cap")
    row_id_map = np.full((T, k), -1, dtype=np.int32)
    row_src = np.full(M_cap, -1, dtype=np.int32)
    probs = np.asarray(probs)
    # float32 unless the caller passes float64 probabilities (exact mode)
    probs_p = np.zeros(M_cap, dtype=np.result_type(probs.dtype, np.float32))
    for e, (t_idx, s_idx) in enumerate(members):
        rows = padded[e] + np.arange(len(t_idx))
        row_id_map[t_idx, s_idx] = rows
        row_src[rows] = t_idx
        probs_p[rows] = probs[t_idx, s_idx]
    return Routing(split.astype(np.int32), offsets.astype(np.int32),
                   padded.astype(np.int32), row_id_map, row_src, probs_p)


def expert_of_rows(rt: Routing) -> np.ndarray:
    """Local expert of every valid row, -1 for pad rows."""
    M_cap = rt.row_src.shape[0]
    out = np.full(M_cap, -1, dtype=np.int64)
    for e in range(len(rt.split_sizes)):
        s = rt.padded_offsets[e]
        out[s:s + rt.split_sizes[e]] = e
    return out


def permute(x: np.ndarray, row_src: np.ndarray) -> np.ndarray:
    """Xp[r] = X[row_src[r]], pad rows (row_src = -1) are zero."""
    x = np.asarray(x)
    out = np.zeros((row_src.shape[0],) + x.shape[1:], dtype=x.dtype)
    ok = row_src >= 0
    out[ok] = x[row_src[ok]]
    return out


def unpermute(yp: np.ndarray, row_id_map: np.ndarray,
              round_out: bool = True) -> np.ndarray:
    """out[t] = sum over slots s with a local row of yp[row_id_map[t, s]],
    summed exactly in slot order and rounded once to bf16 (index-add combine
    of [TE § Challenge 1]); a token with no local expert gets zeros."""
    T, k = row_id_map.shape
    out = np.zeros((T, yp.shape[1]), dtype=np.float64)
    for s in range(k):
        r = row_id_map[:, s]
        ok = r >= 0
        out[ok] += yp[r[ok]]
    return round_bf16(out) if round_out else out


def gather_probs_grad(dp_rows: np.ndarray, row_id_map: np.ndarray
                      ) -> np.ndarray:
    """dprobs[t, s] = dp[row_id_map[t, s]], 0 where the slot is not local."""
    r = row_id_map
    return np.where(r >= 0, dp_rows[np.maximum(r, 0)], 0.0)


# ================================================================ repack ===
def interleave_rows(I: int, g: int = INTERLEAVE) -> np.ndarray:
    """For each packed FC1 output row, the logical row it holds.

    Logical rows [0, I) are the gate half, [I, 2I) the up half.  The packed
    layout alternates blocks of g gate rows and g up rows so that one output
    tile of width 2g holds matching halves of both ([FK § Optimizing GLU
    activations, Fig. 2]).
    """
    if I % g:
        raise ValueError("I must be a multiple of the interleave block")
    packed = np.empty(2 * I, dtype=np.int64)
    for j in range(I):
        base = 2 * g * (j // g) + j % g
        packed[base] = j
        packed[base + g] = I + j
    return packed


def repack_interleave(w1: np.ndarray, g: int = INTERLEAVE,
                      inverse: bool = False) -> np.ndarray:
    """[E][2I][H] gate|up weight <-> interleaved weight (a row permutation)."""
    I = w1.shape[1] // 2
    src = interleave_rows(I, g)
    if not inverse:
        return w1[:, src, :]
    out = np.empty_like(w1)
    out[:, src, :] = w1
    return out


# ============================================================ activation ===
@dataclasses.dataclass
class ActParams:
    act: str = "swiglu"           # "swiglu" | "geglu" | "srelu"
    beta: float = 1.0             # Swish_beta(x) = x * sigmoid(beta x)
    gate_lo: float = -np.inf
    gate_hi: float = np.inf
    lin_lo: float = -np.inf
    lin_hi: float = np.inf
    lin_offset: float = 0.0       # added to the linear half after its clamp

    @staticmethod
    def clamped(c: Optional[float], beta: float = 1.0, act: str = "swiglu"):
        if c is None:
            return ActParams(act=act, beta=beta)
        return ActParams(act=act, beta=beta, gate_lo=-c, gate_hi=c,
                         lin_lo=-c, lin_hi=c)

    @property
    def gated(self) -> bool:
        return self.act != "srelu"


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def swish(x, beta=1.0):
    return x * sigmoid(beta * x)


def swish_grad(x, beta=1.0):
    s = sigmoid(beta * x)
    return s * (1.0 + beta * x * (1.0 - s))


def gelu(x):
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def gelu_grad(x):
    cdf = 0.5 * (1.0 + erf(x / np.sqrt(2.0)))
    pdf = np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)
    return cdf + x * pdf


def _halves(z, prm: ActParams, bias=None):
    """Pre-clamp and clamped gate/linear halves of a logical FC1 output."""
    z = np.asarray(z, dtype=np.float64)
    if bias is not None:
        z = z + bias
    I = z.shape[-1] // 2
    g_pre, u_pre = z[..., :I], z[..., I:]
    g = np.clip(g_pre, prm.gate_lo, prm.gate_hi)
    u = np.clip(u_pre, prm.lin_lo, prm.lin_hi) + prm.lin_offset
    return g_pre, u_pre, g, u


def act_forward(z: np.ndarray, prm: ActParams, bias=None) -> np.ndarray:
    """Unscaled activation output s from the (logical-layout) FC1 output."""
    if not prm.gated:
        zz = np.asarray(z, dtype=np.float64)
        if bias is not None:
            zz = zz + bias
        zz = np.clip(zz, prm.gate_lo, prm.gate_hi)
        return np.maximum(zz, 0.0) ** 2
    _, _, g, u = _halves(z, prm, bias)
    if prm.act == "swiglu":
        return swish(g, prm.beta) * u
    if prm.act == "geglu":
        return gelu(g) * u
    raise ValueError(prm.act)


def act_backward(z: np.ndarray, ds: np.ndarray, prm: ActParams, bias=None
                 ) -> np.ndarray:
    """dL/dz given dL/ds, for the activation of act_forward.  Clamped
    positions pass gradient only where lo <= pre-clamp value <= hi."""
    if not prm.gated:
        zz = np.asarray(z, dtype=np.float64)
        if bias is not None:
            zz = zz + bias
        inside = (zz >= prm.gate_lo) & (zz <= prm.gate_hi)
        zc = np.clip(zz, prm.gate_lo, prm.gate_hi)
        return ds * 2.0 * np.maximum(zc, 0.0) * inside
    g_pre, u_pre, g, u = _halves(z, prm, bias)
    g_in = (g_pre >= prm.gate_lo) & (g_pre <= prm.gate_hi)
    u_in = (u_pre >= prm.lin_lo) & (u_pre <= prm.lin_hi)
    if prm.act == "swiglu":
        f, df = swish(g, prm.beta), swish_grad(g, prm.beta)
    elif prm.act == "geglu":
        f, df = gelu(g), gelu_grad(g)
    else:
        raise ValueError(prm.act)
    dg = ds * u * df * g_in
    du = ds * f * u_in
    return np.concatenate([dg, du], axis=-1)


# ================================================================ layer ====
def _maybe_bf16(v, on):
    return round_bf16(v) if on else v


@dataclasses.dataclass
class Forward:
    rt: Routing
    xp: np.ndarray        # [M_cap][H]   permuted input (bf16 values)
    z: np.ndarray         # [M_cap][N1]  FC1 output, logical layout, stored
    a: np.ndarray         # [M_cap][I]   prob-scaled activation, stored
    y: np.ndarray         # [M_cap][H]   FC2 output, stored
    out: np.ndarray       # [T][H]       combined output, stored
    amax: float           # max |a| over valid rows
    expert: np.ndarray    # [M_cap] local expert of each row, -1 for pad
    a_mx: Optional[tuple] = None    # (codes, scales) rowwise along I
    aT_mx: Optional[tuple] = None   # (codes [I][M_pad], scales) along M


@dataclasses.dataclass
class Backward:
    dyp: np.ndarray       # [M_cap][H]  permuted output gradient
    dz: np.ndarray        # [M_cap][N1] stored FC1-output gradient (logical)
    dp: np.ndarray        # [M_cap]     d loss / d probs_p
    dxp: np.ndarray       # [M_cap][H]  stored FC1 dgrad
    dx: np.ndarray        # [T][H]      stored input gradient
    dprobs: np.ndarray    # [T][k]
    dz_mx: Optional[tuple] = None
    dzT_mx: Optional[tuple] = None


def _mx_operand(v, axis, fmt):
    """The values a GEMM operand carries: v itself (fmt None), or its MXFP8
    or MXFP4 encoding in blocks of 32 along `axis`, decoded."""
    if fmt == "mxfp4":
        return mxfp4_round(v, axis)
    return mx_dequantize(*mx_quantize(v, axis), axis) if fmt else v


def _operand_format(mx, rnd):
    if not (mx and rnd):
        return None
    return "mxfp4" if mx == "mxfp4" else "mxfp8"


def forward(x_bits, w1_bits, w2_bits, expert_idx, probs, E, prm: ActParams,
            *, first_expert=0, M_cap=None, mx=False, exact=False,
            bias1=None, unfused=False) -> Forward:
    """Fused grouped-MLP forward, expert by expert.

    x_bits   uint16 bf16 [T][H]
    w1_bits  uint16 bf16 [E][N1][H], logical layout (N1 = 2I gated, I sReLU)
    w2_bits  uint16 bf16 [E][H][I]
    probs    float32 [T][k]
    mx       feed MXFP8 operands to both GEMMs (blocks of 32 along K);
             "mxfp4": MXFP4 operands instead [FK § Fused MXFP8 and NVFP4
             quantization names a 4-bit recipe; E2M1 with E8M0 scales per
             32 is its counterpart on MI355X]
    exact    skip every bf16/MX storage rounding (pure float64; used by the
             finite-difference pins)
    unfused  the layer run as separate kernels, each reading what the one
             before stored: the activation takes the stored (bf16) z instead
             of FC1's unrounded result [FK § Overcoming training bottlenecks:
             unfused, the activation is a separate kernel after the GEMM]
    """
    rnd = not exact
    fmt = _operand_format(mx, rnd)
    rt = route(expert_idx, probs, E, first_expert, M_cap)
    M_cap = rt.row_src.shape[0]
    x = bf16_to_f64(x_bits) if x_bits.dtype == np.uint16 else x_bits
    w1 = bf16_to_f64(w1_bits) if w1_bits.dtype == np.uint16 else w1_bits
    w2 = bf16_to_f64(w2_bits) if w2_bits.dtype == np.uint16 else w2_bits
    H = x.shape[1]
    N1 = w1.shape[1]
    I = w2.shape[2]
    xp = permute(x, rt.row_src)
    pp = rt.probs_p.astype(np.float64)
    z = np.zeros((M_cap, N1))
    a = np.zeros((M_cap, I))
    y = np.zeros((M_cap, H))
    for e in range(E):
        s0, n = int(rt.padded_offsets[e]), int(rt.split_sizes[e])
        if n == 0:
            continue
        rows = slice(s0, s0 + n)
        xe = _mx_operand(xp[rows], 1, fmt)
        w1e = _mx_operand(w1[e], 1, fmt)
        ze = xe @ w1e.T                                      # FC1
        b = None if bias1 is None else bias1[e]
        ain_z = _maybe_bf16(ze, rnd) if unfused else ze
        ae = pp[rows, None] * act_forward(ain_z, prm, b)     # act + prob scale
        z[rows] = _maybe_bf16(ze, rnd)
        a[rows] = _maybe_bf16(ae, rnd)
        ain = _mx_operand(a[rows], 1, fmt)
        w2e = _mx_operand(w2[e], 1, fmt)
        y[rows] = _maybe_bf16(ain @ w2e.T, rnd)              # FC2
    out = unpermute(y, rt.row_id_map, round_out=rnd)
    ex = expert_of_rows(rt)
    valid = ex >= 0
    amax = float(np.max(np.abs(a[valid]))) if valid.any() else 0.0
    fw = Forward(rt, xp, z, a, y, out, amax, ex)
    if fmt == "mxfp8":
        mp = int(rt.padded_offsets[-1])
        fw.a_mx = mx_quantize(a[:mp], 1)
        fw.aT_mx = mx_quantize(a[:mp].T, 1)
    return fw


def backward(fw: Forward, dout_bits, w1_bits, w2_bits, prm: ActParams, *,
             mx=False, exact=False, bias1=None, unfused=False) -> Backward:
    """Backward of `forward` for the loss sum(out * dOut).  unfused: FC2
    dgrad stores dA (bf16) and the activation gradient reads it."""
    rnd = not exact
    fmt = _operand_format(mx, rnd)
    rt = fw.rt
    E = len(rt.split_sizes)
    dout = bf16_to_f64(dout_bits) if dout_bits.dtype == np.uint16 \
        else dout_bits
    w1 = bf16_to_f64(w1_bits) if w1_bits.dtype == np.uint16 else w1_bits
    w2 = bf16_to_f64(w2_bits) if w2_bits.dtype == np.uint16 else w2_bits
    M_cap = rt.row_src.shape[0]
    N1, H = w1.shape[1], w1.shape[2]
    dyp = permute(dout, rt.row_src)          # unpermute backward = gather
    pp = rt.probs_p.astype(np.float64)
    dz = np.zeros((M_cap, N1))
    dp = np.zeros(M_cap)
    dxp = np.zeros((M_cap, H))
    for e in range(E):
        s0, n = int(rt.padded_offsets[e]), int(rt.split_sizes[e])
        if n == 0:
            continue
        rows = slice(s0, s0 + n)
        dye = _mx_operand(dyp[rows], 1, fmt)                 # along H
        w2e = _mx_operand(w2[e], 0, fmt)                     # along H
        da = dye @ w2e                                       # FC2 dgrad
        if unfused:
            da = _maybe_bf16(da, rnd)
        b = None if bias1 is None else bias1[e]
        ze = fw.z[rows]
        s = act_forward(ze, prm, b)
        dp[rows] = np.sum(da * s, axis=1)                    # d probs_p
        dze = act_backward(ze, pp[rows, None] * da, prm, b)  # dActivation
        dz[rows] = _maybe_bf16(dze, rnd)
        dzin = _mx_operand(dz[rows], 1, fmt)                 # along N1
        w1e = _mx_operand(w1[e], 0, fmt)                     # along N1
        dxp[rows] = _maybe_bf16(dzin @ w1e, rnd)             # FC1 dgrad
    dx = unpermute(dxp, rt.row_id_map, round_out=rnd)
    dprobs = gather_probs_grad(dp, rt.row_id_map)
    bw = Backward(dyp, dz, dp, dxp, dx, dprobs)
    if fmt == "mxfp8":
        mp = int(rt.padded_offsets[-1])
        bw.dz_mx = mx_quantize(dz[:mp], 1)
        bw.dzT_mx = mx_quantize(dz[:mp].T, 1)
    return bw


# ================================================================ router ===
def router_topk(logits: np.ndarray, k: int):
    """Top-k router of the sparse MoE block: each token goes to k of the E
    experts, whose outputs are combined weighted by the router's
    probabilities [TE § the dense vs sparse MoE block, Fig. 1, a top-2 router
    over eight experts].  Probabilities are the softmax of the token's logits
    over all E experts, the k largest kept without renormalisation, in
    descending order, ties to the lower expert id.  The selection compares
    the fp32 logits themselves (softmax is monotone), so it is exact; the
    kept probabilities are computed in float64 from them.

    Returns (expert_idx int32 [T][k], probs float64 [T][k])."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    x = lg.astype(np.float64)
    p = np.exp(x - x.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, -x), axis=1)[:, :k]    # logit descending, then id
    return order.astype(np.int32), np.take_along_axis(p, order, axis=1)


# ======================================================= weight gradients ===
def weight_grads(fw: Forward, bw: Backward, *, mx=False, exact=False):
    """Weight gradients of the loss sum(out * dOut), expert by expert: the
    weight-gradient GEMMs of the MoE backward, which [FK § Overcoming
    training bottlenecks in MoE blocks, Fig. 1] keeps outside the fused
    kernels.  For expert e over its routed rows r (GroupedLinear's per-expert
    weights [TE § Challenge 1]):

        dW1[e] = sum_r dZ[r]^T Xp[r]     [N1][H], logical FC1 layout
        dW2[e] = sum_r dYp[r]^T a[r]     [H][I]

    from the stored dZ, Xp, dYp and a, each result rounded to bf16 once.
    With mx every operand is its MXFP8 copy (mx="mxfp4": its MXFP4 copy)
    blocked along the routed rows, the contraction axis, with blocks
    starting at the group's padded start (the transposed copies of [FK §
    Fused MXFP8 and NVFP4 quantization]); pad rows hold zeros.  exact skips
    the rounding (finite-difference pins).
    """
    rnd = not exact
    rt = fw.rt
    E = len(rt.split_sizes)
    N1, H, I = bw.dz.shape[1], fw.xp.shape[1], fw.a.shape[1]
    dw1 = np.zeros((E, N1, H))
    dw2 = np.zeros((E, H, I))
    for e in range(E):
        s0, n = int(rt.padded_offsets[e]), int(rt.split_sizes[e])
        if n == 0:
            continue
        span = slice(s0, s0 + -(-n // ALIGN) * ALIGN)   # zero past row n
        dz, xp = bw.dz[span], fw.xp[span]
        dy, a = bw.dyp[span], fw.a[span]
        fmt = _operand_format(mx, rnd)
        dw1[e] = _maybe_bf16(_mx_operand(dz, 0, fmt).T @ _mx_operand(xp, 0, fmt), rnd)
        dw2[e] = _maybe_bf16(_mx_operand(dy, 0, fmt).T @ _mx_operand(a, 0, fmt), rnd)
    return dw1, dw2


# ============================================== per-row sampled checks ====
def sample_rows_forward(xp_rows, w1_e, w2_e, p_rows, prm: ActParams,
                        mx=False):
    """FC1 -> activation -> prob scale -> FC2 for a few rows of one expert
    (for spot checks at sizes where the whole layer is too slow).
    xp_rows float64 [n][H]; w1_e [N1][H] logical layout; w2_e [H][I];
    p_rows [n].  Returns the stored (bf16) z, a and y rows."""
    xe = _mx_operand(xp_rows, 1, mx)
    ze = xe @ _mx_operand(w1_e, 1, mx).T
    ae = round_bf16(p_rows[:, None] * act_forward(ze, prm))
    ye = _mx_operand(ae, 1, mx) @ _mx_operand(w2_e, 1, mx).T
    return round_bf16(ze), ae, round_bf16(ye)


def sample_rows_backward(dyp_rows, z_rows, w1_e, w2_e, p_rows,
                         prm: ActParams):
    """The backward of `backward` for a few rows of one expert (bf16
    operands): dA = dyp W2, the activation gradient from the stored z rows,
    dp = sum(dA * s), dxp = dz W1.  Returns the stored dz and dxp rows and
    dp."""
    da = dyp_rows @ w2_e
    s = act_forward(z_rows, prm)
    dp = np.sum(da * s, axis=1)
    dz = round_bf16(act_backward(z_rows, p_rows[:, None] * da, prm))
    dxp = round_bf16(dz @ w1_e)
    return dz, dxp, dp


def flops(M: int, H: int, I: int, gated: bool = True) -> dict:
    """Algorithmic flop counts of the four grouped GEMMs (unpadded rows)."""
    n1 = 2 * I if gated else I
    return {"fc1": 2 * M * H * n1, "fc2": 2 * M * H * I,
            "fc2_dgrad": 2 * M * H * I, "fc1_dgrad": 2 * M * H * n1}
