"""Helpers shared by the GPU parity tests: moving seeded inputs to the
device, running the HIP path through the C ABI, and comparing with the
oracle at the stated tolerances."""

from __future__ import annotations

import numpy as np
import torch

import moe_grouped_mlp_amd as mg
from oracle import moe as om
from oracle import numerics as nu

RTOL, ATOL = 2e-2, 1e-2          # bf16 outputs against the fp64 oracle
REL_ATOL = 1e-2                  # absolute slack relative to the tensor RMS


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.cuda().view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return nu.bf16_to_f64(host_bits(t))
    return t.detach().cpu().numpy().astype(np.float64)


def assert_close(gpu, ora, what, rtol=RTOL, atol=ATOL, rel_atol=REL_ATOL):
    """The stated bar (|d| <= atol + rtol |ref|) and a scale-aware one
    (|d| <= rel_atol * rms(ref) + rtol |ref|), so small-magnitude tensors
    are not waved through by the absolute term."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ora = np.asarray(ora, dtype=np.float64)
    assert gpu.shape == ora.shape, (what, gpu.shape, ora.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    d = np.abs(gpu - ora)
    rms = float(np.sqrt(np.mean(ora * ora))) if ora.size else 0.0
    ok1 = d <= atol + rtol * np.abs(ora)
    ok2 = d <= rel_atol * rms + rtol * np.abs(ora)
    bad = ~(ok1 & ok2)
    if bad.any():
        i = np.flatnonzero(bad.reshape(-1))[:5]
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outside tolerance; rms={rms:.3e} "
            f"max|d|={d.max():.3e}; first gpu={gpu.reshape(-1)[i]} "
            f"oracle={ora.reshape(-1)[i]}")


def act_of(wl, prm_override=None):
    """(binding ActParams, oracle ActParams) for a workload."""
    kind = {"swiglu": mg.ACT_SWIGLU, "geglu": mg.ACT_GEGLU,
            "srelu": mg.ACT_SRELU}[wl.act]
    c = wl.clamp
    gp = mg.act_params(kind, beta=wl.beta, clamp=c)
    op = om.ActParams.clamped(c, beta=wl.beta, act=wl.act)
    return gp, op


def run_gpu_layer(wl, M_cap=None, backward=True, block=None, prec=None,
                  bf16_copies=True, bias1=None):
    """Run the HIP path on a workload; returns the block holding the results
    (with MXFP8, also the optional bf16 a and dz unless bf16_copies=False)."""
    gp, _ = act_of(wl)
    blk = block or mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp,
                                  first_expert=wl.first_expert, M_cap=M_cap,
                                  prec=mg.PREC_BF16 if prec is None else prec,
                                  bf16_copies=bf16_copies)
    w1 = dev_bf16(wl.w1)
    w2 = dev_bf16(wl.w2)
    blk.load_weights(w1, w2, None if bias1 is None else
                     torch.from_numpy(np.asarray(bias1, dtype=np.float32)).cuda())
    x = dev_bf16(wl.x)
    idx = torch.from_numpy(wl.expert_idx.astype(np.int32)).cuda()
    probs = torch.from_numpy(wl.probs.astype(np.float32)).cuda()
    blk.forward(x, idx, probs)
    if backward:
        blk.backward(dev_bf16(wl.dout))
    torch.cuda.synchronize()
    return blk


def tail_split_parts(split_sizes, N: int, K: int, grid: int, k_step: int,
                     split_max: int = 4, split_min_k: int = 2) -> int:
    """K parts the plain-store grouped GEMM gives each tile of its last,
    partial round (the kernel's default rule: split only when the tail
    leaves at least half the grid idle).  Used to make sure a test really
    reaches the split-K path; 1 means no split."""
    total = sum(-(-int(s) // 256) for s in split_sizes) * (-(-N // 256))
    tail = total % grid
    if tail == 0 or 2 * tail > grid:
        return 1
    return min(grid // tail, split_max, max(1, -(-K // k_step) // split_min_k))


def gemm_grid(cu_margin: int, M_cap: int, E: int, N: int) -> int:
    """Workgroups of a grouped GEMM launch (one per CU, minus the margin, a
    multiple of 8, at most the tiles that can exist)."""
    g = torch.cuda.get_device_properties(0).multi_processor_count - cu_margin
    if g >= 8:
        g -= g % 8
    ub = (-(-M_cap // 256) + E) * (-(-N // 256))
    return max(1, min(g, ub))


def uninterleave_cols(packed: np.ndarray, I: int) -> np.ndarray:
    """Packed (gate/up interleaved) columns -> logical gate|up columns."""
    src = om.interleave_rows(I)
    out = np.empty_like(packed)
    out[..., src] = packed
    return out


def oracle_layer(wl, M_cap, backward=True, mx=False, unfused=False, bias1=None):
    _, op = act_of(wl)
    b = None if bias1 is None else np.asarray(bias1, dtype=np.float64)
    fw = om.forward(wl.x, wl.w1, wl.w2, wl.expert_idx, wl.probs, wl.E, op,
                    first_expert=wl.first_expert, M_cap=M_cap, mx=mx, unfused=unfused,
                    bias1=b)
    bw = om.backward(fw, wl.dout, wl.w1, wl.w2, op, mx=mx,
                     unfused=unfused, bias1=b) if backward else None
    return fw, bw


# ---------------------------------------------------------------- MXFP8 ---
def mx_scale_index(R: int, K: int) -> np.ndarray:
    """[R][K/32] byte offsets of the tiled MXFP8 scale layout documented in
    include/moe_gmlp.h (row r, block b)."""
    r = np.arange(R)[:, None]
    b = np.arange(K // 32)[None, :]
    return ((r // 32) * (K // 64) + b // 2) * 64 + (b % 2) * 32 + r % 32


def mx_scales_plain(s_tiled: torch.Tensor, R: int, K: int) -> np.ndarray:
    """Tiled scale bytes (one [R][K] operand) -> plain [R][K/32]."""
    s = s_tiled.detach().cpu().numpy().reshape(-1)
    return s[mx_scale_index(R, K)]


def assert_mx_equal(q_gpu, s_plain_gpu, ref, what):
    """Codes and scales bit-exact against the oracle's (codes, scales)."""
    codes, scales = ref
    q = q_gpu.detach().cpu().numpy() if isinstance(q_gpu, torch.Tensor) else q_gpu
    bad = np.flatnonzero(q.reshape(-1) != codes.reshape(-1))
    assert bad.size == 0, (f"{what}: {bad.size} of {codes.size} codes differ; first at "
                           f"{bad[:5]}: gpu {q.reshape(-1)[bad[:5]]} oracle "
                           f"{codes.reshape(-1)[bad[:5]]}")
    bad = np.flatnonzero(s_plain_gpu.reshape(-1) != scales.reshape(-1))
    assert bad.size == 0, (f"{what}: {bad.size} of {scales.size} scales differ; first at "
                           f"{bad[:5]}: gpu {s_plain_gpu.reshape(-1)[bad[:5]]} oracle "
                           f"{scales.reshape(-1)[bad[:5]]}")


def compare_routing(blk, rt):
    np.testing.assert_array_equal(blk.split_sizes.cpu().numpy(), rt.split_sizes)
    np.testing.assert_array_equal(blk.offsets.cpu().numpy(), rt.offsets)
    np.testing.assert_array_equal(blk.padded_offsets.cpu().numpy(),
                                  rt.padded_offsets)
    np.testing.assert_array_equal(blk.row_id_map.cpu().numpy(), rt.row_id_map)
    np.testing.assert_array_equal(blk.row_src.cpu().numpy(), rt.row_src)
    np.testing.assert_array_equal(blk.probs_p.cpu().numpy(), rt.probs_p)


def compare_layer(blk, wl, fw, bw):
    """Element-by-element comparison of every stored tensor of the step."""
    compare_routing(blk, fw.rt)
    mp = int(fw.rt.padded_offsets[-1])
    valid = fw.expert >= 0
    # permuted input: bit-exact, pad rows zero
    np.testing.assert_array_equal(host_bits(blk.xp)[:mp],
                                  nu.f64_to_bf16_bits(fw.xp[:mp]))
    gated = wl.act != "srelu"
    z = host_f64(blk.z)[valid]
    if gated:
        z = uninterleave_cols(z, wl.I)
    assert_close(z, fw.z[valid], "z")
    a_gpu = host_f64(blk.a)[valid]
    assert_close(a_gpu, fw.a[valid], "a")
    amax = float(blk.amax.cpu()[0])
    assert amax == np.abs(a_gpu).max()
    assert abs(amax - fw.amax) <= 2.0 ** -7 * fw.amax + 1e-30
    assert_close(host_f64(blk.yp)[valid], fw.y[valid], "yp")
    assert_close(host_f64(blk.out), fw.out, "out")
    if bw is None:
        return
    np.testing.assert_array_equal(host_bits(blk.dyp)[valid],
                                  nu.f64_to_bf16_bits(bw.dyp[valid]))
    dz = host_f64(blk.dz)[valid]
    if gated:
        dz = uninterleave_cols(dz, wl.I)
    assert_close(dz, bw.dz[valid], "dz")
    dp = blk.dprobs_p.cpu().numpy().astype(np.float64)
    assert_close(dp[valid], bw.dp[valid], "dprobs_p")
    assert np.all(dp[:mp][~valid[:mp]] == 0)
    assert_close(host_f64(blk.dxp)[valid], bw.dxp[valid], "dxp")
    assert_close(host_f64(blk.dx), bw.dx, "dx")
    assert_close(blk.dprobs.cpu().numpy(), bw.dprobs, "dprobs")


def e4m3_ordinal(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes -> signed ordinal (neighbouring values differ by 1, +0 and
    -0 both map to 0)."""
    c = np.asarray(codes).astype(np.int64)
    m = c & 0x7F
    return np.where(c & 0x80, -m, m)


# MXFP8 outputs against the oracle fed the same MXFP8 operands.  The oracle
# sums exactly; the scaled fp8 MFMA rounds its internal sums (about 16
# significant bits of the block partial sums) and the stored bf16 results can
# then differ from the oracle's by a unit in the last place, which moves the
# MXFP8 code of such a value to a neighbouring code when it sits near a
# rounding boundary of E4M3 (3 mantissa bits), and a flipped code changes one
# term of the next GEMM by 2^-3 of its size.  So:
#   * every element stays within the stated bar (rtol 2e-2, atol 1e-2);
#   * at most MX_OUTLIER_FRAC of the elements leave the scale-aware bar of
#     the bf16 path (rel_atol 1e-2 of the RMS);
#   * the relative L2 error stays below MX_REL_L2.
MX_OUTLIER_FRAC = 5e-3
MX_REL_L2 = 1e-2


def assert_close_mx(gpu, ora, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    ora = np.asarray(ora, dtype=np.float64)
    assert gpu.shape == ora.shape, (what, gpu.shape, ora.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    d = np.abs(gpu - ora)
    bad = d > ATOL + RTOL * np.abs(ora)
    assert not bad.any(), f"{what}: {bad.sum()} elements outside rtol {RTOL} / atol {ATOL}"
    rms = float(np.sqrt(np.mean(ora * ora))) if ora.size else 0.0
    out = d > REL_ATOL * rms + RTOL * np.abs(ora)
    assert out.mean() <= MX_OUTLIER_FRAC, \
        f"{what}: {out.sum()} of {out.size} outside the scale-aware bar"
    l2 = float(np.linalg.norm(d) / max(np.linalg.norm(ora), 1e-300))
    assert l2 <= MX_REL_L2, f"{what}: relative L2 error {l2:.3e}"


# A contraction over MXFP8 operands that the GPU and the oracle encoded from
# values an ulp apart: a code can move by one E4M3 step (2^-3 of its value's
# binade) in either operand, and a block whose amax crosses a power of two
# moves all 32 codes, so one product can change by up to (1 + 2^-3)^2 - 1 <
# 0.27 of |a| |b|.  Every element then lies within 0.27 (|A|^T |B|) of the
# oracle's (plus bf16 output rounding); the scale-aware bar of
# assert_close_mx holds on all but MX_OUTLIER_FRAC of the elements and the
# relative L2 error stays below MX_REL_L2.
MX_PRODUCT_STEP = (1 + 2.0 ** -3) ** 2 - 1


def assert_close_mx_contraction(gpu, ora, abs_prod, what):
    """abs_prod: |A|^T |B| of the contraction, elementwise (same shape)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ora = np.asarray(ora, dtype=np.float64)
    assert gpu.shape == ora.shape == abs_prod.shape, (what, gpu.shape, ora.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    d = np.abs(gpu - ora)
    bound = MX_PRODUCT_STEP * abs_prod + 2.0 ** -8 * np.abs(ora) + 1e-30
    over = d > bound
    assert not over.any(), f"{what}: {over.sum()} elements beyond the MXFP8 step bound"
    rms = float(np.sqrt(np.mean(ora * ora))) if ora.size else 0.0
    out = d > REL_ATOL * rms + RTOL * np.abs(ora)
    assert out.mean() <= MX_OUTLIER_FRAC, \
        f"{what}: {out.sum()} of {out.size} outside the scale-aware bar"
    l2 = float(np.linalg.norm(d) / max(np.linalg.norm(ora), 1e-300))
    assert l2 <= MX_REL_L2, f"{what}: relative L2 error {l2:.3e}"


def assert_mx_near(q_gpu, s_plain_gpu, ref, what, code_frac=2e-3, far_frac=1e-4,
                   scale_frac=1e-3):
    """MXFP8 copies written by a fused epilogue against the oracle's encoding
    of its own pre-cast values (which differ from the GPU's by the GEMM
    rounding, see above): scales equal on all but `scale_frac` of the blocks
    (and then one binade apart); where scales agree, codes equal on all but
    `code_frac` of the values and more than one E4M3 step apart on at most
    `far_frac`."""
    codes, scales = ref
    q = q_gpu.detach().cpu().numpy() if isinstance(q_gpu, torch.Tensor) else q_gpu
    sd = np.abs(s_plain_gpu.astype(np.int64) - scales.astype(np.int64))
    assert sd.max(initial=0) <= 1, f"{what}: a scale differs by {sd.max()} binades"
    assert (sd > 0).mean() <= scale_frac, f"{what}: {(sd > 0).sum()} scales differ"
    # compare codes inside blocks whose scales agree
    K = codes.shape[-1]
    same = np.repeat(sd == 0, 32, axis=-1).reshape(codes.shape)
    dist = np.abs(e4m3_ordinal(q) - e4m3_ordinal(codes))[same]
    if dist.size:
        assert (dist > 0).mean() <= code_frac, \
            f"{what}: {(dist > 0).sum()} of {dist.size} codes differ"
        assert (dist > 1).mean() <= far_frac, \
            f"{what}: {(dist > 1).sum()} codes differ by more than one step"


# The parity rule for the MXFP8 copies a fused epilogue writes: the oracle's
# encoder applied to the GPU's own bf16 pre-cast tensor (the stored a or dz,
# pad rows of each group as zeros) must give the same scales bit for bit,
# and codes may differ by one E4M3 step on at most MX_CODE_FRAC of the
# values.  Both sides encode the same bf16 numbers with the same rule, so no
# difference is expected; the allowance is the stated bar.
MX_CODE_FRAC = 1e-3


def assert_mx_rule(q_gpu, s_plain_gpu, ref, what):
    codes, scales = ref
    q = q_gpu.detach().cpu().numpy() if isinstance(q_gpu, torch.Tensor) else q_gpu
    q = np.asarray(q).reshape(codes.shape)
    s_plain_gpu = np.asarray(s_plain_gpu).reshape(scales.shape)
    bad = np.flatnonzero(s_plain_gpu.reshape(-1) != scales.reshape(-1))
    assert bad.size == 0, (f"{what}: {bad.size} of {scales.size} scales differ; first at "
                           f"{bad[:5]}: gpu {s_plain_gpu.reshape(-1)[bad[:5]]} oracle "
                           f"{scales.reshape(-1)[bad[:5]]}")
    # no NaN code (0x7f / 0xff): the block rule saturates at 448
    nan = np.flatnonzero((q.reshape(-1) & 0x7f) == 0x7f)
    assert nan.size == 0, f"{what}: {nan.size} NaN codes, first at {nan[:5]}"
    dist = np.abs(e4m3_ordinal(q) - e4m3_ordinal(codes))
    assert dist.max(initial=0) <= 1, f"{what}: a code differs by {dist.max()} steps"
    assert (dist > 0).mean() <= MX_CODE_FRAC, \
        f"{what}: {(dist > 0).sum()} of {dist.size} codes differ by one step"


def rows_with_pad_zeroed(values: np.ndarray, valid: np.ndarray) -> np.ndarray:
    """The pre-cast tensor the MXFP8 copies encode: the stored rows where
    they hold data, zeros on the pad rows of each group."""
    out = np.array(values, dtype=np.float64, copy=True)
    out[~valid] = 0.0
    return out


def assert_fused_mx_copies(blk, prefix, values, valid, n, what):
    """The rowwise ({prefix}_q/_s, blocks along n) and transposed
    ({prefix}T_q/_s, blocks of 32 rows along M) MXFP8 copies of the GPU's
    own [mp][n] tensor `values` (GPU column order), under assert_mx_rule."""
    mp = values.shape[0]
    v = rows_with_pad_zeroed(values, valid)
    q, sc = getattr(blk, prefix + "_q"), getattr(blk, prefix + "_s")
    assert_mx_rule(q.cpu().numpy()[:mp], mx_scales_plain(sc, blk.M_cap, n)[:mp],
                   nu.mx_quantize(v, axis=1), f"{what} MX rowwise (self)")
    qT, sT = getattr(blk, prefix + "T_q"), getattr(blk, prefix + "T_s")
    if qT is not None:
        assert_mx_rule(qT.cpu().numpy()[:, :mp], mx_scales_plain(sT, n, blk.M_cap)[:, :mp // 32],
                       nu.mx_quantize(v.T, axis=1), f"{what} MX transposed (self)")
