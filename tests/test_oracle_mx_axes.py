"""Pins of the blocking axis of every MX operand the oracle reads.

A 32-value MXFP8 (or MXFP4) block shares one power-of-two scale ("NVIDIA Transformer
Engine 优化 MoE 生物基础模型训练", § "Challenge 2", Fig. 3: E4M3 values with
one E8M0 scale per 32 consecutive values along the contraction axis).  Data
built so that every block along the documented axis holds values of one
magnitude class from {+-1, +-2} * 2^m is carried exactly by MXFP8 and by
MXFP4 (E2M1 holds 1, 2 and 4 exactly), while a
block along any other axis mixes the classes 2^0 and 2^-20: with the block's
scale set by the large values, 2^-20 lies below half the smallest E4M3
subnormal step (MXFP4: below half its smallest step) and encodes as zero.  So on such data

  * the MX reading of the layer equals its bf16 reading bit for bit, when
    (and only when) each operand is blocked along the axis the format
    prescribes for it, and
  * blocking any one of them along another axis (or, for the transposed
    copies of the weight-gradient GEMMs, from another row origin than the
    group's padded start) zeroes part of an operand and moves the result.

Every product and sum below is exact in float64 (at most 50 significant
bits), so "equal" means equal bits.  The expected weight gradients are
written out directly as sums over each group's rows, with no MX step.
"""

import numpy as np
import pytest

from oracle import moe
from oracle import numerics as nu

SMALL = 2.0 ** -20


def _lossless(x, axis):
    """Both formats carry x exactly in blocks along axis."""
    return (np.array_equal(nu.mx_round(x, axis), x)
            and np.array_equal(nu.mxfp4_round(x, axis), x))


def _lossy(x, axis):
    """Neither format carries x exactly in blocks along axis."""
    return (not np.array_equal(nu.mx_round(x, axis), x)
            and not np.array_equal(nu.mxfp4_round(x, axis), x))


def _signed_pm12(rng, shape):
    """Random values from {+-1, +-2}."""
    return rng.choice(np.array([-2.0, -1.0, 1.0, 2.0]), size=shape)


def _routing(sizes, seed):
    """k = 1 routing whose groups have the given sizes (tokens shuffled, so
    a group's rows are not a contiguous token range)."""
    rng = np.random.default_rng(seed)
    idx = np.concatenate([np.full(n, e, np.int32) for e, n in enumerate(sizes)])
    rng.shuffle(idx)
    T = len(idx)
    probs = np.ones((T, 1), np.float32)
    rt = moe.route(idx[:, None], probs, len(sizes))
    return idx[:, None], probs, rt


def _row_parity(rt):
    """Parity of each row's position inside its group (-1 for pad rows)."""
    par = np.full(rt.row_src.shape[0], -1, np.int64)
    for e, n in enumerate(rt.split_sizes):
        s0 = int(rt.padded_offsets[e])
        par[s0:s0 + n] = np.arange(n) % 2
    return par


def _bf16_bits(v):
    """float64 values on the bf16 grid -> uint16 bf16 bits."""
    assert np.array_equal(nu.round_bf16(v), v)
    return nu.f64_to_bf16_bits(v)


SIZES = [45, 70, 0, 33]        # no size a multiple of 32, one empty group
H, I = 64, 64


# ------------------------------------------------------------- forward ----
FORMATS = [pytest.param(True, id="mxfp8"), pytest.param("mxfp4", id="mxfp4")]


@pytest.mark.parametrize("fmt", FORMATS)
def test_forward_fc1_operands_blocked_along_h(fmt):
    """FC1 reads Xp and W1 blocked along H: rows of Xp alternate magnitude
    along M, rows of W1 alternate along N1; both are uniform along H."""
    rng = np.random.default_rng(1)
    idx, probs, rt = _routing(SIZES, 11)
    T = idx.shape[0]
    par_row = _row_parity(rt)
    tok_par = par_row[rt.row_id_map[:, 0]]
    x = _signed_pm12(rng, (T, H)) * np.where(tok_par == 1, SMALL, 1.0)[:, None]
    w1 = _signed_pm12(rng, (4, 2 * I, H)) * np.where(
        np.arange(2 * I) % 2 == 1, SMALL, 1.0)[None, :, None]
    w2 = _signed_pm12(rng, (4, H, I))
    xp = moe.permute(x, rt.row_src)
    assert _lossless(xp, 1) and _lossy(xp[:64], 0)
    assert _lossless(w1[0], 1) and _lossy(w1[0], 0)
    prm = moe.ActParams()
    args = (_bf16_bits(x), _bf16_bits(w1), _bf16_bits(w2), idx, probs, 4, prm)
    ref = moe.forward(*args)
    got = moe.forward(*args, mx=fmt)
    np.testing.assert_array_equal(got.z, ref.z)
    np.testing.assert_array_equal(got.a, ref.a)


@pytest.mark.parametrize("fmt", FORMATS)
def test_forward_fc2_operands_blocked_along_i_and_copies_of_a(fmt):
    """FC2 reads a and W2 blocked along I.  sReLU of a one-hot FC1 makes a
    row of a hold {0, 1, 4} times its row's class (2^0 or 2^-20), so a
    is exact along I and not along M; W2's rows alternate along H.  The
    forward's rowwise copy of a decodes to a; its transposed copy (blocks
    along M) does not."""
    rng = np.random.default_rng(2)
    idx, probs, rt = _routing(SIZES, 12)
    T = idx.shape[0]
    par_row = _row_parity(rt)
    tok_par = par_row[rt.row_id_map[:, 0]]
    x = np.zeros((T, H))
    hot = rng.integers(0, H, T)
    x[np.arange(T), hot] = rng.choice([-1.0, 1.0], T) * np.where(tok_par == 1, 2.0 ** -10, 1.0)
    w1 = _signed_pm12(rng, (4, I, H))          # sReLU: FC1 width I
    w2 = _signed_pm12(rng, (4, H, I)) * np.where(
        np.arange(H) % 2 == 1, SMALL, 1.0)[None, :, None]
    prm = moe.ActParams(act="srelu")
    args = (_bf16_bits(x), _bf16_bits(w1), _bf16_bits(w2), idx, probs, 4, prm)
    ref = moe.forward(*args)
    got = moe.forward(*args, mx=fmt)
    mp = int(rt.padded_offsets[-1])
    a = ref.a[:mp]
    assert _lossless(a, 1) and _lossy(a, 0)
    assert _lossless(w2[0], 1) and _lossy(w2[0], 0)
    np.testing.assert_array_equal(got.y, ref.y)
    np.testing.assert_array_equal(got.out, ref.out)
    if fmt is True:
        np.testing.assert_array_equal(nu.mx_dequantize(*got.a_mx, 1), a)
        assert not np.array_equal(nu.mx_dequantize(*got.aT_mx, 1), a.T)


# ------------------------------------------------------------ backward ----
def _forward_with_z(rt, z):
    """A Forward whose only fields the backward reads are set (rt, z)."""
    M_cap = rt.row_src.shape[0]
    zero = np.zeros((M_cap, 1))
    return moe.Forward(rt, zero, z, zero, zero, zero, 0.0, moe.expert_of_rows(rt))


@pytest.mark.parametrize("fmt", FORMATS)
def test_backward_fc2_dgrad_operands_blocked_along_h(fmt):
    """FC2 dgrad reads dYp and W2 blocked along H: rows of dYp alternate
    magnitude along M, columns of W2 [H][I] alternate along I; both are
    uniform along H.  dz and dp then come out of the MX reading unchanged."""
    rng = np.random.default_rng(3)
    idx, probs, rt = _routing(SIZES, 13)
    T = idx.shape[0]
    M_cap = rt.row_src.shape[0]
    tok_par = _row_parity(rt)[rt.row_id_map[:, 0]]
    dout = _signed_pm12(rng, (T, H)) * np.where(tok_par == 1, SMALL, 1.0)[:, None]
    w2 = _signed_pm12(rng, (4, H, I)) * np.where(
        np.arange(I) % 2 == 1, SMALL, 1.0)[None, None, :]
    w1 = _signed_pm12(rng, (4, 2 * I, H))
    z = nu.round_bf16(rng.standard_normal((M_cap, 2 * I)))
    dyp = moe.permute(dout, rt.row_src)
    assert _lossless(dyp, 1) and _lossy(dyp[:64], 0)
    assert _lossless(w2[0], 0) and _lossy(w2[0], 1)
    fw = _forward_with_z(rt, z)
    prm = moe.ActParams()
    args = (fw, _bf16_bits(dout), _bf16_bits(w1), _bf16_bits(w2), prm)
    ref = moe.backward(*args)
    got = moe.backward(*args, mx=fmt)
    np.testing.assert_array_equal(got.dz, ref.dz)
    np.testing.assert_array_equal(got.dp, ref.dp)


@pytest.mark.parametrize("fmt", FORMATS)
def test_backward_fc1_dgrad_operands_blocked_along_n1_and_copies_of_dz(fmt):
    """FC1 dgrad reads dZ and W1 blocked along N1.  With the gate half of z
    at 0 and the up half at 2, dSwiGLU gives dz_gate = p dA exactly and
    dz_up = 0 (Swish(0) = 0, Swish'(0) = 1/2); a one-hot dYp row times W2
    makes dA a row of W2 scaled by the row's class, so dz is exact along N1
    and not along M.  W1's columns alternate along H.  dxp and dX then
    come out of the MX reading unchanged, the rowwise copy of dz decodes to
    dz and its transposed copy does not."""
    rng = np.random.default_rng(4)
    idx, probs, rt = _routing(SIZES, 14)
    T = idx.shape[0]
    M_cap = rt.row_src.shape[0]
    tok_par = _row_parity(rt)[rt.row_id_map[:, 0]]
    dout = np.zeros((T, H))
    dout[np.arange(T), rng.integers(0, H, T)] = (
        _signed_pm12(rng, T) * np.where(tok_par == 1, SMALL, 1.0))
    w2 = _signed_pm12(rng, (4, H, I))
    w1 = _signed_pm12(rng, (4, 2 * I, H)) * np.where(
        np.arange(H) % 2 == 1, SMALL, 1.0)[None, None, :]
    z = np.concatenate([np.zeros((M_cap, I)), np.full((M_cap, I), 2.0)], axis=1)
    fw = _forward_with_z(rt, z)
    prm = moe.ActParams()
    args = (fw, _bf16_bits(dout), _bf16_bits(w1), _bf16_bits(w2), prm)
    ref = moe.backward(*args)
    got = moe.backward(*args, mx=fmt)
    mp = int(rt.padded_offsets[-1])
    dz = ref.dz[:mp]
    assert _lossless(dz, 1) and _lossy(dz, 0)
    assert _lossless(w1[0], 0) and _lossy(w1[0], 1)
    np.testing.assert_array_equal(got.dz, ref.dz)
    np.testing.assert_array_equal(got.dxp, ref.dxp)
    np.testing.assert_array_equal(got.dx, ref.dx)
    if fmt is True:
        np.testing.assert_array_equal(nu.mx_dequantize(*got.dz_mx, 1), dz)
        assert not np.array_equal(nu.mx_dequantize(*got.dzT_mx, 1), dz.T)


# ---------------------------------------------------- weight gradients ----
def _wgrad_case(rt, rng, scale_of_row, scale_of_col):
    """Stored dz, xp, dyp, a with magnitudes scale_of_row(r) *
    scale_of_col(c); rows past each group's data are zero (pad rows)."""
    M_cap = rt.row_src.shape[0]
    valid = moe.expert_of_rows(rt) >= 0
    rs = np.array([scale_of_row(r) for r in range(M_cap)]) * valid

    def mk(n):
        return _signed_pm12(rng, (M_cap, n)) * rs[:, None] * np.array(
            [scale_of_col(c) for c in range(n)])[None, :]
    M0 = np.zeros((M_cap, 1))
    fw = moe.Forward(rt, mk(H), M0, mk(I), M0, M0, 0.0, moe.expert_of_rows(rt))
    bw = moe.Backward(mk(H), mk(2 * I), np.zeros(M_cap), M0, M0, M0)
    return fw, bw


def _expected_wgrads(fw, bw):
    """dW1[e] = sum over the group's rows of dz[r]^T xp[r], dW2[e] likewise
    from dyp and a, rounded to bf16 once; no MX step."""
    rt = fw.rt
    E = len(rt.split_sizes)
    dw1 = np.zeros((E, 2 * I, H))
    dw2 = np.zeros((E, H, I))
    for e in range(E):
        s0, n = int(rt.padded_offsets[e]), int(rt.split_sizes[e])
        for r in range(s0, s0 + n):
            dw1[e] += np.outer(bw.dz[r], fw.xp[r])
            dw2[e] += np.outer(bw.dyp[r], fw.a[r])
    return nu.round_bf16(dw1), nu.round_bf16(dw2)


@pytest.mark.parametrize("fmt", FORMATS)
def test_weight_grad_operands_blocked_along_routed_rows(fmt):
    """Every weight-gradient operand is blocked along the routed rows (the
    contraction axis): magnitudes alternating along the columns leave that
    blocking exact and would not survive blocks along the columns."""
    rng = np.random.default_rng(5)
    _, _, rt = _routing(SIZES, 15)
    fw, bw = _wgrad_case(rt, rng, lambda r: 1.0,
                         lambda c: SMALL if c % 2 else 1.0)
    assert _lossy(bw.dz, 1) and _lossy(fw.xp, 1)
    exp1, exp2 = _expected_wgrads(fw, bw)
    got1, got2 = moe.weight_grads(fw, bw, mx=fmt)
    np.testing.assert_array_equal(got1, exp1)
    np.testing.assert_array_equal(got2, exp2)


@pytest.mark.parametrize("fmt", FORMATS)
def test_weight_grad_blocks_start_at_the_padded_group_start(fmt):
    """Blocks of 32 rows start at each group's padded start: magnitudes
    constant over rows [s0 + 32 j, s0 + 32 j + 32) and alternating with j
    are exact in those blocks.  The unpadded offsets (45, 115, 115) are not
    multiples of 32, so blocks counted from them, or from row 0 of the
    unpadded layout, would straddle two classes."""
    rng = np.random.default_rng(6)
    _, _, rt = _routing(SIZES, 16)
    starts = rt.padded_offsets
    assert any(o % 32 for o in rt.offsets[1:-1])

    def row_scale(r):
        e = int(np.searchsorted(starts, r, side="right") - 1)
        return SMALL if ((r - starts[e]) // 32) % 2 else 1.0

    fw, bw = _wgrad_case(rt, rng, row_scale, lambda c: 1.0)
    # blocks shifted by the unpadded start of group 1 lose the small rows
    s1, o1 = int(starts[1]), int(rt.offsets[1])
    shift = (s1 - o1) % 32
    seg = bw.dz[s1 - shift:s1 - shift + 64]
    assert _lossy(seg, 0)
    exp1, exp2 = _expected_wgrads(fw, bw)
    got1, got2 = moe.weight_grads(fw, bw, mx=fmt)
    np.testing.assert_array_equal(got1, exp1)
    np.testing.assert_array_equal(got2, exp2)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("n", [1, 31, 33, 95])
def test_weight_grad_partial_last_block(n, fmt):
    """A group whose size is not a multiple of 32 ends in a partial block
    filled with the zero pad rows; it is still exact."""
    rng = np.random.default_rng(7 + n)
    _, _, rt = _routing([n, 50], 17 + n)
    fw, bw = _wgrad_case(rt, rng, lambda r: 1.0, lambda c: 1.0)
    exp1, exp2 = _expected_wgrads(fw, bw)
    got1, got2 = moe.weight_grads(fw, bw, mx=fmt)
    np.testing.assert_array_equal(got1, exp1)
    np.testing.assert_array_equal(got2, exp2)


def test_weight_grads_mxfp4_rounds_its_operands_on_the_e2m1_grid():
    """mx="mxfp4" encodes the weight-gradient operands in E2M1, not E4M3:
    with dz and dyp entries of magnitude 1.25 in blocks whose largest value
    is 1.25, the block scale is 2^(0 - 2) and the E2M1 grid around 1.25 is
    {1, 1.5} (4 and 6 times the scale): 1.25 is the midpoint and rounds to
    the even code, 1.  MXFP8 carries 1.25 exactly (E4M3 has 3 mantissa
    bits).  The expected gradients are the sums over each group's rows with
    1.25 replaced by 1 (MXFP4) or kept (MXFP8)."""
    rng = np.random.default_rng(8)
    _, _, rt = _routing([40, 70], 18)
    fw, bw = _wgrad_case(rt, rng, lambda r: 1.0, lambda c: 1.0)
    valid = moe.expert_of_rows(rt) >= 0
    for t in (bw.dz, bw.dyp):
        sign = np.sign(t)
        t[valid] = sign[valid] * 1.25       # every routed value is +-1.25
    exp8 = _expected_wgrads(fw, bw)
    got8 = moe.weight_grads(fw, bw, mx=True)
    np.testing.assert_array_equal(got8[0], exp8[0])
    np.testing.assert_array_equal(got8[1], exp8[1])
    # xp and a are +-1 or +-2 (exact in E2M1 with any block maximum of 1 or 2)
    dz4, dy4 = bw.dz.copy(), bw.dyp.copy()
    bw.dz, bw.dyp = np.sign(dz4) * np.minimum(np.abs(dz4), 1.0), np.sign(dy4) * np.minimum(np.abs(dy4), 1.0)
    exp4 = _expected_wgrads(fw, bw)
    bw.dz, bw.dyp = dz4, dy4
    got4 = moe.weight_grads(fw, bw, mx="mxfp4")
    np.testing.assert_array_equal(got4[0], exp4[0])
    np.testing.assert_array_equal(got4[1], exp4[1])
    assert not np.array_equal(got4[0], got8[0])
