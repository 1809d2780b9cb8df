"""Pins of the oracle's expert-block arithmetic.

Checked against things other than the oracle itself:
  * brute-force pure-Python loops on tiny inputs (routing, GEMMs, combine),
  * torch float64 CPU ops for the E=1, k=1, p=1 case (a dense gated MLP),
  * closed forms of the activations,
  * central finite differences of the exact-arithmetic forward for every
    gradient the backward returns (dX, dprobs, and dZ of the activation),
  * invariants: group-size sums, bijective row map, padded starts, identity
    expert, probability linearity, token-order equivariance, empty groups.
"""

import numpy as np
import pytest
import torch

from oracle import moe
from oracle import numerics as nu
from workloads import make_workload

# --------------------------------------------------------------- routing --


def _brute_route(idx, probs, E, first, M_cap, align=128):
    """The per-expert loop: for each expert, scan tokens in order."""
    T, k = idx.shape
    rows = {}
    sizes = []
    for e in range(E):
        members = []
        for t in range(T):
            for s in range(k):
                if idx[t, s] == first + e:
                    members.append((t, s))
        rows[e] = members
        sizes.append(len(members))
    padded = [0]
    for n in sizes:
        padded.append(padded[-1] + ((n + align - 1) // align) * align)
    rmap = [[-1] * k for _ in range(T)]
    src = [-1] * M_cap
    pp = [0.0] * M_cap
    for e in range(E):
        for i, (t, s) in enumerate(rows[e]):
            r = padded[e] + i
            rmap[t][s] = r
            src[r] = t
            pp[r] = float(probs[t, s])
    return sizes, padded, rmap, src, pp


@pytest.mark.parametrize("first,E,k,T", [(0, 4, 2, 37), (2, 3, 3, 50),
                                         (0, 8, 1, 300), (5, 2, 4, 20)])
def test_route_matches_brute_force(first, E, k, T):
    rng = np.random.default_rng(T)
    Et = first + E + 2                      # some ids are not local
    idx = np.stack([rng.permutation(Et)[:k] for _ in range(T)]).astype(
        np.int32)
    probs = rng.random((T, k)).astype(np.float32)
    M_cap = T * k + E * 127 + 5
    rt = moe.route(idx, probs, E, first, M_cap)
    sizes, padded, rmap, src, pp = _brute_route(idx, probs, E, first, M_cap)
    np.testing.assert_array_equal(rt.split_sizes, sizes)
    np.testing.assert_array_equal(rt.padded_offsets, padded)
    np.testing.assert_array_equal(rt.offsets, np.concatenate(
        [[0], np.cumsum(sizes)]))
    np.testing.assert_array_equal(rt.row_id_map, np.array(rmap))
    np.testing.assert_array_equal(rt.row_src, np.array(src))
    np.testing.assert_array_equal(rt.probs_p, np.array(pp, np.float32))


def test_route_invariants_on_config_shapes():
    for name, kw in [("tiny", {}), ("gptoss", dict(T=2048)),
                     ("dsv3", dict(T=4096))]:
        wl = make_workload(name, with_weights=False, with_acts=False, **kw)
        rt = moe.route(wl.expert_idx, wl.probs, wl.E, 0, wl.m_cap())
        assert rt.split_sizes.sum() == wl.T * wl.k     # all experts local
        assert np.all(np.diff(rt.offsets) == rt.split_sizes)
        assert np.all(rt.padded_offsets % 128 == 0)
        assert np.all(np.diff(rt.padded_offsets) >= rt.split_sizes)
        rows = rt.row_id_map.reshape(-1)
        assert np.all(rows >= 0)
        assert len(np.unique(rows)) == rows.size        # injective
        # every valid row maps back to its (t, slot)
        t_of = np.repeat(np.arange(wl.T), wl.k)
        np.testing.assert_array_equal(rt.row_src[rows], t_of)
        assert np.count_nonzero(rt.row_src >= 0) == rows.size
        if name == "dsv3":
            assert rt.split_sizes[0] == 0 and rt.split_sizes[-1] == 0


def test_identity_expert_unpermute_of_permute_is_k_times_x():
    for k in (1, 2, 4, 8):
        T, E, H = 64, 8, 16
        rng = np.random.default_rng(k)
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
        x = nu.round_bf16(rng.standard_normal((T, H)))
        rt = moe.route(idx, np.ones((T, k), np.float32), E, 0, T * k + E * 127)
        out = moe.unpermute(moe.permute(x, rt.row_src), rt.row_id_map)
        np.testing.assert_array_equal(out, k * x)


def test_unpermute_skips_nonlocal_and_sums_in_slot_order():
    yp = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]])
    rmap = np.array([[0, 2], [-1, 1], [-1, -1]], dtype=np.int32)
    out = moe.unpermute(yp, rmap)
    np.testing.assert_array_equal(out, [[101.0, 202.0], [10.0, 20.0],
                                        [0.0, 0.0]])
    dp = np.array([0.5, -1.5, 2.5])
    np.testing.assert_array_equal(moe.gather_probs_grad(dp, rmap),
                                  [[0.5, 2.5], [0.0, -1.5], [0.0, 0.0]])


# ---------------------------------------------------------------- repack --
def test_interleave_rows_small_case_by_hand():
    # I = 4, g = 2: packed = [g0 g1 u0 u1 g2 g3 u2 u3] -> logical rows
    np.testing.assert_array_equal(moe.interleave_rows(4, 2),
                                  [0, 1, 4, 5, 2, 3, 6, 7])


def test_repack_is_a_bijection_and_inverse_undoes_it():
    rng = np.random.default_rng(0)
    w = rng.standard_normal((3, 256, 8))
    wi = moe.repack_interleave(w)
    assert sorted(moe.interleave_rows(128).tolist()) == list(range(256))
    # block structure: packed rows [0,64) gate 0..63, [64,128) up 0..63
    np.testing.assert_array_equal(wi[:, :64], w[:, :64])
    np.testing.assert_array_equal(wi[:, 64:128], w[:, 128:192])
    np.testing.assert_array_equal(wi[:, 128:192], w[:, 64:128])
    np.testing.assert_array_equal(moe.repack_interleave(wi, inverse=True), w)


# ----------------------------------------------------------- activations --
def test_activation_closed_forms():
    assert moe.swish(0.0) == 0.0
    assert moe.swish_grad(0.0) == 0.5
    assert abs(moe.swish(1.0) - 0.7310585786300049) < 1e-15
    assert abs(moe.gelu(1.0) - 0.8413447460685429) < 1e-15
    assert abs(moe.gelu_grad(0.0) - 0.5) < 1e-15
    # Swish_beta(x) = x * sigmoid(beta x): beta=1.702, x=2 by hand
    assert abs(moe.swish(2.0, 1.702) - 2.0 / (1.0 + np.exp(-3.404))) < 1e-15
    # SwiGLU = Swish(gate) * up with gate = first half
    z = np.array([[1.0, -2.0, 3.0, 0.5]])
    s = moe.act_forward(z, moe.ActParams())
    np.testing.assert_allclose(s, [[moe.swish(1.0) * 3.0,
                                    moe.swish(-2.0) * 0.5]], rtol=0, atol=0)
    # clamp +-7 on both halves; linear offset after the clamp
    prm = moe.ActParams.clamped(7.0, beta=1.702)
    prm.lin_offset = 1.0
    z = np.array([[9.0, -8.0]])
    np.testing.assert_allclose(moe.act_forward(z, prm),
                               [[moe.swish(7.0, 1.702) * (-7.0 + 1.0)]])
    assert np.all(moe.act_forward(np.array([[-3.0, 5.0]]),
                                  moe.ActParams(act="srelu")) == [[0, 25]])


@pytest.mark.parametrize("prm", [
    moe.ActParams(),
    moe.ActParams(beta=1.702),
    moe.ActParams(act="geglu"),
    moe.ActParams(act="srelu"),
    moe.ActParams(act="swiglu", beta=1.702, gate_lo=-1.5, gate_hi=1.0,
                  lin_lo=-0.7, lin_hi=2.0, lin_offset=1.0),
])
def test_act_backward_matches_finite_differences(prm):
    rng = np.random.default_rng(1)
    z = rng.standard_normal((5, 16)) * 1.5
    # keep clear of clamp kinks so central differences are valid
    for b in (prm.gate_lo, prm.gate_hi, prm.lin_lo, prm.lin_hi, 0.0):
        z = np.where(np.abs(z - b) < 1e-3, z + 3e-3, z)
    n_out = 8 if prm.gated else 16
    ds = rng.standard_normal((5, n_out))
    g = moe.act_backward(z, ds, prm)
    h = 1e-6
    num = np.zeros_like(z)
    for i in range(z.shape[0]):
        for j in range(z.shape[1]):
            zp, zm = z.copy(), z.copy()
            zp[i, j] += h
            zm[i, j] -= h
            num[i, j] = (np.sum(moe.act_forward(zp, prm) * ds) -
                         np.sum(moe.act_forward(zm, prm) * ds)) / (2 * h)
    np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


# ------------------------------------------------------------ GEMM pins --
def test_fc1_fc2_match_brute_force_loops():
    rng = np.random.default_rng(7)
    T, H, I, E, k = 5, 6, 4, 2, 1
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((E, 2 * I, H))
    w2 = rng.standard_normal((E, H, I))
    idx = np.array([[0], [1], [0], [0], [1]])
    p = rng.random((T, k))
    fw = moe.forward(x, w1, w2, idx, p, E, moe.ActParams(), exact=True)
    for t in range(T):
        e = idx[t, 0]
        r = fw.rt.row_id_map[t, 0]
        z = [sum(x[t, h] * w1[e, n, h] for h in range(H))
             for n in range(2 * I)]
        np.testing.assert_allclose(fw.z[r], z, rtol=1e-13)
        a = [p[t, 0] * z[j] / (1 + np.exp(-z[j])) * z[I + j]
             for j in range(I)]
        np.testing.assert_allclose(fw.a[r], a, rtol=1e-13)
        y = [sum(a[j] * w2[e, h, j] for j in range(I)) for h in range(H)]
        np.testing.assert_allclose(fw.out[t], y, rtol=1e-12, atol=1e-15)


def test_dense_special_case_matches_torch():
    """E=1, k=1, p=1: the layer is a dense gated MLP; compare with torch
    float64 CPU ops (matmul + silu)."""
    rng = np.random.default_rng(2)
    T, H, I = 33, 40, 24
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((1, 2 * I, H)) * 0.2
    w2 = rng.standard_normal((1, H, I)) * 0.2
    dout = rng.standard_normal((T, H))
    idx = np.zeros((T, 1), np.int32)
    p = np.ones((T, 1))
    prm = moe.ActParams()
    fw = moe.forward(x, w1, w2, idx, p, 1, prm, exact=True)
    bw = moe.backward(fw, dout, w1, w2, prm, exact=True)
    xt = torch.tensor(x, requires_grad=True)
    W1 = torch.tensor(w1[0], requires_grad=True)
    W2 = torch.tensor(w2[0], requires_grad=True)
    h = xt @ W1.T
    o = (torch.nn.functional.silu(h[:, :I]) * h[:, I:]) @ W2.T
    (o * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(fw.out, o.detach().numpy(), rtol=1e-12,
                               atol=1e-14)
    np.testing.assert_allclose(bw.dx, xt.grad.numpy(), rtol=1e-12, atol=1e-14)
    dw1, dw2 = moe.weight_grads(fw, bw, exact=True)
    np.testing.assert_allclose(dw1[0], W1.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dw2[0], W2.grad.numpy(), rtol=1e-12, atol=1e-14)


def _loss(x, w1, w2, idx, p, E, prm, dout):
    fw = moe.forward(x, w1, w2, idx, p, E, prm, exact=True)
    return float(np.sum(fw.out * dout))


@pytest.mark.parametrize("prm", [moe.ActParams(),
                                 moe.ActParams(act="geglu"),
                                 moe.ActParams.clamped(0.8, beta=1.702)])
def test_layer_backward_matches_finite_differences(prm):
    rng = np.random.default_rng(4)
    T, H, I, E, k = 6, 5, 4, 3, 2
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((E, 2 * I, H)) * 0.5
    w2 = rng.standard_normal((E, H, I)) * 0.5
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    p = rng.random((T, k))
    dout = rng.standard_normal((T, H))
    fw = moe.forward(x, w1, w2, idx, p, E, prm, exact=True)
    bw = moe.backward(fw, dout, w1, w2, prm, exact=True)
    h = 1e-6
    num_dx = np.zeros_like(x)
    for i in range(T):
        for j in range(H):
            xp_, xm_ = x.copy(), x.copy()
            xp_[i, j] += h
            xm_[i, j] -= h
            num_dx[i, j] = (_loss(xp_, w1, w2, idx, p, E, prm, dout) -
                            _loss(xm_, w1, w2, idx, p, E, prm, dout)) / (2 * h)
    np.testing.assert_allclose(bw.dx, num_dx, rtol=1e-5, atol=1e-8)
    num_dp = np.zeros_like(p)
    for i in range(T):
        for s in range(k):
            pp_, pm_ = p.copy(), p.copy()
            pp_[i, s] += h
            pm_[i, s] -= h
            num_dp[i, s] = (_loss(x, w1, w2, idx, pp_, E, prm, dout) -
                            _loss(x, w1, w2, idx, pm_, E, prm, dout)) / (2 * h)
    np.testing.assert_allclose(bw.dprobs, num_dp, rtol=1e-5, atol=1e-8)


@pytest.mark.parametrize("prm", [moe.ActParams(),
                                 moe.ActParams.clamped(0.8, beta=1.702)])
def test_weight_grads_match_finite_differences(prm):
    """dW1, dW2 against central differences of the float64 layer loss on
    every weight entry; expert 3 gets no rows, so its gradients are 0."""
    rng = np.random.default_rng(6)
    T, H, I, E, k = 7, 5, 4, 4, 2
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((E, 2 * I, H)) * 0.5
    w2 = rng.standard_normal((E, H, I)) * 0.5
    idx = np.stack([rng.permutation(E - 1)[:k] for _ in range(T)])
    p = rng.random((T, k))
    dout = rng.standard_normal((T, H))
    fw = moe.forward(x, w1, w2, idx, p, E, prm, exact=True)
    bw = moe.backward(fw, dout, w1, w2, prm, exact=True)
    dw1, dw2 = moe.weight_grads(fw, bw, exact=True)
    h = 1e-6
    for w, dw, is_w1 in ((w1, dw1, True), (w2, dw2, False)):
        num = np.zeros_like(w)
        for ix in np.ndindex(*w.shape):
            wp_, wm_ = w.copy(), w.copy()
            wp_[ix] += h
            wm_[ix] -= h
            args_p = (wp_, w2) if is_w1 else (w1, wp_)
            args_m = (wm_, w2) if is_w1 else (w1, wm_)
            num[ix] = (_loss(x, *args_p, idx, p, E, prm, dout) -
                       _loss(x, *args_m, idx, p, E, prm, dout)) / (2 * h)
        np.testing.assert_allclose(dw, num, rtol=1e-5, atol=1e-8)
        assert np.all(dw[E - 1] == 0)


def test_prob_linearity_token_equivariance_and_empty_group():
    wl = make_workload("tiny", T=64, H=32, I=64, E=4)
    x = nu.bf16_to_f64(wl.x)
    w1 = nu.bf16_to_f64(wl.w1)
    w2 = nu.bf16_to_f64(wl.w2)
    prm = moe.ActParams()
    p = wl.probs.astype(np.float64)
    f1 = moe.forward(x, w1, w2, wl.expert_idx, p, wl.E, prm, exact=True)
    f2 = moe.forward(x, w1, w2, wl.expert_idx, 2 * p, wl.E, prm, exact=True)
    np.testing.assert_array_equal(f2.out, 2 * f1.out)
    perm = np.random.default_rng(0).permutation(wl.T)
    f3 = moe.forward(x[perm], w1, w2, wl.expert_idx[perm], p[perm], wl.E,
                     prm, exact=True)
    np.testing.assert_allclose(f3.out, f1.out[perm], rtol=1e-12, atol=1e-16)
    # route nobody to expert 2; its weights then cannot matter
    idx = wl.expert_idx.copy()
    idx[idx == 2] = 3
    idx[:, 1] = np.where(idx[:, 0] == idx[:, 1], (idx[:, 1] + 1) % 2,
                         idx[:, 1])
    ga = moe.forward(wl.x, wl.w1, wl.w2, idx, wl.probs, wl.E, prm)
    w1b, w2b = wl.w1.copy(), wl.w2.copy()
    w1b[2] ^= 0x1234
    w2b[2] ^= 0x0F0F
    gb = moe.forward(wl.x, w1b, w2b, idx, wl.probs, wl.E, prm)
    assert ga.rt.split_sizes[2] == 0
    np.testing.assert_array_equal(ga.out, gb.out)


def test_rounded_layer_stores_bf16_values():
    wl = make_workload("tiny")
    prm = moe.ActParams()
    fw = moe.forward(wl.x, wl.w1, wl.w2, wl.expert_idx, wl.probs, wl.E, prm,
                     M_cap=wl.m_cap())
    for t in (fw.z, fw.a, fw.y, fw.out):
        np.testing.assert_array_equal(nu.round_bf16(t), t)
    ex = fw.expert >= 0
    assert fw.amax == np.abs(fw.a[ex]).max()
    assert np.all(fw.a[~ex] == 0) and np.all(fw.xp[~ex] == 0)
    fm = moe.forward(wl.x, wl.w1, wl.w2, wl.expert_idx, wl.probs, wl.E, prm,
                     M_cap=wl.m_cap(), mx=True)
    # MX rounding of operands moves the output by a few percent at most
    err = np.abs(fm.out - fw.out).max() / np.abs(fw.out).max()
    assert 0 < err < 0.1
    c, s = fm.aT_mx
    assert c.shape == (wl.I, int(fm.rt.padded_offsets[-1]))


@pytest.mark.parametrize("act,mx", [("swiglu", False), ("srelu", False), ("swiglu", True)])
def test_sampled_rows_equal_the_full_layer(act, mx):
    """The per-row forward/backward used by the full-size spot checks
    reproduce the full layer's stored rows exactly (same arithmetic on a
    subset of rows)."""
    wl = make_workload("tiny", seed=4, act=act, T=200)
    prm = moe.ActParams.clamped(None, act=act)
    fw = moe.forward(wl.x, wl.w1, wl.w2, wl.expert_idx, wl.probs, wl.E, prm, mx=mx)
    bw = moe.backward(fw, wl.dout, wl.w1, wl.w2, prm)
    x = nu.bf16_to_f64(wl.x)
    dout = nu.bf16_to_f64(wl.dout)
    w1 = nu.bf16_to_f64(wl.w1)
    w2 = nu.bf16_to_f64(wl.w2)
    rng = np.random.default_rng(0)
    for t in rng.choice(wl.T, size=12, replace=False):
        for s in range(wl.k):
            e, r = int(wl.expert_idx[t, s]), int(fw.rt.row_id_map[t, s])
            p = np.array([float(wl.probs[t, s])])
            z, a, y = moe.sample_rows_forward(x[t:t + 1], w1[e], w2[e], p, prm, mx=mx)
            np.testing.assert_array_equal(z[0], fw.z[r])
            np.testing.assert_array_equal(a[0], fw.a[r])
            np.testing.assert_array_equal(y[0], fw.y[r])
            if not mx:
                dz, dxp, dp = moe.sample_rows_backward(dout[t:t + 1], fw.z[r:r + 1], w1[e],
                                                       w2[e], p, prm)
                np.testing.assert_array_equal(dz[0], bw.dz[r])
                np.testing.assert_array_equal(dxp[0], bw.dxp[r])
                assert dp[0] == bw.dp[r]


# ---------------------------------------------------------------- router --
def test_router_matches_brute_force():
    """Pure-Python softmax and a full sort of (-logit, id) per token."""
    import math
    rng = np.random.default_rng(11)
    for T, E, k in ((5, 4, 2), (7, 8, 2), (3, 16, 8), (4, 6, 6)):
        lg = rng.standard_normal((T, E)).astype(np.float32)
        lg[0, 1] = lg[0, 2]                      # a tie: the lower id first
        idx, pr = moe.router_topk(lg, k)
        for t in range(T):
            row = [float(v) for v in lg[t]]
            m = max(row)
            z = sum(math.exp(v - m) for v in row)
            best = sorted(range(E), key=lambda e: (-row[e], e))[:k]
            assert list(idx[t]) == best
            for j, e in enumerate(best):
                assert abs(pr[t, j] - math.exp(row[e] - m) / z) <= 1e-15


def test_router_closed_forms_and_invariants():
    # equal logits: every probability 1/E, ids 0..k-1 (ties to the lower id)
    idx, pr = moe.router_topk(np.full((3, 8), 0.7, np.float32), 2)
    assert np.all(idx == [0, 1]) and np.allclose(pr, 1 / 8, rtol=0, atol=1e-16)
    # k = E keeps the whole softmax: rows sum to 1, descending
    rng = np.random.default_rng(12)
    lg = (rng.standard_normal((50, 16)) * 3).astype(np.float32)
    idx, pr = moe.router_topk(lg, 16)
    assert np.allclose(pr.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(pr, axis=1) <= 0)
    assert all(sorted(r) == list(range(16)) for r in idx)
    # shifting a token's logits by a constant changes nothing
    i2, p2 = moe.router_topk(lg + np.float32(4.0), 16)
    assert np.array_equal(i2, idx) and np.allclose(p2, pr, rtol=1e-6)


def test_unfused_reading_only_moves_rounding_points():
    """The unfused layer differs from the fused one only in where values are
    rounded to bf16: with rounding off both are the same float64 layer, and
    with rounding on the unfused activation equals the fused formula applied
    to the stored z."""
    wl = make_workload("tiny", T=64, H=32, I=64, E=4)
    prm = moe.ActParams()
    f0 = moe.forward(wl.x, wl.w1, wl.w2, wl.expert_idx, wl.probs, wl.E, prm, exact=True)
    f1 = moe.forward(wl.x, wl.w1, wl.w2, wl.expert_idx, wl.probs, wl.E, prm, exact=True,
                     unfused=True)
    b0 = moe.backward(f0, wl.dout, wl.w1, wl.w2, prm, exact=True)
    b1 = moe.backward(f1, wl.dout, wl.w1, wl.w2, prm, exact=True, unfused=True)
    for u, v in ((f0.a, f1.a), (f0.out, f1.out), (b0.dz, b1.dz), (b0.dx, b1.dx),
                 (b0.dprobs, b1.dprobs)):
        np.testing.assert_array_equal(u, v)
    fr = moe.forward(wl.x, wl.w1, wl.w2, wl.expert_idx, wl.probs, wl.E, prm, unfused=True)
    v = fr.expert >= 0
    pp = fr.rt.probs_p.astype(np.float64)[v, None]
    expect = nu.round_bf16(pp * moe.act_forward(fr.z[v], prm))
    np.testing.assert_array_equal(fr.a[v], expect)


def _mxfp4_exact_layer():
    """A layer on which MXFP4 rounds nothing: one-hot tokens and dOut,
    weights in {-1, 0, 1} and probabilities 1/2 with sReLU, so every GEMM
    operand (x, W1, a = p z+^2 in {0, 1/2}, W2, dOut, dZ in {0, +-1}) is an
    exact E2M1 value times a power of two in every 32-block."""
    rng = np.random.default_rng(3)
    E, k, T, H, I = 4, 2, 96, 64, 64
    x = np.zeros((T, H))
    x[np.arange(T), rng.integers(0, H, T)] = 1.0
    dout = np.zeros((T, H))
    dout[np.arange(T), rng.integers(0, H, T)] = 1.0
    w1 = rng.integers(-1, 2, (E, I, H)).astype(np.float64)
    w2 = rng.integers(-1, 2, (E, H, I)).astype(np.float64)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    probs = np.full((T, k), 0.5, np.float32)
    bits = [nu.f64_to_bf16_bits(v) for v in (x, w1, w2, dout)]
    return bits, idx, probs, E


def test_mxfp4_reading_is_exact_on_representable_data():
    (x, w1, w2, dout), idx, probs, E = _mxfp4_exact_layer()
    prm = moe.ActParams(act="srelu")
    kw = dict(unfused=True)
    fb = moe.forward(x, w1, w2, idx, probs, E, prm, **kw)
    f4 = moe.forward(x, w1, w2, idx, probs, E, prm, mx="mxfp4", **kw)
    bb = moe.backward(fb, dout, w1, w2, prm, **kw)
    b4 = moe.backward(f4, dout, w1, w2, prm, mx="mxfp4", **kw)
    assert np.abs(fb.out).max() > 0 and np.abs(bb.dx).max() > 0
    for u, v in ((fb.z, f4.z), (fb.a, f4.a), (fb.out, f4.out), (bb.dz, b4.dz),
                 (bb.dx, b4.dx), (bb.dprobs, b4.dprobs)):
        np.testing.assert_array_equal(u, v)


def test_mxfp4_reading_rounds_every_gemm_operand():
    """On random data each operand's MXFP4 rounding moves the results, more
    than MXFP8's does; forward and backward both see it."""
    wl = make_workload("tiny", seed=8)
    prm = moe.ActParams()
    f16 = moe.forward(wl.x, wl.w1, wl.w2, wl.expert_idx, wl.probs, wl.E, prm)
    f8 = moe.forward(wl.x, wl.w1, wl.w2, wl.expert_idx, wl.probs, wl.E, prm, mx=True)
    f4 = moe.forward(wl.x, wl.w1, wl.w2, wl.expert_idx, wl.probs, wl.E, prm, mx="mxfp4")
    b16 = moe.backward(f16, wl.dout, wl.w1, wl.w2, prm)
    b8 = moe.backward(f8, wl.dout, wl.w1, wl.w2, prm, mx=True)
    b4 = moe.backward(f4, wl.dout, wl.w1, wl.w2, prm, mx="mxfp4")

    def rel(u, v):
        return np.linalg.norm(u - v) / np.linalg.norm(v)
    for q8, q4, ref in ((f8.z, f4.z, f16.z), (f8.out, f4.out, f16.out),
                        (b8.dz, b4.dz, b16.dz), (b8.dx, b4.dx, b16.dx)):
        assert 0 < rel(q8, ref) < rel(q4, ref) < 0.5
    assert f4.a_mx is None and b4.dz_mx is None


# ------------------------------------------------------------ FC1 bias ----
def _augment(x, w1, w2, dout, bias):
    """The bias as one more input column: x' = [x, 1], W1'_e = [W1_e, b_e],
    so x' . W1'_e^T = x . W1_e^T + b_e exactly (float64).  The layer's
    output width follows its input width, so W2 gets a zero output row and
    dOut a zero column: the first H output columns are the original ones."""
    T = x.shape[0]
    xa = np.concatenate([x, np.ones((T, 1))], axis=1)
    w1a = np.concatenate([w1, bias[:, :, None]], axis=2)
    w2a = np.concatenate([w2, np.zeros((w2.shape[0], 1, w2.shape[2]))], axis=1)
    da = np.concatenate([dout, np.zeros((T, 1))], axis=1)
    return xa, w1a, w2a, da


@pytest.mark.parametrize("prm", [moe.ActParams(),
                                 moe.ActParams(act="geglu"),
                                 moe.ActParams.clamped(0.8, beta=1.702),
                                 moe.ActParams(act="srelu")])
def test_bias_is_an_activation_input_offset(prm):
    """FC1 bias (one vector per expert, logical gate|up order): the layer
    with bias b equals the bias-free layer with b as the weight of an extra
    all-ones input column, except that z is stored without b.  Pins where b
    enters (the activation's input, both halves in logical order, per
    expert) and that the backward's dz, dprobs and dx see the same offset."""
    rng = np.random.default_rng(11)
    T, H, I, E, k = 7, 5, 4, 3, 2
    n1 = 2 * I if prm.gated else I
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((E, n1, H)) * 0.5
    w2 = rng.standard_normal((E, H, I)) * 0.5
    bias = rng.standard_normal((E, n1))
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    p = rng.random((T, k))
    dout = rng.standard_normal((T, H))
    fb = moe.forward(x, w1, w2, idx, p, E, prm, exact=True, bias1=bias)
    xa, w1a, w2a, da = _augment(x, w1, w2, dout, bias)
    fa = moe.forward(xa, w1a, w2a, idx, p, E, prm, exact=True)
    valid = fb.expert >= 0
    ex = fb.expert[valid]
    np.testing.assert_allclose(fb.z[valid] + bias[ex], fa.z[valid], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(fb.a[valid], fa.a[valid], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fb.out, fa.out[:, :H], rtol=1e-12, atol=1e-14)
    assert not fa.out[:, H].any()
    bb = moe.backward(fb, dout, w1, w2, prm, exact=True, bias1=bias)
    ba = moe.backward(fa, da, w1a, w2a, prm, exact=True)
    np.testing.assert_allclose(bb.dz[valid], ba.dz[valid], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(bb.dprobs, ba.dprobs, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(bb.dx, ba.dx[:, :H], rtol=1e-12, atol=1e-14)
    # a wrong reading is caught: the bias on the other half, or stored in z
    if prm.gated:
        swapped = np.concatenate([bias[:, I:], bias[:, :I]], axis=1)
        fs = moe.forward(x, w1, w2, idx, p, E, prm, exact=True, bias1=swapped)
        assert np.abs(fs.a[valid] - fa.a[valid]).max() > 1e-3
    assert np.abs(fb.z[valid] - fa.z[valid]).max() > 1e-3


def test_bias_gradient_is_the_sum_of_dz_over_the_expert_rows():
    """dL/db_e = sum of dz over expert e's rows (central differences of the
    float64 layer loss), the reading the C ABI documents for dz."""
    rng = np.random.default_rng(12)
    T, H, I, E, k = 6, 4, 4, 2, 2
    prm = moe.ActParams.clamped(1.5, beta=1.702)
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((E, 2 * I, H)) * 0.5
    w2 = rng.standard_normal((E, H, I)) * 0.5
    bias = rng.standard_normal((E, 2 * I)) * 0.3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    p = rng.random((T, k))
    dout = rng.standard_normal((T, H))

    def loss(b):
        fw = moe.forward(x, w1, w2, idx, p, E, prm, exact=True, bias1=b)
        return float(np.sum(fw.out * dout))

    fw = moe.forward(x, w1, w2, idx, p, E, prm, exact=True, bias1=bias)
    bw = moe.backward(fw, dout, w1, w2, prm, exact=True, bias1=bias)
    h = 1e-6
    for e in range(E):
        rows = fw.expert == e
        db = bw.dz[rows].sum(axis=0)
        for n in range(2 * I):
            bp, bm = bias.copy(), bias.copy()
            bp[e, n] += h
            bm[e, n] -= h
            num = (loss(bp) - loss(bm)) / (2 * h)
            assert abs(db[n] - num) <= 1e-5 * max(1.0, abs(num)), (e, n, db[n], num)
