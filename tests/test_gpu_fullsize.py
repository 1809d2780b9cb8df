"""Parity at the benchmark's full sizes and launch configuration (needs an
MI355X).

The inputs are bench.py's own (bench.device_inputs: routing from the host
generator, activations and weights drawn on the device), the block is built
exactly as bench.py builds it, and one forward + backward step runs.  The
whole-layer oracle is too slow at these sizes, so:
  * routing metadata (split sizes, offsets, row map, row sources, permuted
    probabilities) is compared in full, bit-exact;
  * bf16: every stored tensor of sampled tokens (both of their slots) is
    recomputed one row at a time by the oracle (oracle.moe.sample_rows_*):
    z, a, yp, out, dz, dxp, dprobs_p, dx and dprobs;
  * MXFP8 (Mixtral, GPT-OSS, DSv3 share): the fused MXFP8 copies of a and
    dz, rowwise and transposed, on whole sampled 32-row blocks against the
    oracle's encoder applied to the GPU's own bf16 a and dz (scales
    bit-exact, codes within one E4M3 step on at most 0.1%); the oracle's
    cost is in encoding whole weight matrices, so the values use sampled
    (row, column) outputs that need only the weight rows or columns
    involved: the MXFP8 copy of the permuted input rows (bit-exact), FC1
    outputs z, the activation a, the FC2-dgrad + dActivation output dz, and
    secondarily the MXFP8 copies of the oracle's own a and dz;
  * MXFP4 (Mixtral, GPT-OSS): the fused MXFP4 copies of a and dz, rowwise
    and transposed, on whole sampled 32-row blocks bit-exact against the
    oracle's encoding of the GPU's own bf16 rows; the permuted input rows'
    copy bit-exact; sampled z, a and dz against the oracle on MXFP4 operands;
  * amax equals max |a| over the valid rows (a property at any size);
  * the whole DSv3-share step captured in one HIP graph replays to the eager
    results bit for bit (bf16 and MXFP8).
"""

import numpy as np
import pytest
import torch

import bench
import moe_grouped_mlp_amd as mg
from oracle import moe as om
from oracle import numerics as nu
from workloads.gen import CONFIGS

from .gpu_util import (assert_close, assert_close_mx, assert_mx_equal, assert_mx_near,
                       assert_mx_rule, compare_routing, mx_scale_index, rows_with_pad_zeroed,
                       uninterleave_cols)

pytestmark = pytest.mark.gpu


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    mg.lib()


def _run(name, prec):
    cfg = dict(CONFIGS[name])
    E, k, T, H, I = (cfg[n] for n in ("E", "k", "T", "H", "I"))
    dev = torch.device("cuda")
    print(f"full-size {name} {prec}: generating inputs", flush=True)
    x, dout, w1, w2, idx, probs = bench.device_inputs(cfg, 0, dev)
    kind = {"swiglu": mg.ACT_SWIGLU, "geglu": mg.ACT_GEGLU, "srelu": mg.ACT_SRELU}[cfg["act"]]
    act = mg.act_params(kind, beta=cfg["beta"], clamp=cfg["clamp"])
    # bench.py's block; with MXFP8 the bf16 a and dz are kept for the checks
    # (they do not change what is computed)
    blk = mg.ExpertBlock(E, H, I, T, k, act=act,
                         prec={"bf16": mg.PREC_BF16, "mxfp8": mg.PREC_MXFP8,
                               "mxfp4": mg.PREC_MXFP4}[prec],
                         bf16_copies=True)
    blk.load_weights(w1, w2)
    blk.forward(x, idx, probs)
    blk.backward(dout)
    torch.cuda.synchronize()
    assert int(blk.err_flag.cpu()[0]) == 0
    idx_h, probs_h = idx.cpu().numpy(), probs.cpu().numpy()
    rt = om.route(idx_h, probs_h, E, 0, blk.M_cap)
    compare_routing(blk, rt)
    op = om.ActParams.clamped(cfg["clamp"], beta=cfg["beta"], act=cfg["act"])
    return cfg, blk, (x, dout, w1, w2, idx_h, probs_h), rt, op


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _rows_f64(t, rows):
    return nu.bf16_to_f64(_bits(t[torch.as_tensor(rows, device=t.device)]))


def _amax_property(blk):
    valid = blk.row_src >= 0
    a_max = blk.a[valid].float().abs().max().item()
    assert float(blk.amax.cpu()[0]) == a_max


def _sample_tokens(rt, idx, n, seed):
    """The first and last token, a token routed to the largest group, one
    routed to the smallest non-empty group, and n random tokens."""
    sizes = rt.split_sizes
    live = np.flatnonzero(sizes > 0)
    big, small = int(live[np.argmax(sizes[live])]), int(live[np.argmin(sizes[live])])
    T = idx.shape[0]
    t_big = int(np.flatnonzero(np.any(idx == big, axis=1))[0])
    t_small = int(np.flatnonzero(np.any(idx == small, axis=1))[-1])
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1, t_big, t_small], rng.choice(T, n, replace=False)]))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral", "gptoss", "dsv3"])
def test_full_size_bf16_sampled_tokens(name):
    cfg, blk, (x, dout, w1, w2, idx, probs), rt, op = _run(name, "bf16")
    E, k, I = cfg["E"], cfg["k"], cfg["I"]
    if name == "dsv3":
        assert rt.split_sizes[0] == 0 and rt.split_sizes[-1] == 0
    _amax_property(blk)
    tokens = _sample_tokens(rt, idx, 4 if name == "mixtral" else 8, seed=len(name))
    chosen = np.unique(idx[tokens])
    print(f"checking {len(tokens)} tokens on experts {chosen.tolist()}", flush=True)
    x_h = nu.bf16_to_f64(_bits(x[torch.as_tensor(tokens, device=x.device)]))
    d_h = nu.bf16_to_f64(_bits(dout[torch.as_tensor(tokens, device=x.device)]))
    res = {}
    for e in chosen.tolist():
        sel = [(i, s) for i, t in enumerate(tokens) for s in range(k) if idx[t, s] == e]
        if not sel:
            continue
        w1e = nu.bf16_to_f64(_bits(w1[e]))
        w2e = nu.bf16_to_f64(_bits(w2[e]))
        xi = np.stack([x_h[i] for i, _ in sel])
        di = np.stack([d_h[i] for i, _ in sel])
        p = np.array([float(probs[tokens[i], s]) for i, s in sel])
        z, a, y = om.sample_rows_forward(xi, w1e, w2e, p, op)
        dz, dxp, dp = om.sample_rows_backward(di, z, w1e, w2e, p, op)
        for n_, (i, s) in enumerate(sel):
            res[(i, s)] = (z[n_], a[n_], y[n_], dz[n_], dxp[n_], dp[n_])
        del w1e, w2e
    keys = sorted(res)
    rows = [int(rt.row_id_map[tokens[i], s]) for i, s in keys]
    z_g = nu.bf16_to_f64(_bits(blk.z[torch.as_tensor(rows, device="cuda")]))
    if cfg["act"] != "srelu":
        z_g = uninterleave_cols(z_g, I)
    dz_g = nu.bf16_to_f64(_bits(blk.dz[torch.as_tensor(rows, device="cuda")]))
    if cfg["act"] != "srelu":
        dz_g = uninterleave_cols(dz_g, I)
    assert_close(z_g, np.stack([res[kk][0] for kk in keys]), "z rows")
    assert_close(_rows_f64(blk.a, rows), np.stack([res[kk][1] for kk in keys]), "a rows")
    assert_close(_rows_f64(blk.yp, rows), np.stack([res[kk][2] for kk in keys]), "yp rows")
    assert_close(dz_g, np.stack([res[kk][3] for kk in keys]), "dz rows")
    assert_close(_rows_f64(blk.dxp, rows), np.stack([res[kk][4] for kk in keys]), "dxp rows")
    dpp = blk.dprobs_p[torch.as_tensor(rows, device="cuda")].cpu().numpy().astype(np.float64)
    assert_close(dpp, np.array([res[kk][5] for kk in keys]), "dprobs_p rows")
    # combined outputs of the sampled tokens (all their slots were computed)
    out_ref = np.stack([om.round_bf16(sum(res[(i, s)][2] for s in range(k)))
                        for i in range(len(tokens))])
    dx_ref = np.stack([om.round_bf16(sum(res[(i, s)][4] for s in range(k)))
                       for i in range(len(tokens))])
    assert_close(_rows_f64(blk.out, tokens), out_ref, "out tokens")
    assert_close(_rows_f64(blk.dx, tokens), dx_ref, "dx tokens")
    dpr = blk.dprobs.cpu().numpy()[tokens].astype(np.float64)
    assert_close(dpr, np.array([[res[(i, s)][5] for s in range(k)] for i in range(len(tokens))]),
                 "dprobs tokens")


def _sample_row_blocks(rt, n, seed):
    """32-row blocks of the padded layout to check whole: the first block of
    the largest group, the last (partial) block of the smallest non-empty
    group, and n random blocks that hold data."""
    sizes, pad = rt.split_sizes, rt.padded_offsets
    live = np.flatnonzero(sizes > 0)
    big, small = int(live[np.argmax(sizes[live])]), int(live[np.argmin(sizes[live])])
    blocks = {int(pad[big]) // 32, (int(pad[small]) + int(sizes[small]) - 1) // 32}
    data_blocks = np.unique(np.flatnonzero(rt.row_src >= 0) // 32)
    rng = np.random.default_rng(seed)
    blocks.update(int(b) for b in rng.choice(data_blocks, size=n, replace=False))
    return sorted(blocks)


def _self_consistent_copies(blk, rt, prefix, bf16_t, n, blocks, what):
    """The parity rule on sampled 32-row blocks: the fused MXFP8 copies
    (rowwise along n, transposed along M) against the oracle's encoder
    applied to the GPU's own bf16 rows, pad rows as zeros."""
    M_cap = blk.M_cap
    valid = rt.row_src >= 0
    sidx = mx_scale_index(M_cap, n)
    q, sc = getattr(blk, prefix + "_q"), getattr(blk, prefix + "_s").cpu().numpy()
    qT, sT = getattr(blk, prefix + "T_q"), getattr(blk, prefix + "T_s").cpu().numpy()
    sidx_t = mx_scale_index(n, M_cap)
    for b in blocks:
        r = np.arange(32 * b, 32 * b + 32)
        rt_rows = torch.as_tensor(r, device="cuda")
        v = rows_with_pad_zeroed(nu.bf16_to_f64(_bits(bf16_t[rt_rows])), valid[r])
        assert_mx_rule(q[rt_rows].cpu().numpy(), sc[sidx[r]], nu.mx_quantize(v, axis=1),
                       f"{what} MX rowwise rows {32 * b}..")
        assert_mx_rule(qT[:, 32 * b:32 * b + 32].cpu().numpy(), sT[sidx_t[:, b:b + 1]],
                       nu.mx_quantize(v.T, axis=1), f"{what} MX transposed rows {32 * b}..")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral_mx", "gptoss", "dsv3"])
def test_full_size_mx_sampled(name):
    """MXFP8 at the full Mixtral, GPT-OSS (128 experts, clamped SwiGLU with
    slope 1.702, H = I = 2880) and DSv3-share (Zipf groups, empty ones)
    sizes, bench.py's launch configuration."""
    cfg, blk, (x, dout, w1, w2, idx, probs), rt, op = _run(name, "mxfp8")
    E, k, H, I = cfg["E"], cfg["k"], cfg["H"], cfg["I"]
    M_cap = blk.M_cap
    _amax_property(blk)
    # the fused copies of a and dz, whole sampled row blocks: parity rule
    blocks = _sample_row_blocks(rt, 6, seed=len(name))
    print(f"checking the MXFP8 copies of a and dz on row blocks {blocks}", flush=True)
    _self_consistent_copies(blk, rt, "a", blk.a, I, blocks, "a")
    _self_consistent_copies(blk, rt, "dz", blk.dz, 2 * I, blocks, "dz")
    rng = np.random.default_rng(11)
    valid_rows = np.flatnonzero(rt.row_src >= 0)
    rows = np.sort(rng.choice(valid_rows, size=16, replace=False))
    blocks = np.sort(rng.choice(I // 32, size=2, replace=False))   # 32-column blocks of a
    cols = np.concatenate([32 * b + np.arange(32) for b in blocks])
    expert = om.expert_of_rows(rt)
    packed = np.argsort(om.interleave_rows(I))   # packed position of each logical column
    sidx_x = mx_scale_index(M_cap, H)
    sidx_a = mx_scale_index(M_cap, I)
    sidx_dz = mx_scale_index(M_cap, 2 * I)
    xq_g = blk.xp_q.cpu().numpy()
    xs_g = blk.xp_s.cpu().numpy()
    z_g = nu.bf16_to_f64(_bits(blk.z[torch.as_tensor(rows, device="cuda")]))
    a_g = nu.bf16_to_f64(_bits(blk.a[torch.as_tensor(rows, device="cuda")]))
    dz_g = nu.bf16_to_f64(_bits(blk.dz[torch.as_tensor(rows, device="cuda")]))
    aq_g = blk.a_q[torch.as_tensor(rows, device="cuda")].cpu().numpy()
    as_g = blk.a_s.cpu().numpy()
    dzq_g = blk.dz_q[torch.as_tensor(rows, device="cuda")].cpu().numpy()
    dzs_g = blk.dz_s.cpu().numpy()
    z_ref, z_got, a_ref, a_got, dz_ref, dz_got = [], [], [], [], [], []
    mx_checks = []   # run after the value checks, which localise a problem better
    for n_, r in enumerate(rows):
        t, e = int(rt.row_src[r]), int(expert[r])
        p = float(rt.probs_p[r])
        xr = nu.bf16_to_f64(_bits(x[t]))
        # permuted input row, MXFP8 along H: bit-exact
        assert_mx_equal(xq_g[r], xs_g[sidx_x[r]], nu.mx_quantize(xr[None, :], axis=1),
                        f"xp MX row {r}")
        xq = nu.mx_round(xr[None, :], axis=1)[0]
        w1e = w1[e]
        g_rows = nu.mx_round(nu.bf16_to_f64(_bits(w1e[torch.as_tensor(cols, device="cuda")])), 1)
        u_rows = nu.mx_round(nu.bf16_to_f64(_bits(w1e[torch.as_tensor(I + cols, device="cuda")])), 1)
        zg, zu = g_rows @ xq, u_rows @ xq
        z_ref += [om.round_bf16(zg), om.round_bf16(zu)]
        z_got += [z_g[n_][packed[cols]], z_g[n_][packed[I + cols]]]
        s_half = om.act_forward(np.concatenate([zg, zu])[None, :], op)[0]
        a_cols = om.round_bf16(p * s_half)
        a_ref.append(a_cols)
        a_got.append(a_g[n_][cols])
        # the fused MXFP8 copy of a on the sampled blocks (secondary: the
        # oracle's encoding of its own a)
        for bi, b in enumerate(blocks):
            ref = nu.mx_quantize(a_cols[None, 32 * bi:32 * bi + 32], axis=1)
            mx_checks.append((aq_g[n_][32 * b:32 * b + 32][None, :],
                              as_g[sidx_a[r, b:b + 1]][None, :], ref, f"a MX row {r} block {b}"))
        # FC2 dgrad + dActivation on the same columns: dA needs the columns
        # of W2 (along H) and the quantized dOut row
        dr = nu.bf16_to_f64(_bits(dout[t]))
        dq = nu.mx_round(dr[None, :], axis=1)[0]
        w2c = nu.bf16_to_f64(_bits(w2[e][:, torch.as_tensor(cols, device="cuda")].contiguous()))
        da = dq @ nu.mx_round(w2c, axis=0)
        zs = np.concatenate([om.round_bf16(zg), om.round_bf16(zu)])[None, :]
        d = om.act_backward(zs, p * da[None, :], op)[0]
        dzc = om.round_bf16(d)
        dz_ref.append(dzc)
        dz_got.append(np.concatenate([dz_g[n_][packed[cols]], dz_g[n_][packed[I + cols]]]))
        for bi, b in enumerate(blocks):
            for half, off in ((0, 0), (1, I)):
                pk = packed[off + 32 * b]          # first packed column of the block
                ref = nu.mx_quantize(dzc[None, half * len(cols) + 32 * bi:
                                          half * len(cols) + 32 * bi + 32], axis=1)
                mx_checks.append((dzq_g[n_][pk:pk + 32][None, :],
                                  dzs_g[sidx_dz[r, pk // 32:pk // 32 + 1]][None, :], ref,
                                  f"dz MX row {r} block {pk // 32} (gpu dz "
                                  f"{dz_g[n_][pk:pk + 4]} oracle {dzc[half * len(cols) + 32 * bi:][:4]})"))
    assert_close_mx(np.concatenate(z_got), np.concatenate(z_ref), "z samples")
    assert_close_mx(np.concatenate(a_got), np.concatenate(a_ref), "a samples")
    assert_close_mx(np.concatenate(dz_got), np.concatenate(dz_ref), "dz samples")
    # secondary, against the oracle's own values (which differ from the
    # GPU's bf16 a and dz by the GEMMs' rounding): scales at most one binade
    # apart on at most a quarter of the sampled blocks, codes as in the
    # multi-tile layer tests where the scales agree
    for q, sc, ref, what in mx_checks:
        assert_mx_near(q, sc, ref, what, code_frac=0.05, far_frac=0.01, scale_frac=1.0)
    n_scale = sum(int(np.any(sc != ref[1])) for q, sc, ref, what in mx_checks)
    assert n_scale <= len(mx_checks) // 4, f"{n_scale} of {len(mx_checks)} block scales differ"


def _unpack4(b):
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def _mx4_copies_exact(blk, rt, prefix, bf16_t, n, blocks, what):
    """The fused MXFP4 copies (rowwise along n, transposed along M) of whole
    sampled 32-row blocks against the oracle's MXFP4 encoding of the GPU's
    own bf16 rows (pad rows as zeros), bit for bit."""
    M_cap = blk.M_cap
    valid = rt.row_src >= 0
    sidx = mx_scale_index(M_cap, n)
    sidx_t = mx_scale_index(n, M_cap)
    q = getattr(blk, prefix + "_q4").view(M_cap, n // 2)
    sc = getattr(blk, prefix + "_s4").cpu().numpy()
    qT = getattr(blk, prefix + "T_q4").view(n, M_cap // 2)
    sT = getattr(blk, prefix + "T_s4").cpu().numpy()
    for b in blocks:
        r = np.arange(32 * b, 32 * b + 32)
        rows = torch.as_tensor(r, device="cuda")
        v = rows_with_pad_zeroed(nu.bf16_to_f64(_bits(bf16_t[rows])), valid[r])
        codes, scales = nu.mxfp4_quantize(v, axis=1)
        np.testing.assert_array_equal(sc[sidx[r]], scales, err_msg=f"{what} rowwise scales {b}")
        np.testing.assert_array_equal(q[rows].cpu().numpy(), nu.pack_nibbles(codes),
                                      err_msg=f"{what} rowwise codes {b}")
        codes, scales = nu.mxfp4_quantize(v.T, axis=1)
        np.testing.assert_array_equal(sT[sidx_t[:, b:b + 1]], scales,
                                      err_msg=f"{what} transposed scales {b}")
        np.testing.assert_array_equal(qT[:, 16 * b:16 * b + 16].cpu().numpy(),
                                      nu.pack_nibbles(codes), err_msg=f"{what} transposed codes {b}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral", "gptoss"])
def test_full_size_mxfp4_sampled(name):
    """The fused MXFP4 layer at the full Mixtral and GPT-OSS sizes: routing
    in full; the MXFP4 copies of a and dz (rowwise and transposed) on whole
    sampled 32-row blocks, bit-exact against the oracle's encoding of the
    GPU's own bf16 rows; the permuted input rows' MXFP4 copy bit-exact; and
    sampled (row, column) outputs z, a and dz against the oracle on MXFP4
    operands (the weight rows or columns involved, encoded along their K)."""
    cfg, blk, (x, dout, w1, w2, idx, probs), rt, op = _run(name, "mxfp4")
    H, I = cfg["H"], cfg["I"]
    M_cap = blk.M_cap
    _amax_property(blk)
    blocks = _sample_row_blocks(rt, 6, seed=3 + len(name))
    print(f"checking the MXFP4 copies of a and dz on row blocks {blocks}", flush=True)
    _mx4_copies_exact(blk, rt, "a", blk.a, I, blocks, "a")
    _mx4_copies_exact(blk, rt, "dz", blk.dz, 2 * I, blocks, "dz")
    rng = np.random.default_rng(12)
    valid_rows = np.flatnonzero(rt.row_src >= 0)
    rows = np.sort(rng.choice(valid_rows, size=12, replace=False))
    cblocks = np.sort(rng.choice(I // 32, size=2, replace=False))
    cols = np.concatenate([32 * b + np.arange(32) for b in cblocks])
    expert = om.expert_of_rows(rt)
    packed = np.argsort(om.interleave_rows(I))
    sidx_x = mx_scale_index(M_cap, H)
    xq_g = blk.xp_q4.view(M_cap, H // 2)[torch.as_tensor(rows, device="cuda")].cpu().numpy()
    xs_g = blk.xp_s4.cpu().numpy()
    sel = torch.as_tensor(rows, device="cuda")
    z_g = nu.bf16_to_f64(_bits(blk.z[sel]))
    a_g = nu.bf16_to_f64(_bits(blk.a[sel]))
    dz_g = nu.bf16_to_f64(_bits(blk.dz[sel]))
    z_ref, z_got, a_ref, a_got, dz_ref, dz_got = [], [], [], [], [], []
    for n_, r in enumerate(rows):
        t, e = int(rt.row_src[r]), int(expert[r])
        p = float(rt.probs_p[r])
        xr = nu.bf16_to_f64(_bits(x[t]))
        codes, scales = nu.mxfp4_quantize(xr[None, :], axis=1)
        np.testing.assert_array_equal(xq_g[n_], nu.pack_nibbles(codes)[0], err_msg=f"xp row {r}")
        np.testing.assert_array_equal(xs_g[sidx_x[r]], scales[0], err_msg=f"xp scales row {r}")
        xq = nu.mxfp4_round(xr[None, :], axis=1)[0]
        w1e = w1[e]
        g_rows = nu.mxfp4_round(nu.bf16_to_f64(_bits(w1e[torch.as_tensor(cols, device="cuda")])), 1)
        u_rows = nu.mxfp4_round(nu.bf16_to_f64(_bits(w1e[torch.as_tensor(I + cols, device="cuda")])), 1)
        zg, zu = g_rows @ xq, u_rows @ xq
        z_ref += [om.round_bf16(zg), om.round_bf16(zu)]
        z_got += [z_g[n_][packed[cols]], z_g[n_][packed[I + cols]]]
        s_half = om.act_forward(np.concatenate([zg, zu])[None, :], op)[0]
        a_ref.append(om.round_bf16(p * s_half))
        a_got.append(a_g[n_][cols])
        dr = nu.bf16_to_f64(_bits(dout[t]))
        dq = nu.mxfp4_round(dr[None, :], axis=1)[0]
        w2c = nu.bf16_to_f64(_bits(w2[e][:, torch.as_tensor(cols, device="cuda")].contiguous()))
        da = dq @ nu.mxfp4_round(w2c, axis=0)
        zs = np.concatenate([om.round_bf16(zg), om.round_bf16(zu)])[None, :]
        dz_ref.append(om.round_bf16(om.act_backward(zs, p * da[None, :], op)[0]))
        dz_got.append(np.concatenate([dz_g[n_][packed[cols]], dz_g[n_][packed[I + cols]]]))
    assert_close_mx(np.concatenate(z_got), np.concatenate(z_ref), "z samples")
    assert_close_mx(np.concatenate(a_got), np.concatenate(a_ref), "a samples")
    assert_close_mx(np.concatenate(dz_got), np.concatenate(dz_ref), "dz samples")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
def test_dsv3_graph_replays_match_eager(prec):
    """The whole DSv3-share step (32 local experts, Zipf groups with empty
    ones, H = 7168, I = 2048) captured in one HIP graph in global mode and
    replayed three times, outputs cleared before each replay: every replay
    reproduces the eager step bit for bit (routed rows of the per-row
    tensors, the whole of out, dX and dprobs)."""
    cfg = dict(CONFIGS["dsv3"])
    E, k, T, H, I = (cfg[n] for n in ("E", "k", "T", "H", "I"))
    print(f"graph replay, dsv3 share {prec}: generating inputs", flush=True)
    x, dout, w1, w2, idx, probs = bench.device_inputs(cfg, 0, torch.device("cuda"))
    blk = mg.ExpertBlock(E, H, I, T, k, act=mg.act_params(mg.ACT_SWIGLU),
                         prec=mg.PREC_MXFP8 if prec == "mxfp8" else mg.PREC_BF16)
    blk.load_weights(w1, w2)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        blk.forward(x, idx, probs)
        blk.backward(dout)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert int(blk.err_flag.cpu()[0]) == 0
    rows = blk.row_src >= 0
    per_row = ([blk.z, blk.yp, blk.dxp] +
               ([blk.a, blk.dz] if prec == "bf16" else [blk.a_q, blk.dz_q]))
    whole = [blk.out, blk.dx, blk.dprobs]
    eager_rows = [t[rows].clone() for t in per_row]
    eager_whole = [t.clone() for t in whole]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="global"):
        blk.forward(x, idx, probs)
        blk.backward(dout)
    for rep in range(3):
        for t in per_row + whole:
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"replay {rep} done", flush=True)
        for i, (t, e) in enumerate(zip(per_row, eager_rows)):
            assert torch.equal(t[rows], e), f"per-row output {i} differs on replay {rep}"
        for i, (t, e) in enumerate(zip(whole, eager_whole)):
            assert torch.equal(t, e), f"output {i} differs on replay {rep}"
    del g
