"""GPU parity of the MXFP8 path against the CPU oracle (needs an MI355X).

* moe_quantize_mxfp8 and the MXFP8 output of moe_permute: codes and scales
  bit-exact against oracle.numerics.mx_quantize of the same bf16 values.
* Layers on sparse integer data (sReLU, and SwiGLU with slope 0, where the
  gate's sigmoid is exactly 1/2): every GEMM and epilogue value is then exact
  on both sides, so z, a, dz, dprobs_p and the four MXFP8 copies the fused
  epilogues write (a and dz, rowwise and transposed) must equal the oracle's
  bit for bit.
* Layers on the configs' random data: outputs against the fp64 oracle fed the
  same MXFP8 operands; the fused MXFP8 copies of a and dz (rowwise and
  transposed) against the oracle's encoder applied to the GPU's own bf16 a
  and dz (scales bit-exact, codes within one E4M3 step on at most 0.1%),
  and secondarily against the oracle's encoding of its own values, to the
  bounds explained in gpu_util (the fp8 MFMA's internal rounding moves a
  few values across E4M3 rounding boundaries).
Every call goes through the C ABI.
"""

import numpy as np
import pytest
import torch

import moe_grouped_mlp_amd as mg
from oracle import moe as om
from oracle import numerics as nu
from workloads import make_workload

from .gpu_util import (act_of, assert_close, assert_close_mx, assert_fused_mx_copies,
                       assert_mx_equal, assert_mx_near, compare_routing, dev_bf16, gemm_grid,
                       host_bits, host_f64, mx_scales_plain, oracle_layer,
                       run_gpu_layer, tail_split_parts, uninterleave_cols)

pytestmark = pytest.mark.gpu


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    mg.lib()


def _hard_bf16(rng, shape):
    """bf16 values over many binades with zero blocks, bf16 subnormals,
    values near the bf16 maximum and (naturally) saturating blocks."""
    x = rng.standard_normal(shape) * np.exp2(
        rng.integers(-60, 60, size=shape[:-1] + (1,)).astype(np.float64))
    x[..., ::7, :32] = 0.0
    x[..., 3, :] *= 2.0 ** -128                 # bf16 subnormals and zeros
    x[..., 5, 32:64] = np.sign(x[..., 5, 32:64]) * 3.0e38
    x[..., 6, 64:96] = -0.0
    return nu.f64_to_bf16_bits(nu.round_bf16(x))


@pytest.mark.parametrize("mode", [mg.QUANT_ROW, mg.QUANT_COL])
@pytest.mark.parametrize("batch,rows,cols,pad", [(1, 64, 64, 0), (3, 128, 192, 0),
                                                 (2, 192, 2880, 40)])
def test_quantize_bit_exact(mode, batch, rows, cols, pad):
    rng = np.random.default_rng(rows + cols + mode)
    bits = _hard_bf16(rng, (batch, rows, cols))
    stride = rows * cols + pad
    flat = np.zeros(batch * stride, np.uint16)
    for b in range(batch):
        flat[b * stride:b * stride + rows * cols] = bits[b].reshape(-1)
    x = dev_bf16(flat)
    q = torch.full((batch * rows * cols,), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((batch * rows * cols // 32,), 0xAB, dtype=torch.uint8, device="cuda")
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    mg.moe_quantize_mxfp8(mode=mode, batch=batch, rows=rows, cols=cols, x=x, q=q,
                          s=s, x_stride=stride if pad else 0, amax=amax)
    torch.cuda.synchronize()
    v = nu.bf16_to_f64(bits)
    qh = q.cpu().numpy().reshape(batch, -1)
    sh = s.cpu().numpy().reshape(batch, -1)
    for b in range(batch):
        if mode == mg.QUANT_ROW:
            ref = nu.mx_quantize(v[b], axis=1)
            R, K = rows, cols
        else:
            ref = nu.mx_quantize(v[b].T, axis=1)
            R, K = cols, rows
        s_plain = mx_scales_plain(torch.from_numpy(sh[b]), R, K)
        assert_mx_equal(qh[b].reshape(R, K), s_plain, ref, f"quantize mode {mode} batch {b}")
    assert float(amax.cpu()[0]) == np.abs(v).max()


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("batch,rows,cols,pad", [(1, 64, 64, 0), (3, 128, 192, 0),
                                                 (2, 192, 2880, 40)])
def test_quantize_both_copies_in_one_pass(fmt, batch, rows, cols, pad):
    """MOE_QUANT_BOTH writes the ROW copy to q / s and the COL copy to qT /
    sT in one pass: each bit-exact against the oracle's encoding along its
    axis (and so equal to the one-copy modes)."""
    rng = np.random.default_rng(rows + cols + 17)
    bits = _hard_bf16(rng, (batch, rows, cols))
    stride = rows * cols + pad
    flat = np.zeros(batch * stride, np.uint16)
    for b in range(batch):
        flat[b * stride:b * stride + rows * cols] = bits[b].reshape(-1)
    x = dev_bf16(flat)
    nq = batch * rows * cols // (2 if fmt == "mxfp4" else 1)
    q, qT = (torch.full((nq,), 0xAB, dtype=torch.uint8, device="cuda") for _ in range(2))
    s, sT = (torch.full((batch * rows * cols // 32,), 0xAB, dtype=torch.uint8, device="cuda")
             for _ in range(2))
    kw = dict(mode=mg.QUANT_BOTH, batch=batch, rows=rows, cols=cols, x=x, q=q, s=s, qT=qT, sT=sT,
              x_stride=stride if pad else 0)
    if fmt == "mxfp8":
        amax = torch.zeros(1, dtype=torch.float32, device="cuda")
        mg.moe_quantize_mxfp8(amax=amax, **kw)
    else:
        mg.moe_quantize_mxfp4(**kw)
    torch.cuda.synchronize()
    v = nu.bf16_to_f64(bits)
    for qq, ss, transposed in ((q, s, False), (qT, sT, True)):
        R, K = (cols, rows) if transposed else (rows, cols)
        qh = qq.cpu().numpy().reshape(batch, -1)
        sh = ss.cpu().numpy().reshape(batch, -1)
        for b in range(batch):
            src = v[b].T if transposed else v[b]
            s_plain = mx_scales_plain(torch.from_numpy(sh[b]), R, K)
            what = f"{fmt} BOTH {'COL' if transposed else 'ROW'} batch {b}"
            if fmt == "mxfp8":
                assert_mx_equal(qh[b].reshape(R, K), s_plain, nu.mx_quantize(src, axis=1), what)
            else:
                codes, scales = nu.mxfp4_quantize(src, axis=1)
                np.testing.assert_array_equal(qh[b].reshape(R, K // 2), nu.pack_nibbles(codes),
                                              err_msg=what)
                np.testing.assert_array_equal(s_plain, scales, err_msg=what)
    if fmt == "mxfp8":
        assert float(amax.cpu()[0]) == np.abs(v).max()


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("batch,rows,cols", [(4, 128, 192), (300, 64, 320), (1100, 64, 128)])
def test_quantize_skips_entries_that_are_not_live(fmt, batch, rows, cols):
    """With live (a device int32 per batch entry), entries whose count is 0
    keep what their codes and scales held; the others are encoded as
    without the mask: a hand-picked mask on 4 entries, and random masks
    (about 30% of the entries off, the first always off) on 300 and 1100
    small entries."""
    rng = np.random.default_rng(23 + batch)
    bits = _hard_bf16(rng, (batch, rows, cols))
    x = dev_bf16(bits.reshape(-1))
    if batch == 4:
        counts = np.array([3, 0, 1, 0], dtype=np.int32)
    else:
        counts = rng.integers(0, 4, batch).astype(np.int32) * (rng.random(batch) < 0.7)
        counts[:2] = (0, 5)
    dead = set(np.flatnonzero(counts == 0).tolist())
    live = torch.from_numpy(counts).to("cuda")
    nq = batch * rows * cols // (2 if fmt == "mxfp4" else 1)
    outs = [torch.full((n,), 0xAB, dtype=torch.uint8, device="cuda")
            for n in (nq, batch * rows * cols // 32, nq, batch * rows * cols // 32)]
    q, s, qT, sT = outs
    quant = mg.moe_quantize_mxfp8 if fmt == "mxfp8" else mg.moe_quantize_mxfp4
    quant(mode=mg.QUANT_BOTH, batch=batch, rows=rows, cols=cols, x=x, q=q, s=s, qT=qT, sT=sT,
          live=live)
    ref = [torch.full_like(t, 0xAB) for t in outs]
    quant(mode=mg.QUANT_BOTH, batch=batch, rows=rows, cols=cols, x=x, q=ref[0], s=ref[1],
          qT=ref[2], sT=ref[3])
    torch.cuda.synchronize()
    for got, full in zip(outs, ref):
        g = got.view(batch, -1)
        f = full.view(batch, -1)
        written = (g != 0xAB).any(dim=1).cpu().numpy()
        same = (g == f).all(dim=1).cpu().numpy()
        for b in range(batch):
            if b in dead:
                assert not written[b], f"entry {b} was written"
            else:
                assert same[b], f"entry {b}"


@pytest.mark.parametrize("fmt,mode", [("mxfp8", mg.QUANT_BOTH), ("mxfp8", mg.QUANT_ROW),
                                      ("mxfp8", mg.QUANT_COL), ("mxfp4", mg.QUANT_BOTH),
                                      ("mxfp4", mg.QUANT_ROW), ("mxfp4", mg.QUANT_COL)])
def test_quantize_many_slices_per_workgroup(fmt, mode):
    """Inputs larger than one pass of the launch (more 128 x 128 slices than
    workgroups, more 32 x 64 units than waves), with 64-row and 64-column
    tails: sampled slices bit-exact against the oracle's encoding along the
    copy's axis, so each workgroup's later slices (loaded while the one
    before was being encoded) are checked too."""
    batch, rows, cols = 3, 4160, 4160
    rng = np.random.default_rng(77 + mode)
    bits = _hard_bf16(rng, (batch, rows, cols))
    x = dev_bf16(bits.reshape(-1))
    n = batch * rows * cols
    f4 = fmt == "mxfp4"
    nq = n // 2 if f4 else n
    q, qT = (torch.full((nq,), 0xAB, dtype=torch.uint8, device="cuda") for _ in range(2))
    s, sT = (torch.full((n // 32,), 0xAB, dtype=torch.uint8, device="cuda") for _ in range(2))
    kw = dict(mode=mode, batch=batch, rows=rows, cols=cols, x=x, q=q, s=s)
    if mode == mg.QUANT_BOTH:
        kw.update(qT=qT, sT=sT)
    (mg.moe_quantize_mxfp4 if f4 else mg.moe_quantize_mxfp8)(**kw)
    torch.cuda.synchronize()
    # (codes, scales) of the ROW copy (q / s unless COL-only) and the COL copy
    row_out = (q, s) if mode in (mg.QUANT_ROW, mg.QUANT_BOTH) else None
    col_out = (qT, sT) if mode == mg.QUANT_BOTH else ((q, s) if mode == mg.QUANT_COL else None)
    per_b = nq // batch
    ts = 128
    n_r, n_c = -(-rows // ts), -(-cols // ts)
    picks = [(b, i, j) for b in range(batch) for i, j in
             [(n_r - 1, n_c - 1), (0, 0), (n_r - 1, 0), (0, n_c - 1)]] + \
            [(int(rng.integers(batch)), int(rng.integers(n_r)), int(rng.integers(n_c)))
             for _ in range(24)]

    def check(out, transposed, b, r0, c0, rr, cw):
        qq, ss = out
        R, K = (cols, rows) if transposed else (rows, cols)
        qb = qq[b * per_b:(b + 1) * per_b].cpu().numpy().reshape(R, K // 2 if f4 else K)
        sb = mx_scales_plain(ss[b * (n // batch // 32):(b + 1) * (n // batch // 32)], R, K)
        v = nu.bf16_to_f64(bits[b, r0:r0 + rr, c0:c0 + cw])
        if transposed:
            v, (a0, a1, k0, kn) = v.T, (c0, cw, r0, rr)
        else:
            a0, a1, k0, kn = r0, rr, c0, cw
        what = f"{fmt} mode {mode} {'COL' if transposed else 'ROW'} batch {b} slice ({r0}, {c0})"
        s_got = sb[a0:a0 + a1, k0 // 32:(k0 + kn) // 32]
        if f4:
            codes, scales = nu.mxfp4_quantize(v, axis=1)
            np.testing.assert_array_equal(qb[a0:a0 + a1, k0 // 2:(k0 + kn) // 2],
                                          nu.pack_nibbles(codes), err_msg=what)
            np.testing.assert_array_equal(s_got, scales, err_msg=what)
        else:
            assert_mx_equal(qb[a0:a0 + a1, k0:k0 + kn], s_got, nu.mx_quantize(v, axis=1), what)

    for b, i, j in picks:
        r0, c0 = i * ts, j * ts
        rr, cw = min(ts, rows - r0), min(ts, cols - c0)
        if row_out is not None:
            check(row_out, False, b, r0, c0, rr, cw)
        if col_out is not None:
            check(col_out, True, b, r0, c0, rr, cw)


def test_permute_write_mx_bit_exact():
    wl = make_workload("dsv3", T=1500, H=448, with_weights=False)
    x = wl.x
    T, k = wl.expert_idx.shape
    M_cap = -(-(T * k + wl.E * 127) // 128) * 128
    rt = om.route(wl.expert_idx, wl.probs, wl.E, 0, M_cap)
    blk = mg.ExpertBlock(wl.E, wl.H, 64, T, k, M_cap=M_cap, prec=mg.PREC_MXFP8)
    blk.xp_q.fill_(0xAB)
    blk.xp_s.fill_(0xAB)
    blk.route(torch.from_numpy(wl.expert_idx).cuda(), torch.from_numpy(wl.probs).cuda(),
              dev_bf16(x))
    torch.cuda.synchronize()
    compare_routing(blk, rt)
    mp = int(rt.padded_offsets[-1])
    xp = om.permute(nu.bf16_to_f64(x), rt.row_src)
    ref = nu.mx_quantize(xp[:mp], axis=1)
    s_plain = mx_scales_plain(blk.xp_s, M_cap, wl.H)[:mp]
    assert_mx_equal(blk.xp_q.cpu().numpy()[:mp], s_plain, ref, "permuted X")
    assert int(blk.err_flag.cpu()[0]) == 0


def compare_layer_mx(blk, wl, fw, bw, exact=False):
    """exact: the data make every value exact on both sides (bit-exact
    comparisons); else the MXFP8 bounds of gpu_util."""
    compare_routing(blk, fw.rt)
    mp = int(fw.rt.padded_offsets[-1])
    M_cap = blk.M_cap
    valid = fw.expert >= 0
    vmp = valid[:mp]
    gated = wl.act != "srelu"
    N1 = blk.N1
    close = assert_close if exact else assert_close_mx
    mx_cmp = assert_mx_equal if exact else assert_mx_near

    def same(gpu, ora, what):
        if exact:
            np.testing.assert_array_equal(gpu, ora, err_msg=what)
        else:
            close(gpu, ora, what)

    # permuted input, MXFP8 along H: an exact copy, so always bit-exact
    assert_mx_equal(blk.xp_q.cpu().numpy()[:mp],
                    mx_scales_plain(blk.xp_s, M_cap, wl.H)[:mp],
                    nu.mx_quantize(fw.xp[:mp], axis=1), "xp MX")
    z = host_f64(blk.z)[valid]
    if gated:
        z = uninterleave_cols(z, wl.I)
    same(z, fw.z[valid], "z")
    a_gpu = host_f64(blk.a)[valid]
    same(a_gpu, fw.a[valid], "a")
    amax = float(blk.amax.cpu()[0])
    assert amax == np.abs(a_gpu).max()
    assert abs(amax - fw.amax) <= 2.0 ** -7 * fw.amax + 1e-30
    # MXFP8 copies of a: the parity rule, the oracle's encoder applied to the
    # GPU's own bf16 a (pad rows of each group as zeros)
    assert blk.a is not None and blk.dz is not None, "run with bf16_copies=True"
    assert_fused_mx_copies(blk, "a", host_f64(blk.a)[:mp], vmp, wl.I, "a")
    # and, secondarily, against the oracle's encoding of its own a
    mx_cmp(blk.a_q.cpu().numpy()[:mp], mx_scales_plain(blk.a_s, M_cap, wl.I)[:mp],
           nu.mx_quantize(fw.a[:mp], axis=1), "a MX rowwise")
    mx_cmp(blk.aT_q.cpu().numpy()[:, :mp],
           mx_scales_plain(blk.aT_s, wl.I, M_cap)[:, :mp // 32],
           nu.mx_quantize(fw.a[:mp].T, axis=1), "a MX transposed")
    close(host_f64(blk.yp)[valid], fw.y[valid], "yp")
    close(host_f64(blk.out), fw.out, "out")
    # backward
    assert_mx_equal(blk.dyp_q.cpu().numpy()[:mp],
                    mx_scales_plain(blk.dyp_s, M_cap, wl.H)[:mp],
                    nu.mx_quantize(bw.dyp[:mp], axis=1), "dyp MX")
    dz = host_f64(blk.dz)[valid]
    if gated:
        dz = uninterleave_cols(dz, wl.I)
    same(dz, bw.dz[valid], "dz")
    # the parity rule on the GPU's own dz (GPU column order), then the
    # oracle's dz in the interleaved column order of the GPU's copies
    assert_fused_mx_copies(blk, "dz", host_f64(blk.dz)[:mp], vmp, N1, "dz")
    dz_or = bw.dz[:mp][:, om.interleave_rows(wl.I)] if gated else bw.dz[:mp]
    mx_cmp(blk.dz_q.cpu().numpy()[:mp], mx_scales_plain(blk.dz_s, M_cap, N1)[:mp],
           nu.mx_quantize(dz_or, axis=1), "dz MX rowwise")
    mx_cmp(blk.dzT_q.cpu().numpy()[:, :mp],
           mx_scales_plain(blk.dzT_s, N1, M_cap)[:, :mp // 32],
           nu.mx_quantize(dz_or.T, axis=1), "dz MX transposed")
    dp = blk.dprobs_p.cpu().numpy().astype(np.float64)
    same(dp[valid], bw.dp[valid], "dprobs_p")
    close(host_f64(blk.dxp)[valid], bw.dxp[valid], "dxp")
    close(host_f64(blk.dx), bw.dx, "dx")
    close(blk.dprobs.cpu().numpy(), bw.dprobs, "dprobs")


MX_CASES = {
    "tiny": dict(name="tiny"),
    "multi_tile_ragged": dict(name="tiny", E=8, k=2, T=1024, H=640, I=320),
    "gptoss_act": dict(name="gptoss", T=512, H=128, I=192, E=16),
    "clamp_binding": dict(name="gptoss", T=512, H=128, I=192, E=16, clamp=0.25),
    "geglu": dict(name="tiny", act="geglu", T=384, I=192),
    "srelu": dict(name="tiny", act="srelu", T=384, I=192),
    "dsv3_zipf_empty": dict(name="dsv3", T=2000, H=256, I=128),
}


@pytest.mark.parametrize("case", list(MX_CASES))
def test_layer_mx_parity(case):
    kw = dict(MX_CASES[case])
    wl = make_workload(kw.pop("name"), seed=5, **kw)
    M_cap = -(-wl.m_cap() // 128) * 128
    blk = run_gpu_layer(wl, M_cap, prec=mg.PREC_MXFP8)
    fw, bw = oracle_layer(wl, M_cap, mx=True)
    compare_layer_mx(blk, wl, fw, bw)
    assert int(blk.err_flag.cpu()[0]) == 0


def test_layer_mx_partial_last_round_parity():
    """MXFP8 plain-store GEMMs (FC2, FC1 dgrad) with a partial last round (a
    grid of 8 workgroups over 26 output tiles): the tail tiles run whole (the
    K split of the last round is bf16 only), results against the oracle."""
    wl = make_workload("tiny", seed=13, E=4, k=2, T=1536, H=512, I=512)
    M_cap = -(-wl.m_cap() // 128) * 128
    margin = torch.cuda.get_device_properties(0).multi_processor_count - 8
    G = gemm_grid(margin, M_cap, wl.E, wl.H)
    sizes = [int((wl.expert_idx == e).sum()) for e in range(wl.E)]
    assert G == 8
    # the bf16 kernels would split this tail (the case stays a split-sized one)
    assert tail_split_parts(sizes, wl.H, wl.I, G, 128) > 1         # FC2
    assert tail_split_parts(sizes, wl.H, 2 * wl.I, G, 128) > 1     # FC1 dgrad
    gp, _ = act_of(wl)
    blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp, M_cap=M_cap,
                         cu_margin=margin, prec=mg.PREC_MXFP8, bf16_copies=True)
    run_gpu_layer(wl, M_cap, block=blk)
    fw, bw = oracle_layer(wl, M_cap, mx=True)
    compare_layer_mx(blk, wl, fw, bw)
    assert int(blk.err_flag.cpu()[0]) == 0


def _sparse_ints(rng, shape, nnz_per_row):
    """Rows of {-1, 0, 1} with `nnz_per_row` non-zeros (as bf16 bits)."""
    v = np.zeros(shape)
    n = shape[-1]
    flat = v.reshape(-1, n)
    for r in range(flat.shape[0]):
        cols = rng.choice(n, size=nnz_per_row, replace=False)
        flat[r, cols] = rng.choice([-1.0, 1.0], size=nnz_per_row)
    return nu.f64_to_bf16_bits(v)


@pytest.mark.parametrize("act,beta", [("srelu", 1.0), ("swiglu", 0.0), ("geglu", 1.0)])
def test_layer_mx_exact_on_integer_data(act, beta):
    """With at most 8 non-zeros of +-1 per row of X and dOut, weights in
    {-1, 0, 1} and probabilities that are powers of two, |z|, |dA| <= 8, so z,
    a, dz and dprobs_p are exact in bf16 / fp32 on both sides (for GeGLU the
    gate weights are zero, so g = 0 and GELU(g) = 0, GELU'(0) = 1/2 exactly)."""
    wl = make_workload("tiny", seed=9, act=act, beta=beta, E=6, T=640, H=192, I=192)
    rng = np.random.default_rng(123)
    wl.x = _sparse_ints(rng, (wl.T, wl.H), 8)
    wl.dout = _sparse_ints(rng, (wl.T, wl.H), 8)
    n1 = 2 * wl.I if act != "srelu" else wl.I
    w1 = rng.integers(-1, 2, size=(wl.E, n1, wl.H)).astype(np.float64)
    if act == "geglu":
        w1[:, :wl.I, :] = 0.0
    wl.w1 = nu.f64_to_bf16_bits(w1)
    wl.w2 = nu.f64_to_bf16_bits(rng.integers(-1, 2, size=(wl.E, wl.H, wl.I)).astype(np.float64))
    wl.probs = rng.choice([1.0, 0.5, 0.25, 0.125], size=wl.probs.shape).astype(np.float32)
    M_cap = -(-wl.m_cap() // 128) * 128
    blk = run_gpu_layer(wl, M_cap, prec=mg.PREC_MXFP8)
    fw, bw = oracle_layer(wl, M_cap, mx=True)
    assert np.abs(fw.z).max() <= 8
    assert np.abs(bw.dz).max() > 0 and (act == "geglu" or np.abs(fw.a).max() > 0)
    compare_layer_mx(blk, wl, fw, bw, exact=True)


def test_weight_copies_bit_exact():
    """The four weight copies the MXFP8 GEMMs read (ExpertBlock.quantize_weights)."""
    wl = make_workload("tiny", seed=2, E=3, H=192, I=128)
    blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, prec=mg.PREC_MXFP8)
    blk.load_weights(dev_bf16(wl.w1), dev_bf16(wl.w2))
    torch.cuda.synchronize()
    w1i = nu.bf16_to_f64(om.repack_interleave(wl.w1))
    w2 = nu.bf16_to_f64(wl.w2)
    E, H, I, N1 = wl.E, wl.H, wl.I, blk.N1
    for name, q, s, ref_fn, R, K in (
            ("w1 along H", blk.w1_q, blk.w1_s, lambda e: w1i[e], N1, H),
            ("w2 along I", blk.w2_q, blk.w2_s, lambda e: w2[e], H, I),
            ("w2 along H", blk.w2t_q, blk.w2t_s, lambda e: w2[e].T, I, H),
            ("w1 along N1", blk.w1t_q, blk.w1t_s, lambda e: w1i[e].T, H, N1)):
        qh = q.cpu().numpy()
        sh = s.cpu().numpy().reshape(E, -1)
        for e in range(E):
            assert_mx_equal(qh[e], mx_scales_plain(torch.from_numpy(sh[e]), R, K),
                            nu.mx_quantize(ref_fn(e), axis=1), f"{name} expert {e}")


def test_mx_graph_capture_replays_match_eager():
    wl = make_workload("tiny", seed=13, E=8, T=1024, H=256, I=256)
    blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, prec=mg.PREC_MXFP8)
    blk.load_weights(dev_bf16(wl.w1), dev_bf16(wl.w2))
    x, dout = dev_bf16(wl.x), dev_bf16(wl.dout)
    idx = torch.from_numpy(wl.expert_idx).cuda()
    probs = torch.from_numpy(wl.probs).cuda()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        blk.forward(x, idx, probs)
        blk.backward(dout)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    outs = (blk.out, blk.dx, blk.dprobs, blk.a_q, blk.dz_q)
    eager = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="global"):
        blk.forward(x, idx, probs)
        blk.backward(dout)
    mp = int(blk.padded_offsets[-1].item())
    for _ in range(3):
        for t in outs:
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outs, eager)):
            if i >= 3:
                t, e = t[:mp], e[:mp]
            assert torch.equal(t, e)


def test_mx_outputs_do_not_depend_on_bf16_copies():
    """Without the optional bf16 a and dz the MXFP8 outputs are bit-identical."""
    wl = make_workload("tiny", seed=21, E=8, T=768, H=256, I=192)
    M_cap = -(-wl.m_cap() // 128) * 128
    b1 = run_gpu_layer(wl, M_cap, prec=mg.PREC_MXFP8, bf16_copies=True)
    r1 = [t.clone() for t in (b1.a_q, b1.aT_q, b1.dz_q, b1.dzT_q, b1.out, b1.dx, b1.dprobs)]
    b2 = run_gpu_layer(wl, M_cap, prec=mg.PREC_MXFP8, bf16_copies=False)
    assert b2.a is None and b2.dz is None
    mp = int(b2.padded_offsets[-1].item())
    for i, (u, v) in enumerate(zip(r1, (b2.a_q, b2.aT_q, b2.dz_q, b2.dzT_q, b2.out, b2.dx,
                                         b2.dprobs))):
        if i in (0, 2):
            u, v = u[:mp], v[:mp]
        elif i in (1, 3):
            u, v = u[:, :mp], v[:, :mp]
        assert torch.equal(u, v), i
