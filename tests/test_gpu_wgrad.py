"""Weight-gradient grouped GEMMs (moe_grouped_mlp_wgrad) against the oracle's
weight_grads, through the C ABI.

bf16: the GEMMs read dz, Xp, dYp and a as the layer stored them (rows
outside the groups' data, which the epilogues never write, are not read).
MXFP8: a and dz come from the epilogues' transposed copies, Xp and dYp from
moe_quantize_mxfp8 (MOE_QUANT_COL) of their bf16 rows, which the permutes
produce exactly (bit for bit the oracle's values).  The MXFP8 GEMMs are checked against the oracle's
contraction of the very MXFP8 operands the GPU read (the epilogues' copies
can differ from the oracle's own encoding by a code where a bf16 value
differs by an ulp, which the fused-epilogue tests bound), and element by
element against the independent MXFP8 oracle
(gpu_util.assert_close_mx_contraction: every element within the bound one
E4M3 step per operand puts on its terms, the scale-aware bar on all but
0.5%, relative L2 below 1e-2)."""

import dataclasses

import numpy as np
import pytest
import torch

import moe_grouped_mlp_amd as mg
from oracle import moe as om
from oracle import numerics as nu
from workloads import make_workload

from .gpu_util import (assert_close, assert_close_mx_contraction, dev_bf16, host_f64,
                       mx_scales_plain, oracle_layer, run_gpu_layer, uninterleave_cols)

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": dict(name="tiny"),
    "multi_tile_ragged": dict(name="tiny", E=8, k=2, T=1024, H=640, I=320),
    "gptoss_act": dict(name="gptoss", T=512, H=128, I=192, E=16),
    "dsv3_zipf_empty": dict(name="dsv3", T=2000, H=256, I=128),
    "srelu": dict(name="tiny", act="srelu", T=384, I=192),
}


def _m_cap(wl):
    return -(-wl.m_cap() // 128) * 128


def _abs_products(fw, bw):
    """|dz_e|^T |xp_e| and |dyp_e|^T |a_e| over each expert's rows (logical
    column order): the scale of each weight-gradient element's terms."""
    rt = fw.rt
    E = len(rt.split_sizes)
    p1 = np.zeros((E, bw.dz.shape[1], fw.xp.shape[1]))
    p2 = np.zeros((E, bw.dyp.shape[1], fw.a.shape[1]))
    for e in range(E):
        r = slice(int(rt.padded_offsets[e]), int(rt.padded_offsets[e]) + int(rt.split_sizes[e]))
        p1[e] = np.abs(bw.dz[r]).T @ np.abs(fw.xp[r])
        p2[e] = np.abs(bw.dyp[r]).T @ np.abs(fw.a[r])
    return p1, p2


def _logical_dw1(dw1, wl):
    """GPU dW1 rows follow dz's (interleaved) column order; the oracle's are
    logical (gate | up)."""
    g = host_f64(dw1)
    if wl.act == "srelu":
        return g
    return np.stack([uninterleave_cols(g[e].T, wl.I).T for e in range(wl.E)])


@pytest.mark.parametrize("case", list(CASES))
def test_wgrad_bf16_parity(case):
    kw = dict(CASES[case])
    wl = make_workload(kw.pop("name"), seed=3, **kw)
    # bf16 takes any M_cap (here T k + E (A - 1), as ExpertBlock allocates)
    M_cap = wl.m_cap()
    blk = run_gpu_layer(wl, M_cap)
    fw, bw = oracle_layer(wl, M_cap)
    # rows the layer never wrote hold NaN: they must not be read
    pad = torch.from_numpy(fw.expert < 0).cuda()
    for t in (blk.a, blk.dz):
        t[pad] = float("nan")
    gated = wl.act != "srelu"
    N1 = 2 * wl.I if gated else wl.I
    dw1 = torch.empty(wl.E, N1, wl.H, dtype=torch.bfloat16, device="cuda")
    dw2 = torch.empty(wl.E, wl.H, wl.I, dtype=torch.bfloat16, device="cuda")
    mg.moe_grouped_mlp_wgrad(
        E=wl.E, H=wl.H, I=wl.I, M_cap=M_cap, gated=gated,
        split_sizes=blk.split_sizes, padded_offsets=blk.padded_offsets,
        prec=mg.PREC_BF16, dz=blk.dz, xp=blk.xp, dyp=blk.dyp, a=blk.a, dw1=dw1, dw2=dw2)
    torch.cuda.synchronize()
    ow1, ow2 = om.weight_grads(fw, bw)
    assert_close(_logical_dw1(dw1, wl), ow1, "dw1")
    assert_close(host_f64(dw2), ow2, "dw2")
    empty = np.flatnonzero(fw.rt.split_sizes == 0)
    if case == "dsv3_zipf_empty":
        assert len(empty) >= 2
    for e in empty:     # an expert without rows gets exact zeros
        assert np.all(host_f64(dw1[e]) == 0) and np.all(host_f64(dw2[e]) == 0)


@pytest.mark.parametrize("case", ["multi_tile_ragged", "dsv3_zipf_empty"])
def test_wgrad_mxfp8_parity(case):
    kw = dict(CASES[case])
    wl = make_workload(kw.pop("name"), seed=4, **kw)
    M_cap = _m_cap(wl)
    blk = run_gpu_layer(wl, M_cap, prec=mg.PREC_MXFP8)
    fw, bw = oracle_layer(wl, M_cap, mx=True)
    u8 = dict(dtype=torch.uint8, device="cuda")
    copies = {}
    for name, rows in (("xp", fw.xp), ("dyp", bw.dyp)):
        x = dev_bf16(nu.f64_to_bf16_bits(rows))
        q = torch.empty(wl.H, M_cap, **u8)
        s = torch.empty(wl.H * M_cap // 32, **u8)
        mg.moe_quantize_mxfp8(mode=mg.QUANT_COL, batch=1, rows=M_cap, cols=wl.H,
                              x=x, q=q, s=s)
        copies[name] = (q, s)
    N1 = 2 * wl.I
    dw1 = torch.empty(wl.E, N1, wl.H, dtype=torch.bfloat16, device="cuda")
    dw2 = torch.empty(wl.E, wl.H, wl.I, dtype=torch.bfloat16, device="cuda")
    mg.moe_grouped_mlp_wgrad(
        E=wl.E, H=wl.H, I=wl.I, M_cap=M_cap, gated=True,
        split_sizes=blk.split_sizes, padded_offsets=blk.padded_offsets,
        prec=mg.PREC_MXFP8, dzT_q=blk.dzT_q, dzT_s=blk.dzT_s,
        xpT_q=copies["xp"][0], xpT_s=copies["xp"][1],
        dypT_q=copies["dyp"][0], dypT_s=copies["dyp"][1],
        aT_q=blk.aT_q, aT_s=blk.aT_s, dw1=dw1, dw2=dw2)
    torch.cuda.synchronize()

    def deq(q, s_, R):     # a GPU MXFP8 copy [R][M_cap] -> its values
        codes = q.cpu().numpy().reshape(R, M_cap)
        return nu.mx_dequantize(codes, mx_scales_plain(s_, R, M_cap), axis=1)

    # the oracle's contraction of the GPU's operands (dz rows interleaved,
    # like the GPU's dW1 rows)
    fw_g = dataclasses.replace(fw, xp=deq(*copies["xp"], wl.H).T,
                               a=deq(blk.aT_q, blk.aT_s, wl.I).T)
    bw_g = dataclasses.replace(bw, dz=deq(blk.dzT_q, blk.dzT_s, N1).T,
                               dyp=deq(*copies["dyp"], wl.H).T)
    rw1, rw2 = om.weight_grads(fw_g, bw_g)
    assert_close(host_f64(dw1), rw1, "dw1")
    assert_close(host_f64(dw2), rw2, "dw2")
    # and the independent MXFP8 oracle, element by element
    ow1, ow2 = om.weight_grads(fw, bw, mx=True)
    p1, p2 = _abs_products(fw, bw)
    assert_close_mx_contraction(_logical_dw1(dw1, wl), ow1, p1, "dw1 vs independent oracle")
    assert_close_mx_contraction(host_f64(dw2), ow2, p2, "dw2 vs independent oracle")
    for e in np.flatnonzero(fw.rt.split_sizes == 0):
        assert np.all(host_f64(dw1[e]) == 0) and np.all(host_f64(dw2[e]) == 0)


def test_wgrad_rejects_bad_arguments():
    wl = make_workload("tiny", seed=1)
    M_cap = _m_cap(wl)
    i32 = dict(dtype=torch.int32, device="cuda")
    split = torch.zeros(wl.E, **i32)
    pad = torch.zeros(wl.E + 1, **i32)
    t = torch.zeros(wl.H, M_cap, dtype=torch.bfloat16, device="cuda")
    base = dict(E=wl.E, H=wl.H, I=wl.I, M_cap=M_cap, split_sizes=split,
                padded_offsets=pad, dyp=t, a=t,
                dw2=torch.empty(wl.E, wl.H, wl.I, dtype=torch.bfloat16, device="cuda"))
    for bad in (dict(M_cap=0), dict(H=100), dict(a=None),
                dict(prec=mg.PREC_MXFP8), dict(E=0)):
        with pytest.raises(mg.MoeError):
            mg.moe_grouped_mlp_wgrad(**{**base, **bad})


@pytest.mark.parametrize("prec", [mg.PREC_BF16, mg.PREC_MXFP8])
def test_block_weight_grads(prec):
    """ExpertBlock(wgrad=True).weight_grads() after a forward + backward: the
    bf16 path against the oracle's bf16 weight gradients, the MXFP8 path
    (transposed copies of Xp and dYp made by the block) against the MXFP8
    oracle element by element (gpu_util.assert_close_mx_contraction)."""
    wl = make_workload("tiny", seed=8, E=8, k=2, T=1024, H=640, I=320)
    M_cap = _m_cap(wl)
    gp = mg.act_params(mg.ACT_SWIGLU, beta=wl.beta)
    blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp, M_cap=M_cap,
                         prec=prec, wgrad=True)
    run_gpu_layer(wl, M_cap, block=blk)
    dw1, dw2 = blk.weight_grads()
    torch.cuda.synchronize()
    mx = prec == mg.PREC_MXFP8
    fw, bw = oracle_layer(wl, M_cap, mx=mx)
    ow1, ow2 = om.weight_grads(fw, bw, mx=mx)
    g1, g2 = _logical_dw1(dw1, wl), host_f64(dw2)
    if mx:
        p1, p2 = _abs_products(fw, bw)
        assert_close_mx_contraction(g1, ow1, p1, "dw1")
        assert_close_mx_contraction(g2, ow2, p2, "dw2")
    else:
        assert_close(g1, ow1, "dw1")
        assert_close(g2, ow2, "dw2")
