"""The unfused MXFP4 layer (ExpertBlock(prec=PREC_MXFP4, unfused=True): the
separate passes with every GEMM operand quantized by moe_quantize_mxfp4 and
multiplied by the MXFP4 grouped GEMM) against the oracle's MXFP4 unfused
reading.  Where a
GEMM reads the MXFP4 encoding of a tensor the GPU computed (a for FC2, dz
for FC1 dgrad), a one-ulp difference in that bf16 tensor can move an E2M1
code by a whole step; those outputs are checked element by element against
the oracle fed the GPU's own tensor, and against the independent oracle by
relative L2 error.  The combines (out, dX) and the dprobs gather are checked
bit for bit against the oracle's unpermute / gather of the GPU's own yp, dxp
and dprobs_p."""

import numpy as np
import pytest
import torch

import moe_grouped_mlp_amd as mg
from oracle import moe as om
from oracle import numerics as nu
from workloads import make_workload

from .gpu_util import (act_of, assert_close, compare_routing, host_bits, host_f64,
                       oracle_layer, run_gpu_layer, uninterleave_cols)

pytestmark = pytest.mark.gpu

CASES = {
    "multi_tile_ragged": dict(name="tiny", E=8, k=2, T=1024, H=640, I=320),
    "gptoss_act": dict(name="gptoss", T=512, H=128, I=192, E=16),
    "dsv3_zipf_empty": dict(name="dsv3", T=2000, H=256, I=128),
    "srelu": dict(name="tiny", act="srelu", T=384, I=192),
}


def _rel_l2(u, v):
    return float(np.linalg.norm(u - v) / max(np.linalg.norm(v), 1e-30))


@pytest.mark.parametrize("case", list(CASES))
def test_mxfp4_layer_parity(case):
    kw = dict(CASES[case])
    wl = make_workload(kw.pop("name"), seed=9, **kw)
    M_cap = -(-wl.m_cap() // 128) * 128
    gp, _ = act_of(wl)
    blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp, first_expert=wl.first_expert,
                         M_cap=M_cap, prec=mg.PREC_MXFP4, unfused=True)
    run_gpu_layer(wl, M_cap, block=blk)
    fw, bw = oracle_layer(wl, M_cap, mx="mxfp4", unfused=True)
    compare_routing(blk, fw.rt)
    gated = wl.act != "srelu"
    valid = fw.expert >= 0
    pad = fw.rt.padded_offsets
    w1 = nu.bf16_to_f64(wl.w1)
    w2 = nu.bf16_to_f64(wl.w2)
    np.testing.assert_array_equal(host_bits(blk.xp)[valid], nu.f64_to_bf16_bits(fw.xp[valid]))
    z = host_f64(blk.z)[valid]
    assert_close(uninterleave_cols(z, wl.I) if gated else z, fw.z[valid], "z")
    a = host_f64(blk.a)
    assert_close(a[valid], fw.a[valid], "a")
    # FC2 on the MXFP4 encoding of the GPU's a
    yp = host_f64(blk.yp)
    for e in range(wl.E):
        rows = slice(int(pad[e]), int(pad[e]) + int(fw.rt.split_sizes[e]))
        if rows.stop == rows.start:
            continue
        ref = nu.round_bf16(nu.mxfp4_round(a[rows], 1) @ nu.mxfp4_round(w2[e], 1).T)
        assert_close(yp[rows], ref, f"yp expert {e}")
    assert _rel_l2(yp[valid], fw.y[valid]) < 2e-2
    assert _rel_l2(host_f64(blk.out), fw.out) < 2e-2
    # the combine, element by element: bit-exact against the oracle's
    # unpermute of the GPU's own yp
    np.testing.assert_array_equal(host_bits(blk.out),
                                  nu.f64_to_bf16_bits(om.unpermute(yp, fw.rt.row_id_map)))
    # backward
    np.testing.assert_array_equal(host_bits(blk.dyp)[valid], nu.f64_to_bf16_bits(bw.dyp[valid]))
    dz = host_f64(blk.dz)
    dz = uninterleave_cols(dz, wl.I) if gated else dz
    assert_close(dz[valid], bw.dz[valid], "dz")
    dp = blk.dprobs_p.cpu().numpy().astype(np.float64)
    assert_close(dp[valid], bw.dp[valid], "dprobs_p")
    assert_close(blk.dprobs.cpu().numpy(), bw.dprobs, "dprobs")
    dxp = host_f64(blk.dxp)
    for e in range(wl.E):
        rows = slice(int(pad[e]), int(pad[e]) + int(fw.rt.split_sizes[e]))
        if rows.stop == rows.start:
            continue
        ref = nu.round_bf16(nu.mxfp4_round(dz[rows], 1) @ nu.mxfp4_round(w1[e], 0))
        assert_close(dxp[rows], ref, f"dxp expert {e}")
    assert _rel_l2(dxp[valid], bw.dxp[valid]) < 2e-2
    assert _rel_l2(host_f64(blk.dx), bw.dx) < 2e-2
    # dX and dprobs, element by element: bit-exact against the oracle's
    # unpermute of the GPU's dxp and gather of the GPU's dprobs_p
    np.testing.assert_array_equal(host_bits(blk.dx),
                                  nu.f64_to_bf16_bits(om.unpermute(dxp, fw.rt.row_id_map)))
    np.testing.assert_array_equal(
        blk.dprobs.cpu().numpy(),
        om.gather_probs_grad(blk.dprobs_p.cpu().numpy(), fw.rt.row_id_map).astype(np.float32))


def test_mxfp4_layer_rejects_fused_only_options():
    """Weight gradients and recompute belong to the fused MXFP4 layer."""
    for kw in (dict(recompute=True), dict(wgrad=True)):
        with pytest.raises(ValueError):
            mg.ExpertBlock(4, 256, 128, 64, 2, prec=mg.PREC_MXFP4, unfused=True, **kw)


def _graph_replays_match_eager(blk, wl, rows_tensors):
    """Eager step on a side stream, then the same step captured in one graph
    and replayed three times with the outputs cleared before each replay:
    every replay must reproduce the eager outputs bit for bit."""
    from .gpu_util import dev_bf16
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
    outs = [blk.out, blk.dx, blk.dprobs] + [getattr(blk, n) for n in rows_tensors]
    # routed rows only: the GEMMs do not write pad rows
    split = blk.split_sizes.cpu().numpy()
    pad = blk.padded_offsets.cpu().numpy()
    rows = np.zeros(blk.M_cap, dtype=bool)
    for e in range(blk.E):
        rows[pad[e]:pad[e] + split[e]] = True
    rows = torch.from_numpy(rows).cuda()
    eager = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="global"):
        blk.forward(x, idx, probs)
        blk.backward(dout)
    for _ in range(3):
        for t in outs:
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outs, eager)):
            if i >= 3:
                t, e = t[rows], e[rows]
            assert torch.equal(t, e), f"output {i} differs on a replay"


@pytest.mark.parametrize("unfused", [True, False])
def test_mxfp4_layer_graph_capture_replays_match_eager(unfused):
    wl = make_workload("tiny", seed=13, E=8, T=1024, H=256, I=256)
    blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, prec=mg.PREC_MXFP4, unfused=unfused)
    _graph_replays_match_eager(blk, wl, ("yp", "dxp"))


@pytest.mark.parametrize("prec", [mg.PREC_BF16, mg.PREC_MXFP8])
def test_recompute_graph_capture_replays_match_eager(prec):
    """The recompute step (forward without z, z rebuilt in the backward) in
    one graph."""
    wl = make_workload("tiny", seed=14, E=8, T=1024, H=256, I=256)
    blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, prec=prec, recompute=True,
                         z_scratch=torch.empty((wl.m_cap() + 128) * 2 * wl.I,
                                               dtype=torch.bfloat16, device="cuda"))
    blk.keep_recomputed_z = True
    _graph_replays_match_eager(blk, wl, ("z", "dxp"))
