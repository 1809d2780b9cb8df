"""The fused MXFP4 layer (ExpertBlock(prec=PREC_MXFP4)): permutes that write
MXFP4 rows, GLU / dGLU epilogues that write the MXFP4 copies of a and dz,
four MXFP4 grouped GEMMs, against the oracle's fused MXFP4 reading.

Every MXFP4 copy is checked bit for bit: the permuted X and dOut against the
oracle's encoding of the permuted rows, and the epilogues' copies of a and
dz against the oracle's encoding of the GPU's own bf16 a and dz (pad rows of
each group as zeros): both sides encode the same bf16 numbers with the same
rule, in exact arithmetic.  The GEMM outputs that read an encoding of a
tensor the GPU computed (yp from a, dxp from dz) are checked element by
element against the oracle fed the GPU's tensor, and against the
independent oracle by relative L2 error (a one-ulp difference in a bf16
value can move its E2M1 code by a whole step)."""

import numpy as np
import pytest
import torch

import moe_grouped_mlp_amd as mg
from oracle import moe as om
from oracle import numerics as nu
from workloads import make_workload

from .gpu_util import (act_of, assert_close, compare_routing, dev_bf16, host_bits,
                       host_f64, mx_scales_plain, oracle_layer, rows_with_pad_zeroed,
                       run_gpu_layer, uninterleave_cols)

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": dict(name="tiny"),
    "multi_tile_ragged": dict(name="tiny", E=8, k=2, T=1024, H=640, I=320),
    "gptoss_act": dict(name="gptoss", T=512, H=128, I=192, E=16),
    "clamp_binding": dict(name="gptoss", T=512, H=128, I=192, E=16, clamp=0.25),
    "geglu": dict(name="tiny", act="geglu", T=384, I=192),
    "srelu": dict(name="tiny", act="srelu", T=384, I=192),
    "dsv3_zipf_empty": dict(name="dsv3", T=2000, H=256, I=128),
}


def _rel_l2(u, v):
    return float(np.linalg.norm(u - v) / max(np.linalg.norm(v), 1e-30))


def assert_mx4_equal(q, s, M_cap, K, mp, values, what):
    """Packed codes q ([M_cap][K/2] bytes) and tiled scales s of an MXFP4
    operand, rows [0, mp), bit for bit against the oracle's encoding of
    `values` ([mp][K], blocks along K)."""
    codes, scales = nu.mxfp4_quantize(values, axis=1)
    qg = q.detach().cpu().numpy().reshape(M_cap, K // 2)[:mp]
    sg = mx_scales_plain(s, M_cap, K)[:mp]
    bad = np.flatnonzero(sg.reshape(-1) != scales.reshape(-1))
    assert bad.size == 0, (f"{what}: {bad.size} of {scales.size} scales differ; first at "
                           f"{bad[:5]}: gpu {sg.reshape(-1)[bad[:5]]} oracle "
                           f"{scales.reshape(-1)[bad[:5]]}")
    ref = nu.pack_nibbles(codes)
    bad = np.flatnonzero(qg.reshape(-1) != ref.reshape(-1))
    assert bad.size == 0, (f"{what}: {bad.size} of {ref.size} code bytes differ; first at "
                           f"{bad[:5]}: gpu {qg.reshape(-1)[bad[:5]]} oracle "
                           f"{ref.reshape(-1)[bad[:5]]}")


def compare_layer_mx4(blk, wl, fw, bw):
    compare_routing(blk, fw.rt)
    M_cap, mp = blk.M_cap, int(fw.rt.padded_offsets[-1])
    valid = fw.expert >= 0
    vmp = valid[:mp]
    pad = fw.rt.padded_offsets
    gated = wl.act != "srelu"
    N1 = blk.N1
    w1i = nu.bf16_to_f64(om.repack_interleave(wl.w1)) if gated else nu.bf16_to_f64(wl.w1)
    w2 = nu.bf16_to_f64(wl.w2)

    def groups():
        for e in range(wl.E):
            rows = slice(int(pad[e]), int(pad[e]) + int(fw.rt.split_sizes[e]))
            if rows.stop > rows.start:
                yield e, rows

    # permuted input: the bf16 rows and their MXFP4 encoding along H
    np.testing.assert_array_equal(host_bits(blk.xp)[valid], nu.f64_to_bf16_bits(fw.xp[valid]))
    assert_mx4_equal(blk.xp_q4, blk.xp_s4, M_cap, wl.H, mp, fw.xp[:mp], "xp MXFP4")
    z = host_f64(blk.z)[valid]
    assert_close(uninterleave_cols(z, wl.I) if gated else z, fw.z[valid], "z")
    a = host_f64(blk.a)
    assert_close(a[valid], fw.a[valid], "a")
    # the GLU epilogue's MXFP4 copy of its own bf16 a
    assert_mx4_equal(blk.a_q4, blk.a_s4, M_cap, wl.I, mp,
                     rows_with_pad_zeroed(a[:mp], vmp), "a MXFP4")
    yp = host_f64(blk.yp)
    for e, rows in groups():
        ref = nu.round_bf16(nu.mxfp4_round(a[rows], 1) @ nu.mxfp4_round(w2[e], 1).T)
        assert_close(yp[rows], ref, f"yp expert {e}")
    assert _rel_l2(yp[valid], fw.y[valid]) < 2e-2
    assert _rel_l2(host_f64(blk.out), fw.out) < 2e-2
    np.testing.assert_array_equal(host_bits(blk.out),
                                  nu.f64_to_bf16_bits(om.unpermute(yp, fw.rt.row_id_map)))
    # backward
    np.testing.assert_array_equal(host_bits(blk.dyp)[valid], nu.f64_to_bf16_bits(bw.dyp[valid]))
    assert_mx4_equal(blk.dyp_q4, blk.dyp_s4, M_cap, wl.H, mp, bw.dyp[:mp], "dyp MXFP4")
    dz_st = host_f64(blk.dz)                       # GPU column order
    dz = uninterleave_cols(dz_st, wl.I) if gated else dz_st
    assert_close(dz[valid], bw.dz[valid], "dz")
    # the dGLU epilogue's MXFP4 copy of its own bf16 dz, in its column order
    assert_mx4_equal(blk.dz_q4, blk.dz_s4, M_cap, N1, mp,
                     rows_with_pad_zeroed(dz_st[:mp], vmp), "dz MXFP4")
    dp = blk.dprobs_p.cpu().numpy().astype(np.float64)
    assert_close(dp[valid], bw.dp[valid], "dprobs_p")
    assert_close(blk.dprobs.cpu().numpy(), bw.dprobs, "dprobs")
    dxp = host_f64(blk.dxp)
    for e, rows in groups():
        ref = nu.round_bf16(nu.mxfp4_round(dz_st[rows], 1) @ nu.mxfp4_round(w1i[e], 0))
        assert_close(dxp[rows], ref, f"dxp expert {e}")
    assert _rel_l2(dxp[valid], bw.dxp[valid]) < 2e-2
    assert _rel_l2(host_f64(blk.dx), bw.dx) < 2e-2
    np.testing.assert_array_equal(host_bits(blk.dx),
                                  nu.f64_to_bf16_bits(om.unpermute(dxp, fw.rt.row_id_map)))
    np.testing.assert_array_equal(
        blk.dprobs.cpu().numpy(),
        om.gather_probs_grad(blk.dprobs_p.cpu().numpy(), fw.rt.row_id_map).astype(np.float32))


@pytest.mark.parametrize("case", list(CASES))
def test_fused_mxfp4_layer_parity(case):
    kw = dict(CASES[case])
    wl = make_workload(kw.pop("name"), seed=11, **kw)
    M_cap = -(-wl.m_cap() // 128) * 128
    blk = run_gpu_layer(wl, M_cap, prec=mg.PREC_MXFP4, bf16_copies=True)
    assert not blk.unfused
    fw, bw = oracle_layer(wl, M_cap, mx="mxfp4")
    compare_layer_mx4(blk, wl, fw, bw)
    assert int(blk.err_flag.cpu()[0]) == 0


def test_fused_mxfp4_partial_last_round():
    """A grid of 8 workgroups over many output tiles: the MXFP4 plain-store
    GEMMs run their last, partial round unsplit."""
    wl = make_workload("tiny", seed=13, E=4, k=2, T=1536, H=512, I=512)
    M_cap = -(-wl.m_cap() // 128) * 128
    margin = torch.cuda.get_device_properties(0).multi_processor_count - 8
    gp, _ = act_of(wl)
    blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp, M_cap=M_cap,
                         cu_margin=margin, prec=mg.PREC_MXFP4, bf16_copies=True)
    run_gpu_layer(wl, M_cap, block=blk)
    fw, bw = oracle_layer(wl, M_cap, mx="mxfp4")
    compare_layer_mx4(blk, wl, fw, bw)
    assert int(blk.err_flag.cpu()[0]) == 0


def test_fused_mxfp4_outputs_do_not_depend_on_bf16_copies():
    """Without the bf16 Xp, dYp, a and dz the MXFP4 results are bit-identical."""
    wl = make_workload("tiny", seed=21, E=8, T=768, H=256, I=192)
    M_cap = -(-wl.m_cap() // 128) * 128
    b1 = run_gpu_layer(wl, M_cap, prec=mg.PREC_MXFP4, bf16_copies=True)
    names = ("xp_q4", "dyp_q4", "a_q4", "dz_q4", "a_s4", "dz_s4", "out", "dx", "dprobs")
    r1 = [getattr(b1, n).clone() for n in names]
    b2 = run_gpu_layer(wl, M_cap, prec=mg.PREC_MXFP4, bf16_copies=False)
    assert b2.a is None and b2.dz is None and b2.xp is None and b2.dyp is None
    mp = int(b2.padded_offsets[-1].item())
    rows = {"xp_q4": wl.H // 2, "dyp_q4": wl.H // 2, "a_q4": wl.I // 2, "dz_q4": b2.N1 // 2,
            "a_s4": wl.I // 32, "dz_s4": b2.N1 // 32}
    for n, u in zip(names, r1):
        v = getattr(b2, n)
        if n in rows:     # rows [0, mp) of the copies (tiled scales: 32-row tiles)
            u, v = u[:mp * rows[n]], v[:mp * rows[n]]
        assert torch.equal(u, v), n


def test_permute_write_mx4_bit_exact():
    """moe_permute WRITE_MX4 with and without the bf16 copy: codes and
    scales of the permuted rows (group pad rows encoded as zeros)."""
    wl = make_workload("dsv3", T=1500, H=448, with_weights=False)
    T, k = wl.expert_idx.shape
    M_cap = -(-(T * k + wl.E * 127) // 128) * 128
    rt = om.route(wl.expert_idx, wl.probs, wl.E, 0, M_cap)
    mp = int(rt.padded_offsets[-1])
    xp = om.permute(nu.bf16_to_f64(wl.x), rt.row_src)
    for bf16_copy in (True, False):
        blk = mg.ExpertBlock(wl.E, wl.H, 64, T, k, M_cap=M_cap, prec=mg.PREC_MXFP4,
                             bf16_copies=bf16_copy)
        blk.xp_q4.fill_(0xAB)
        blk.xp_s4.fill_(0xAB)
        blk.route(torch.from_numpy(wl.expert_idx).cuda(), torch.from_numpy(wl.probs).cuda(),
                  dev_bf16(wl.x))
        torch.cuda.synchronize()
        compare_routing(blk, rt)
        assert_mx4_equal(blk.xp_q4, blk.xp_s4, M_cap, wl.H, mp, xp[:mp], "permuted X")
        if bf16_copy:
            valid = rt.row_src >= 0
            np.testing.assert_array_equal(host_bits(blk.xp)[valid],
                                          nu.f64_to_bf16_bits(xp[valid]))
        assert int(blk.err_flag.cpu()[0]) == 0


def test_fused_and_unfused_mxfp4_share_operands():
    """The fused and the unfused MXFP4 layers encode the same permuted rows
    (bit-identical Xp and dYp copies) and compute the same z; from there
    they differ by where the activation reads z (unrounded in the epilogue,
    bf16 in the separate pass), which moves some E2M1 codes of a by a step,
    so their outputs are each checked against their own oracle reading
    (the fused and the unfused parity tests), not against one another."""
    wl = make_workload("tiny", seed=31, E=8, T=768, H=256, I=192)
    M_cap = -(-wl.m_cap() // 128) * 128
    gp, _ = act_of(wl)
    fused = run_gpu_layer(wl, M_cap, prec=mg.PREC_MXFP4, bf16_copies=True)
    unf = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp, M_cap=M_cap,
                         prec=mg.PREC_MXFP4, unfused=True)
    run_gpu_layer(wl, M_cap, block=unf)
    mp = int(fused.padded_offsets[-1].item())
    for n in ("xp_q4", "dyp_q4"):
        assert torch.equal(getattr(fused, n)[:mp * wl.H // 2], getattr(unf, n)[:mp * wl.H // 2]), n
    valid = np.zeros(M_cap, dtype=bool)
    pad, split = fused.padded_offsets.cpu().numpy(), fused.split_sizes.cpu().numpy()
    for e in range(wl.E):
        valid[pad[e]:pad[e] + split[e]] = True
    assert_close(host_f64(fused.z)[valid], host_f64(unf.z)[valid], "z")
