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


# ------------------------------------------------ transposed copies, dW ---
def _unpack(b):
    """Packed E2M1 codes (element 2 i in the low nibble of byte i) -> one
    code per element."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def _decode_T(q, s, n, M_cap):
    """A transposed MXFP4 copy ([n][M_cap / 2] codes, tiled scales with
    R = n, K = M_cap) decoded to float64 [n][M_cap]."""
    codes = _unpack(q.detach().cpu().numpy().reshape(n, M_cap // 2))
    scales = mx_scales_plain(s, n, M_cap)
    return nu.mxfp4_dequantize(codes, scales, axis=1)


def _routed_rows(blk):
    split = blk.split_sizes.cpu().numpy()
    pad = blk.padded_offsets.cpu().numpy()
    valid = np.zeros(blk.M_cap, dtype=bool)
    for e in range(blk.E):
        valid[pad[e]:pad[e] + split[e]] = True
    return valid, split, pad


@pytest.mark.parametrize("case", ["tiny", "gptoss_act", "dsv3_zipf_empty", "srelu"])
def test_fused_mxfp4_transposed_copies_bit_exact(case):
    """The GLU and dGLU epilogues' transposed MXFP4 copies of a and dz
    ([n][M_cap / 2], blocks of 32 rows along M) are the oracle's MXFP4
    encoding of the GPU's own bf16 a and dz (pad rows as zeros), bit for
    bit; the rowwise copies stay so too."""
    kw = dict(CASES[case])
    wl = make_workload(kw.pop("name"), seed=12, **kw)
    M_cap = -(-wl.m_cap() // 128) * 128
    blk = run_gpu_layer(wl, M_cap, prec=mg.PREC_MXFP4, bf16_copies=True)
    assert blk.aT_q4 is not None and blk.dzT_q4 is not None
    valid, _, _ = _routed_rows(blk)
    mp = int(blk.padded_offsets[-1].item())
    for name, src, n in (("a", blk.a, wl.I), ("dz", blk.dz, blk.N1)):
        v = rows_with_pad_zeroed(host_f64(src)[:mp], valid[:mp])
        assert_mx4_equal(getattr(blk, name + "_q4"), getattr(blk, name + "_s4"), M_cap, n, mp,
                         v, f"{name} MXFP4 rowwise")
        codes, scales = nu.mxfp4_quantize(v.T, axis=1)        # [n][mp]
        qT = getattr(blk, name + "T_q4").cpu().numpy().reshape(n, M_cap // 2)[:, :mp // 2]
        sT = mx_scales_plain(getattr(blk, name + "T_s4"), n, M_cap)[:, :mp // 32]
        np.testing.assert_array_equal(sT, scales, err_msg=f"{name} MXFP4 transposed scales")
        np.testing.assert_array_equal(qT, nu.pack_nibbles(codes),
                                      err_msg=f"{name} MXFP4 transposed codes")
    assert int(blk.err_flag.cpu()[0]) == 0


@pytest.mark.parametrize("case", ["tiny", "multi_tile_ragged", "gptoss_act", "dsv3_zipf_empty"])
def test_mxfp4_weight_grads(case):
    """MXFP4 weight gradients (moe_grouped_mlp_wgrad, prec MXFP4) from the
    transposed copies: element by element against the float64 contraction
    of the GPU's own operands decoded (each group's rows, one bf16
    rounding), the Xp and dYp copies bit-exact against the oracle's
    encoding of the permuted rows, and against the independent oracle
    (weight_grads(mx="mxfp4")) by relative L2 error."""
    kw = dict(CASES[case])
    wl = make_workload(kw.pop("name"), seed=14, **kw)
    M_cap = -(-wl.m_cap() // 128) * 128
    gp, _ = act_of(wl)
    blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp, first_expert=wl.first_expert,
                         M_cap=M_cap, prec=mg.PREC_MXFP4, wgrad=True)
    run_gpu_layer(wl, M_cap, block=blk)
    blk.dw1.fill_(float("nan"))
    blk.dw2.fill_(float("nan"))
    blk.weight_grads()
    torch.cuda.synchronize()
    assert int(blk.err_flag.cpu()[0]) == 0
    fw, bw = oracle_layer(wl, M_cap, mx="mxfp4")
    mp = int(fw.rt.padded_offsets[-1])
    H, I, N1 = wl.H, wl.I, blk.N1
    # the quantize passes' copies of Xp and dYp: exact inputs, so bit-exact
    for name, ref, n in (("xp", fw.xp, H), ("dyp", bw.dyp, H)):
        codes, scales = nu.mxfp4_quantize(ref[:mp].T, axis=1)
        qT = getattr(blk, name + "T_q4").cpu().numpy().reshape(n, M_cap // 2)[:, :mp // 2]
        np.testing.assert_array_equal(qT, nu.pack_nibbles(codes), err_msg=name)
        np.testing.assert_array_equal(
            mx_scales_plain(getattr(blk, name + "T_s4"), n, M_cap)[:, :mp // 32], scales,
            err_msg=name)
    D = _decode_T(blk.dzT_q4, blk.dzT_s4, N1, M_cap)
    X = _decode_T(blk.xpT_q4, blk.xpT_s4, H, M_cap)
    Y = _decode_T(blk.dypT_q4, blk.dypT_s4, H, M_cap)
    A = _decode_T(blk.aT_q4, blk.aT_s4, I, M_cap)
    _, split, pad = _routed_rows(blk)
    dw1 = host_f64(blk.dw1)
    dw2 = host_f64(blk.dw2)
    for e in range(wl.E):
        r = slice(int(pad[e]), int(pad[e]) + int(split[e]))
        assert_close(dw1[e], nu.round_bf16(D[:, r] @ X[:, r].T), f"dW1 expert {e}")
        assert_close(dw2[e], nu.round_bf16(Y[:, r] @ A[:, r].T), f"dW2 expert {e}")
    o1, o2 = om.weight_grads(fw, bw, mx="mxfp4")
    gated = wl.act != "srelu"
    # dW1 rows follow dz's interleaved column order; the oracle's are logical
    g1 = np.stack([uninterleave_cols(dw1[e].T, wl.I).T for e in range(wl.E)]) if gated else dw1
    for got, ref, what in ((g1, o1, "dW1"), (dw2, o2, "dW2")):
        l2 = _rel_l2(got, ref)
        assert l2 < 5e-2, f"{what}: relative L2 error {l2:.3e} against the oracle"


def test_mxfp4_recompute_rebuilds_z_bit_for_bit():
    """Activation recompute in MXFP4: z rebuilt by the MXFP4 plain-store GEMM
    from the saved Xp and W1 copies equals the z the fused forward stores,
    and the backward's outputs are those of the block that keeps z."""
    wl = make_workload("tiny", seed=15, E=8, T=1024, H=256, I=256)
    M_cap = -(-wl.m_cap() // 128) * 128
    keep = run_gpu_layer(wl, M_cap, prec=mg.PREC_MXFP4, bf16_copies=False)
    gp, _ = act_of(wl)
    rc = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp, M_cap=M_cap,
                        prec=mg.PREC_MXFP4, recompute=True, bf16_copies=False)
    rc.keep_recomputed_z = True
    run_gpu_layer(wl, M_cap, block=rc)
    valid, _, _ = _routed_rows(keep)
    v = torch.from_numpy(valid).cuda()
    assert torch.equal(rc.z[v], keep.z[v])
    for n in ("out", "dx", "dprobs"):
        assert torch.equal(getattr(rc, n), getattr(keep, n)), n
