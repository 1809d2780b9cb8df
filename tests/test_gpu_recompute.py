"""Activation recompute through the C ABI: a forward with z = NULL stores no
z, and the backward rebuilds it with moe_grouped_gemm (FC1's GEMM, no
workspace, so no split-K).  Every tile then sums K in FC1's order, so the
rebuilt z and every output of the step must equal, bit for bit, those of
the block that keeps z; that block is held to the oracle by the layer
parity tests, and one case here checks the recompute block against the
oracle directly."""

import numpy as np
import pytest
import torch

import moe_grouped_mlp_amd as mg
from workloads import make_workload

from .gpu_util import (act_of, compare_layer, dev_bf16, gemm_grid, oracle_layer,
                       run_gpu_layer, tail_split_parts)

pytestmark = pytest.mark.gpu

CASES = {
    "multi_tile_ragged": dict(name="tiny", E=8, k=2, T=1024, H=640, I=320),
    "gptoss_act": dict(name="gptoss", T=512, H=128, I=192, E=16),
    "dsv3_zipf_empty": dict(name="dsv3", T=2000, H=256, I=128),
    "srelu": dict(name="tiny", act="srelu", T=384, I=192),
    # 8 workgroups: with a workspace the plain GEMM would split the K of
    # this FC1 shape's last round, and a rebuilt z would sum in another order
    "split_shape_8wg": dict(name="tiny", seed=13, E=4, k=2, T=1536, H=512, I=512,
                            grid8=True),
}
SENTINEL = 0x7FC1  # a bf16 NaN no GEMM of finite inputs produces


def _valid_rows(blk):
    split = blk.split_sizes.cpu().numpy()
    pad = blk.padded_offsets.cpu().numpy()
    rows = np.zeros(blk.M_cap, dtype=bool)
    for e in range(blk.E):
        rows[pad[e]:pad[e] + split[e]] = True
    return torch.from_numpy(rows).cuda()


MX_COPIES = ("a_q", "a_s", "aT_q", "aT_s", "dz_q", "dz_s", "dzT_q", "dzT_s")


def _block(wl, M_cap, prec, margin, recompute):
    gp, _ = act_of(wl)
    blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp,
                         first_expert=wl.first_expert, M_cap=M_cap, prec=prec,
                         cu_margin=margin, bf16_copies=True, recompute=recompute)
    # rows past the last group are never written: start both blocks equal
    for n in MX_COPIES:
        t = getattr(blk, n, None)
        if t is not None:
            t.zero_()
    return blk


def _run_recompute(wl, M_cap, prec, margin=0):
    blk = _block(wl, M_cap, prec, margin, True)
    # z lives in a caller's scratch buffer during the backward; the test
    # keeps it afterwards to compare it
    n1 = 2 * wl.I if wl.act != "srelu" else wl.I
    scratch = torch.empty(M_cap * n1, dtype=torch.bfloat16, device="cuda")
    scratch.view(torch.int16).fill_(SENTINEL)
    blk._z_scratch = scratch
    blk.keep_recomputed_z = True
    blk.load_weights(dev_bf16(wl.w1), dev_bf16(wl.w2))
    idx = torch.from_numpy(wl.expert_idx.astype(np.int32)).cuda()
    probs = torch.from_numpy(wl.probs.astype(np.float32)).cuda()
    blk.forward(dev_bf16(wl.x), idx, probs)
    torch.cuda.synchronize()
    # the forward kept no z
    assert blk.z is None
    assert bool((scratch.view(torch.int16) == SENTINEL).all())
    blk.backward(dev_bf16(wl.dout))
    torch.cuda.synchronize()
    return blk


def _assert_same(rc, ref, names, rows=None):
    for n in names:
        a, b = getattr(rc, n), getattr(ref, n)
        if a is None:
            continue
        if rows is not None:
            a, b = a[rows], b[rows]
        a = a.view(torch.int16) if a.dtype == torch.bfloat16 else a
        b = b.view(torch.int16) if b.dtype == torch.bfloat16 else b
        assert torch.equal(a, b), f"{n} differs from the path that keeps z"


@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
@pytest.mark.parametrize("case", list(CASES))
def test_recompute_bit_identical(case, prec):
    kw = dict(CASES[case])
    grid8 = kw.pop("grid8", False)
    wl = make_workload(kw.pop("name"), seed=kw.pop("seed", 5), **kw)
    mx = prec == "mxfp8"
    M_cap = wl.m_cap()
    if mx:
        M_cap = -(-M_cap // 128) * 128
    p = mg.PREC_MXFP8 if mx else mg.PREC_BF16
    margin = 0
    if grid8:
        margin = torch.cuda.get_device_properties(0).multi_processor_count - 8
        n1 = 2 * wl.I
        assert gemm_grid(margin, M_cap, wl.E, n1) == 8
        sizes = [int((wl.expert_idx == e).sum()) for e in range(wl.E)]
        if not mx:   # (MXFP8 plain GEMMs never split)
            assert tail_split_parts(sizes, n1, wl.H, 8, 64) > 1
    ref = run_gpu_layer(wl, M_cap=M_cap, block=_block(wl, M_cap, p, margin, False))
    rc = _run_recompute(wl, M_cap, p, margin)
    rows = _valid_rows(ref)
    assert torch.equal(rows, _valid_rows(rc))
    _assert_same(rc, ref, ("z", "xp", "a", "yp", "dyp", "dz", "dxp"), rows)
    _assert_same(rc, ref, ("out", "dx", "dprobs", "dprobs_p", "amax"))
    if mx:
        _assert_same(rc, ref, MX_COPIES)


def test_recompute_oracle_parity():
    wl = make_workload("tiny", seed=6, E=8, k=2, T=1024, H=640, I=320)
    M_cap = wl.m_cap()
    rc = _run_recompute(wl, M_cap, mg.PREC_BF16)
    fw, bw = oracle_layer(wl, M_cap)
    compare_layer(rc, wl, fw, bw)


def test_recompute_z_repeatable():
    """recompute_z gives the same z again, and a second backward on it the
    same dX."""
    wl = make_workload("tiny", seed=7, E=4, k=2, T=300, H=256, I=192)
    M_cap = wl.m_cap()
    rc = _run_recompute(wl, M_cap, mg.PREC_BF16)
    rows = _valid_rows(rc)
    z1 = rc.z[rows].clone()
    dx1 = rc.dx.clone()
    rc.recompute_z()
    rc.backward(dev_bf16(wl.dout))
    torch.cuda.synchronize()
    assert torch.equal(rc.z[rows].view(torch.int16), z1.view(torch.int16))
    assert torch.equal(rc.dx.view(torch.int16), dx1.view(torch.int16))


def test_recompute_holds_no_z_between_forward_and_backward():
    """The recompute block allocates no z: between its forward and its
    backward it holds M_cap * N1 bf16 elements less than the block that
    keeps z, and the z it rebuilds in the backward is released at the end."""
    wl = make_workload("tiny", seed=8, E=4, k=2, T=512, H=256, I=256)
    M_cap = wl.m_cap()
    gp, _ = act_of(wl)
    z_bytes = M_cap * 2 * wl.I * 2
    torch.cuda.synchronize()
    m0 = torch.cuda.memory_allocated()
    rc = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp, M_cap=M_cap, recompute=True)
    m1 = torch.cuda.memory_allocated()
    keep = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp, M_cap=M_cap)
    m2 = torch.cuda.memory_allocated()
    assert (m2 - m1) - (m1 - m0) >= z_bytes
    for blk in (rc, keep):
        blk.load_weights(dev_bf16(wl.w1), dev_bf16(wl.w2))
    idx = torch.from_numpy(wl.expert_idx.astype(np.int32)).cuda()
    probs = torch.from_numpy(wl.probs.astype(np.float32)).cuda()
    x, dout = dev_bf16(wl.x), dev_bf16(wl.dout)
    rc.forward(x, idx, probs)
    keep.forward(x, idx, probs)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    rc.backward(dout)
    keep.backward(dout)
    torch.cuda.synchronize()
    assert rc.z is None
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(rc.dx.view(torch.int16), keep.dx.view(torch.int16))
