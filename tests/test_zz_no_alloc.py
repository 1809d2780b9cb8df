"""moe_grouped_mlp_bwd_noalloc -- the backward for callers that cannot
allocate, whose workspace is the library's fixed per-device scratch array --
through the C ABI, against moe_grouped_mlp_bwd (needs an MI355X).

Two calls in a row on one device, the second on a smaller problem (the
array then holds the first call's partial sums, which nothing may read):
  * bit for bit against moe_grouped_mlp_bwd given a workspace of the
    array's size (the same launch configuration, so the same summation
    order), over every output buffer, including rows no kernel writes;
  * within the bf16 bar (rtol 2e-2 / atol 1e-2) against the block's own
    backward with its full workspace (whose FC1 dgrad may split the K of
    its last round of tiles).
A problem whose dprobs partials do not fit in the array is rejected with
MOE_ERR_UNSUPPORTED before any launch, and leaves the outputs untouched.
"""

import numpy as np
import pytest
import torch

import moe_grouped_mlp_amd as mg
from workloads import make_workload

from .gpu_util import act_of, assert_close, dev_bf16, host_f64, run_gpu_layer

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1   # a bf16 NaN no kernel of finite inputs writes


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    mg.lib()


def _inputs(blk):
    kw = dict(E=blk.E, H=blk.H, I=blk.I, M_cap=blk.M_cap, split_sizes=blk.split_sizes,
              padded_offsets=blk.padded_offsets, probs_p=blk.probs_p, z=blk.z,
              act=blk.act, prec=blk.prec, err_flag=blk.err_flag)
    if blk.mx:
        kw.update(dyp_q=blk.dyp_q, dyp_s=blk.dyp_s, w2t_q=blk.w2t_q, w2t_s=blk.w2t_s,
                  w1t_q=blk.w1t_q, w1t_s=blk.w1t_s)
    else:
        kw.update(dyp=blk.dyp, w2=blk.w2, w1i=blk.w1i)
    return kw


def _outputs(blk):
    """Fresh output buffers of the block's shapes, filled with a sentinel."""
    out = {}
    for name in ("dz", "dprobs_p", "dxp") + (
            ("dz_q", "dz_s", "dzT_q", "dzT_s") if blk.mx else ()):
        ref = getattr(blk, name)
        if ref is None:
            continue
        t = torch.empty_like(ref)
        if t.dtype == torch.bfloat16:
            t.view(torch.int16).fill_(SENTINEL)
        elif t.dtype == torch.float32:
            t.view(torch.int32).fill_(0x7FC00001)
        else:
            t.fill_(0xAB)
        out[name] = t
    return out


def _same_bits(a, b, what):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    elif a.dtype == torch.float32:
        a, b = a.view(torch.int32), b.view(torch.int32)
    assert torch.equal(a, b), f"{what} differs from moe_grouped_mlp_bwd"


CASES = [
    dict(name="tiny", seed=21, E=8, k=2, T=1024, H=640, I=320),    # multi-tile, ragged
    dict(name="dsv3", seed=22, T=700, H=256, I=192),               # smaller, Zipf, empty groups
]


@pytest.mark.parametrize("prec", [mg.PREC_BF16, mg.PREC_MXFP8])
def test_noalloc_backward_matches_the_backward_with_workspace(prec):
    for i, case in enumerate(CASES):
        kw = dict(case)
        wl = make_workload(kw.pop("name"), **kw)
        M_cap = -(-wl.m_cap() // 128) * 128
        gp, _ = act_of(wl)
        blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp, M_cap=M_cap, prec=prec,
                             bf16_copies=True)
        print(f"call {i}: E={wl.E} T={wl.T} H={wl.H} I={wl.I} prec={prec}", flush=True)
        run_gpu_layer(wl, M_cap, block=blk)       # forward + the block's own backward
        assert M_cap * -(-wl.I // 256) * 4 <= mg.NOALLOC_SCRATCH_BYTES
        got, ref = _outputs(blk), _outputs(blk)
        mg.moe_grouped_mlp_bwd_noalloc(**_inputs(blk), **got)
        ws = torch.empty(mg.NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
        mg.moe_grouped_mlp_bwd(**_inputs(blk), **ref, workspace=ws)
        torch.cuda.synchronize()
        assert int(blk.err_flag.cpu()[0]) == 0
        for name in got:
            _same_bits(got[name], ref[name], f"call {i}: {name}")
        # the bar against the block's backward with its full workspace
        valid = (blk.row_src >= 0).cpu().numpy()
        assert_close(host_f64(got["dxp"])[valid], host_f64(blk.dxp)[valid], "dxp")
        assert_close(got["dprobs_p"].cpu().numpy()[valid],
                     blk.dprobs_p.cpu().numpy()[valid], "dprobs_p")
        if got.get("dz") is not None:
            assert_close(host_f64(got["dz"])[valid], host_f64(blk.dz)[valid], "dz")
        del blk, got, ref, ws


def test_noalloc_backward_rejects_problems_past_the_scratch_size():
    """M_cap * ceil(I / 256) fp32 partials past the array's size: rejected
    before any launch (no buffer is touched)."""
    I = 1024
    M_cap = mg.NOALLOC_SCRATCH_BYTES // (4 * (I // 256)) + 128
    dxp = torch.full((8,), 7, dtype=torch.int32, device="cuda")
    with pytest.raises(mg.MoeError) as ei:
        mg.moe_grouped_mlp_bwd_noalloc(E=1, H=256, I=I, M_cap=M_cap, split_sizes=dxp,
                                       padded_offsets=dxp, probs_p=dxp, z=dxp,
                                       dprobs_p=dxp, dxp=dxp, dyp=dxp, w2=dxp, w1i=dxp,
                                       dz=dxp)
    assert ei.value.status == mg.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((dxp == 7).all())
