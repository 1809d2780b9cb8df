"""The unfused baseline (moe_grouped_gemm + moe_glu_unfused: the layer without
the fused epilogues) against the oracle's unfused reading, through the C
ABI: every stored tensor of the step within the bf16 tolerances.  Unfused,
each kernel reads what the one before stored: the activation takes the bf16
z, the activation gradient the bf16 dA (the fused epilogues take FC1's and
FC2 dgrad's unrounded results)."""

import numpy as np
import pytest
import torch

import moe_grouped_mlp_amd as mg
from workloads import make_workload

from .gpu_util import act_of, compare_layer, dev_bf16, oracle_layer

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": dict(name="tiny"),
    "multi_tile_ragged": dict(name="tiny", E=8, k=2, T=1024, H=640, I=320),
    "gptoss_act": dict(name="gptoss", T=512, H=128, I=192, E=16),
    "geglu": dict(name="tiny", act="geglu", T=384, I=192),
    "srelu": dict(name="tiny", act="srelu", T=384, I=192),
    "dsv3_zipf_empty": dict(name="dsv3", T=2000, H=256, I=128),
}


@pytest.mark.parametrize("case", list(CASES))
def test_unfused_layer_parity(case):
    kw = dict(CASES[case])
    wl = make_workload(kw.pop("name"), seed=3, **kw)
    M_cap = wl.m_cap()
    gp, _ = act_of(wl)
    blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp, M_cap=M_cap)
    blk.load_weights(dev_bf16(wl.w1), dev_bf16(wl.w2))
    blk.route(torch.from_numpy(wl.expert_idx).cuda(),
              torch.from_numpy(wl.probs).cuda(), dev_bf16(wl.x))
    blk.experts_forward_unfused()
    blk.combine(blk.yp, blk.out)
    blk.gather(dev_bf16(wl.dout), blk.dyp)
    blk.experts_backward_unfused()
    blk.combine(blk.dxp, blk.dx, dprobs=True)
    torch.cuda.synchronize()
    fw, bw = oracle_layer(wl, M_cap, unfused=True)
    compare_layer(blk, wl, fw, bw)


@pytest.mark.parametrize("case", ["multi_tile_ragged", "gptoss_act", "dsv3_zipf_empty"])
def test_unfused_layer_mx_parity(case):
    """MXFP8: plain MXFP8 grouped GEMMs, the activation passes and
    moe_quantize_mxfp8 for the rowwise and transposed copies of a and dz,
    against the oracle's MXFP8 unfused reading (MXFP8 bounds)."""
    from .test_gpu_mx import compare_layer_mx
    kw = dict(CASES[case])
    wl = make_workload(kw.pop("name"), seed=4, **kw)
    M_cap = -(-wl.m_cap() // 128) * 128
    gp, _ = act_of(wl)
    blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp, M_cap=M_cap,
                         prec=mg.PREC_MXFP8, bf16_copies=True)
    blk.load_weights(dev_bf16(wl.w1), dev_bf16(wl.w2))
    blk.route(torch.from_numpy(wl.expert_idx).cuda(),
              torch.from_numpy(wl.probs).cuda(), dev_bf16(wl.x))
    blk.experts_forward_unfused()
    blk.combine(blk.yp, blk.out)
    blk.gather(dev_bf16(wl.dout), None, blk.dyp_q, blk.dyp_s)
    blk.experts_backward_unfused()
    blk.combine(blk.dxp, blk.dx, dprobs=True)
    torch.cuda.synchronize()
    fw, bw = oracle_layer(wl, M_cap, mx=True, unfused=True)
    compare_layer_mx(blk, wl, fw, bw)
