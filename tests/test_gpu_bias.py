"""FC1 bias (moe_fwd_args.bias1 / moe_bwd_args.bias1) against the oracle's
bias reading, element by element, through the C ABI: z is stored without
the bias, a, yp, out and the backward's dz, dprobs_p, dxp, dx see it added
to the activation's input (gate and up halves in logical order, one vector
per expert).  A bias takes the general activation instantiation even for
the unclamped SwiGLU, so that case is covered too, in bf16 and MXFP8."""

import numpy as np
import pytest
import torch

import moe_grouped_mlp_amd as mg
from workloads import make_workload

from .gpu_util import compare_layer, oracle_layer, run_gpu_layer
from .test_gpu_mx import compare_layer_mx

pytestmark = pytest.mark.gpu

CASES = {
    "swiglu_free": dict(name="tiny"),
    "multi_tile_ragged": dict(name="tiny", E=8, k=2, T=1024, H=640, I=320),
    "gptoss_act": dict(name="gptoss", T=512, H=128, I=192, E=16),
    "geglu": dict(name="tiny", act="geglu", T=384, I=192),
    "srelu": dict(name="tiny", act="srelu", T=384, I=192),
    "dsv3_zipf_empty": dict(name="dsv3", T=2000, H=256, I=128),
}


def _bias(wl, seed):
    n1 = wl.I if wl.act == "srelu" else 2 * wl.I
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((wl.E, n1)) * 0.5).astype(np.float32)


@pytest.mark.parametrize("case", list(CASES))
def test_layer_with_bias_parity(case):
    kw = dict(CASES[case])
    wl = make_workload(kw.pop("name"), seed=7, **kw)
    M_cap = wl.m_cap()
    bias = _bias(wl, 70)
    blk = run_gpu_layer(wl, M_cap, bias1=bias)
    fw, bw = oracle_layer(wl, M_cap, bias1=bias)
    compare_layer(blk, wl, fw, bw)
    assert int(blk.err_flag.cpu()[0]) == 0


@pytest.mark.parametrize("case", ["swiglu_free", "gptoss_act", "srelu", "dsv3_zipf_empty"])
def test_layer_with_bias_mx_parity(case):
    kw = dict(CASES[case])
    wl = make_workload(kw.pop("name"), seed=8, **kw)
    M_cap = -(-wl.m_cap() // 128) * 128
    bias = _bias(wl, 80)
    blk = run_gpu_layer(wl, M_cap, prec=mg.PREC_MXFP8, bias1=bias)
    fw, bw = oracle_layer(wl, M_cap, mx=True, bias1=bias)
    compare_layer_mx(blk, wl, fw, bw)
    assert int(blk.err_flag.cpu()[0]) == 0


def test_bias_changes_the_outputs():
    """The bias is really applied: a with a large bias differs from a
    without it on most outputs, and z does not change."""
    wl = make_workload("tiny", seed=9)
    M_cap = wl.m_cap()
    plain = run_gpu_layer(wl, M_cap, backward=False)
    a0, z0 = plain.a.clone(), plain.z.clone()
    biased = run_gpu_layer(wl, M_cap, backward=False, bias1=_bias(wl, 90) * 4)
    rows = (plain.row_src[:M_cap] >= 0).nonzero().squeeze(1)
    assert torch.equal(biased.z[rows], z0[rows])
    assert (biased.a[rows] != a0[rows]).float().mean().item() > 0.9
