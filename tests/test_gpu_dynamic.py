"""Dynamic tile scheduling of the grouped GEMMs (per-XCD work counters in
the workspace): results are bit-identical to the static walk, because each
tile's K sum runs in one fixed order whichever workgroup takes it; this
holds for the plain GEMM on skewed groups over many rounds (with its split
last round), for the fused forward and backward, and while another kernel
holds a quarter of the CUs for the first part of the GEMM."""

import numpy as np
import pytest
import torch

import moe_grouped_mlp_amd as mg
from workloads import make_workload

from .gpu_util import dev_bf16, run_gpu_layer

pytestmark = pytest.mark.gpu


def _gemm_case(dev, seed=2):
    wl = make_workload("gptoss", T=3000, H=512, I=640, E=16, with_weights=False, seed=seed)
    sizes = wl.group_sizes().tolist()
    pad = [0]
    for n in sizes:
        pad.append(pad[-1] + -(-n // mg.GROUP_ALIGN) * mg.GROUP_ALIGN)
    E, N, K, M_cap = len(sizes), 512, 640, pad[-1]
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    a = torch.randn(M_cap, K, generator=g, device=dev).to(torch.bfloat16)
    b = (torch.randn(E, N, K, generator=g, device=dev) * 0.05).to(torch.bfloat16)
    args = dict(E=E, N=N, K=K, M_cap=M_cap,
                split_sizes=torch.tensor(sizes, dtype=torch.int32, device=dev),
                padded_offsets=torch.tensor(pad, dtype=torch.int32, device=dev), a=a, b=b)
    rows = torch.cat([torch.arange(p, p + n) for p, n in zip(pad, sizes)]).to(dev)
    return args, rows


def _ws(dynamic, dev):
    n = mg.moe_grouped_gemm_workspace_size(dynamic)
    return torch.zeros(n, dtype=torch.uint8, device=dev)


def test_plain_gemm_dynamic_equals_static():
    dev = torch.device("cuda:0")
    args, rows = _gemm_case(dev)
    outs = {}
    for dyn in (False, True):
        c = torch.full((args["M_cap"], args["N"]), 3.0, dtype=torch.bfloat16, device=dev)
        for _ in range(2):      # the counters are zeroed by each call
            mg.moe_grouped_gemm(c=c, workspace=_ws(dyn, dev), **args)
        torch.cuda.synchronize()
        outs[dyn] = c
    assert torch.equal(outs[True][rows], outs[False][rows])
    ref = args["a"][rows].float() @ args["b"][0].float().T   # shape check only
    assert ref.shape[0] == rows.numel()


def test_plain_gemm_dynamic_beside_a_busy_kernel():
    """A kernel holds 64 CUs for ~2 ms while the GEMM starts: the GEMM's
    results equal those of an isolated run."""
    dev = torch.device("cuda:0")
    args, rows = _gemm_case(dev, seed=5)
    ws = _ws(True, dev)
    ref = torch.empty((args["M_cap"], args["N"]), dtype=torch.bfloat16, device=dev)
    mg.moe_grouped_gemm(c=ref, workspace=ws, **args)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    rate = mg.moe_clock_tick_rate_hz()
    c = torch.empty_like(ref)
    with torch.cuda.stream(side):
        mg.moe_bench_occupy(workgroups=64, ticks=max(1, int(rate * 2e-3)))
    mg.moe_grouped_gemm(c=c, workspace=ws, **args)
    torch.cuda.synchronize()
    assert torch.equal(c[rows], ref[rows])


def test_fused_layer_dynamic_equals_static():
    """The same step with the full workspace (work counters) and with one
    just short of them (static walk, same split-K): every stored output is
    bit-identical."""
    wl = make_workload("gptoss", T=2048, H=256, I=384, E=16, seed=6)
    M_cap = wl.m_cap()
    blk = run_gpu_layer(wl, M_cap)
    full = blk.ws
    names = ("z", "a", "yp", "out", "dz", "dprobs_p", "dxp", "dx", "dprobs")
    dyn = {n: getattr(blk, n).clone() for n in names}
    blk.ws = full[: full.numel() - 2 * 8 * 64]
    try:
        run_gpu_layer(wl, M_cap, block=blk)
    finally:
        blk.ws = full
    # row-indexed outputs on the routed rows (pad rows are never written and
    # hold whatever the allocation held); token-indexed ones whole
    rows = (blk.row_src[:M_cap] >= 0).nonzero().squeeze(1)
    for n in names:
        x, y = getattr(blk, n), dyn[n]
        if n not in ("out", "dx", "dprobs"):
            x, y = x[rows], y[rows]
        assert torch.equal(x, y), n


def test_bench_occupy_rejects_bad_sizes():
    for w, t in ((0, 10), (1025, 10), (1, 0)):
        with pytest.raises(mg.MoeError) as ei:
            mg.moe_bench_occupy(workgroups=w, ticks=t)
        assert ei.value.status == mg.ERR_INVALID_ARG
