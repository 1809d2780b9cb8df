"""GEMM clock trace (moe_gemm_clock_trace) through the C ABI: while it is
set, each grouped-GEMM launch takes the next record area in turn and its
persistent workgroups write {shader cycles, constant-rate ticks}; the
derived clock lies between the card's idle floor and its 2.4 GHz maximum
(with margin); areas past the launch's workgroups stay untouched; clearing
the trace stops the writes; the GEMM's output does not change."""

import numpy as np
import pytest
import torch

import moe_grouped_mlp_amd as mg

pytestmark = pytest.mark.gpu

W = mg.CLOCK_MAX_WORKGROUPS


def _gemm_inputs(dev):
    sizes = [300, 0, 517, 1024]
    pad = [0]
    for n in sizes:
        pad.append(pad[-1] + -(-n // mg.GROUP_ALIGN) * mg.GROUP_ALIGN)
    E, N, K, M_cap = len(sizes), 512, 1024, pad[-1]
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    a = torch.randn(M_cap, K, generator=g, device=dev).to(torch.bfloat16)
    b = (torch.randn(E, N, K, generator=g, device=dev) * 0.05).to(torch.bfloat16)
    split = torch.tensor(sizes, dtype=torch.int32, device=dev)
    padded = torch.tensor(pad, dtype=torch.int32, device=dev)
    return dict(E=E, N=N, K=K, M_cap=M_cap, split_sizes=split, padded_offsets=padded, a=a, b=b)


def _clock_ghz(rec, rate):
    ok = (rec[:, 0] > 0) & (rec[:, 1] > 0)
    return rec[ok, 0] / (rec[ok, 1] / rate) / 1e9, int(ok.sum())


def test_gemm_clock_trace_records_and_clears():
    dev = torch.device("cuda:0")
    args = _gemm_inputs(dev)
    ref = torch.empty(args["M_cap"], args["N"], dtype=torch.bfloat16, device=dev)
    mg.moe_grouped_gemm(c=ref, **args)
    rate = mg.moe_clock_tick_rate_hz()
    assert rate > 0
    buf = torch.zeros(3, W, 2, dtype=torch.int64, device=dev)
    outs = [torch.empty_like(ref) for _ in range(2)]
    mg.moe_gemm_clock_trace(buf, 2)
    try:
        for o in outs:
            mg.moe_grouped_gemm(c=o, **args)
        torch.cuda.synchronize()
    finally:
        mg.moe_gemm_clock_trace(None)
    sizes = args["split_sizes"].cpu().tolist()
    pad = args["padded_offsets"].cpu().tolist()
    rows = torch.cat([torch.arange(p, p + n) for p, n in zip(pad, sizes)]).to(dev)
    for o in outs:   # the trace does not touch results (the group rows)
        assert torch.equal(o[rows], ref[rows])
    h = buf.cpu().numpy()
    assert not h[2].any(), "only the set areas are written"
    cu = torch.cuda.get_device_properties(dev).multi_processor_count
    for j in range(2):
        ghz, n = _clock_ghz(h[j], rate)
        assert 1 <= n <= cu, n
        assert not h[j, n:].any(), "records past the launch's workgroups"
        print(f"launch {j}: {n} workgroups, clock {ghz.mean():.3f} GHz "
              f"(min {ghz.min():.3f}, max {ghz.max():.3f})")
        assert (ghz > 0.3).all() and (ghz < 3.0).all(), ghz
    # cleared: nothing more is written
    buf.zero_()
    mg.moe_grouped_gemm(c=outs[0], **args)
    torch.cuda.synchronize()
    assert not buf.any()


def test_gemm_clock_trace_rejects_bad_slots():
    dev = torch.device("cuda:0")
    buf = torch.zeros(1, W, 2, dtype=torch.int64, device=dev)
    for slots in (0, -1, 65):
        with pytest.raises(mg.MoeError) as ei:
            mg.moe_gemm_clock_trace(buf, slots)
        assert ei.value.status == mg.ERR_INVALID_ARG
    mg.moe_gemm_clock_trace(None)
