"""Top-k router (moe_router_topk) against the oracle's router_topk through
the C ABI: expert ids bit-exact (the selection compares the fp32 logits on
both sides), kept probabilities within rtol 1e-5 of the float64 softmax.
The router with the routing metadata in one launch (moe_router_route)
against the oracle's router and routing, and bit for bit against
moe_router_topk + moe_permute(BUILD_MAP)."""

import numpy as np
import pytest
import torch

import moe_grouped_mlp_amd as mg
from oracle import moe as om

pytestmark = pytest.mark.gpu


def _logits(kind, T, E, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal((T, E), dtype=np.float32)
    if kind == "biased":      # per-expert offsets ~ N(0, 2): strong imbalance
        mu = rng.standard_normal(E) * np.sqrt(2.0)
        return (mu[None, :] + rng.standard_normal((T, E))).astype(np.float32)
    if kind == "wide":
        return (rng.standard_normal((T, E)) * 3.0).astype(np.float32)
    if kind == "ties":        # four distinct values: ties everywhere
        return rng.integers(0, 4, size=(T, E)).astype(np.float32)
    raise ValueError(kind)


CASES = [
    ("tiny", "normal", 256, 4, 2),
    ("mixtral", "normal", 8192, 8, 2),
    ("gptoss", "biased", 16384, 128, 4),
    ("dsv3_256", "normal", 4096, 256, 8),
    ("max_experts", "wide", 777, 1024, 8),
    ("ties", "ties", 1000, 64, 8),
    ("k_equals_E", "normal", 33, 6, 6),
    ("one_token", "normal", 1, 16, 1),
]


@pytest.mark.parametrize("name,kind,T,E,k", CASES, ids=[c[0] for c in CASES])
def test_router_parity(name, kind, T, E, k):
    lg = _logits(kind, T, E, seed=sum(map(ord, name)))
    dev = torch.device("cuda")
    idx = torch.full((T, k), -1, dtype=torch.int32, device=dev)
    probs = torch.full((T, k), -1.0, dtype=torch.float32, device=dev)
    mg.moe_router_topk(T=T, E=E, k=k, logits=torch.from_numpy(lg).to(dev),
                       expert_idx=idx, probs=probs)
    torch.cuda.synchronize()
    oi, op = om.router_topk(lg, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_allclose(probs.cpu().numpy().astype(np.float64), op,
                               rtol=1e-5, atol=1e-9)


def test_block_route_logits_matches_host_routing():
    """ExpertBlock.route_logits (device router + routing metadata) gives the
    row map of the oracle's router fed to the oracle's routing."""
    T, E, k = 3000, 32, 4
    lg = _logits("biased", T, E, seed=5)
    blk = mg.ExpertBlock(E, 64, 64, T, k)
    blk.route_logits(torch.from_numpy(lg).cuda())
    torch.cuda.synchronize()
    oi, op = om.router_topk(lg, k)
    rt = om.route(oi, op.astype(np.float32), E, M_cap=blk.M_cap)
    np.testing.assert_array_equal(blk.row_id_map.cpu().numpy(), rt.row_id_map)
    np.testing.assert_array_equal(blk.split_sizes.cpu().numpy(), rt.split_sizes)
    np.testing.assert_array_equal(blk.row_src.cpu().numpy(), rt.row_src)


# ------------------------------------------------- router + routing, fused --
ROUTE_CASES = [
    # name, logits, T, E_total, k, local E, first local expert
    ("mixtral", "normal", 8192, 8, 2, 8, 0),
    ("gptoss", "biased", 16384, 128, 4, 128, 0),
    ("dsv3_share", "normal", 16384, 256, 8, 32, 0),
    ("dsv3_share_mid", "normal", 5000, 256, 8, 32, 96),
    ("max_experts", "wide", 777, 1024, 8, 1024, 0),
    ("ties", "ties", 1000, 64, 8, 64, 0),
    ("k_equals_E", "normal", 33, 6, 6, 6, 0),
    ("one_token", "normal", 1, 16, 1, 16, 0),
    ("partial_last_chunk", "biased", 2049, 16, 2, 12, 2),
]


def _assert_counters_consistent(ws):
    """After a call: the group counters are back at zero and the generation
    equals the arrival counter (what the next call expects)."""
    hdr = ws[:4096].view(torch.int32).cpu().numpy()
    assert hdr[0] == hdr[64] and hdr[0] != 0
    assert not hdr[128:].any()


def _route_buffers(T, k, E, M_cap, fill=-7):
    dev = torch.device("cuda")
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    return dict(expert_idx=torch.full((T, k), fill, **i32),
                probs=torch.full((T, k), float(fill), **f32),
                split_sizes=torch.full((E,), fill, **i32),
                offsets=torch.full((E + 1,), fill, **i32),
                padded_offsets=torch.full((E + 1,), fill, **i32),
                row_id_map=torch.full((T, k), fill, **i32),
                row_src=torch.full((M_cap,), fill, **i32),
                probs_p=torch.full((M_cap,), float(fill), **f32),
                err_flag=torch.zeros(1, **i32))


def _fused(lg_dev, T, E_all, k, E, first, M_cap, ws):
    b = _route_buffers(T, k, E, M_cap)
    mg.moe_router_route(T=T, E_total=E_all, k=k, E=E, first_expert=first, M_cap=M_cap,
                        logits=lg_dev, workspace=ws, **b)
    return b


def _separate(lg_dev, T, E_all, k, E, first, M_cap):
    """moe_router_topk, then moe_permute(BUILD_MAP): four launches."""
    b = _route_buffers(T, k, E, M_cap)
    mg.moe_router_topk(T=T, E=E_all, k=k, logits=lg_dev, expert_idx=b["expert_idx"],
                       probs=b["probs"])
    ws = torch.empty(mg.moe_permute_workspace_size(T, E), dtype=torch.uint8, device="cuda")
    mg.moe_permute(flags=mg.PERMUTE_BUILD_MAP, T=T, k=k, E=E, H=64, M_cap=M_cap,
                   first_expert=first, expert_idx=b["expert_idx"], probs=b["probs"],
                   split_sizes=b["split_sizes"], offsets=b["offsets"],
                   padded_offsets=b["padded_offsets"], row_id_map=b["row_id_map"],
                   row_src=b["row_src"], probs_p=b["probs_p"], err_flag=b["err_flag"],
                   workspace=ws)
    return b


@pytest.mark.parametrize("name,kind,T,E_all,k,E,first", ROUTE_CASES,
                         ids=[c[0] for c in ROUTE_CASES])
def test_router_route_parity(name, kind, T, E_all, k, E, first):
    """moe_router_route (one launch): expert ids bit-exact and probabilities
    within rtol 1e-5 against the oracle's router; split sizes, offsets, row
    map, row sources and permuted probabilities bit-exact against the
    oracle's routing of those ids and the GPU's probabilities; every output
    bit-identical to moe_router_topk + moe_permute(BUILD_MAP)."""
    lg = _logits(kind, T, E_all, seed=sum(map(ord, name)) + 1)
    lg_dev = torch.from_numpy(lg).cuda()
    M_cap = T * k + E * 127
    ws = torch.zeros(mg.moe_router_route_workspace_size(T, E_all, E), dtype=torch.uint8,
                     device="cuda")
    f = _fused(lg_dev, T, E_all, k, E, first, M_cap, ws)
    s = _separate(lg_dev, T, E_all, k, E, first, M_cap)
    torch.cuda.synchronize()
    oi, op = om.router_topk(lg, k)
    np.testing.assert_array_equal(f["expert_idx"].cpu().numpy(), oi)
    np.testing.assert_allclose(f["probs"].cpu().numpy().astype(np.float64), op,
                               rtol=1e-5, atol=1e-9)
    rt = om.route(oi, f["probs"].cpu().numpy(), E, first, M_cap)
    np.testing.assert_array_equal(f["split_sizes"].cpu().numpy(), rt.split_sizes)
    np.testing.assert_array_equal(f["offsets"].cpu().numpy(), rt.offsets)
    np.testing.assert_array_equal(f["padded_offsets"].cpu().numpy(), rt.padded_offsets)
    np.testing.assert_array_equal(f["row_id_map"].cpu().numpy(), rt.row_id_map)
    np.testing.assert_array_equal(f["row_src"].cpu().numpy(), rt.row_src)
    np.testing.assert_array_equal(f["probs_p"].cpu().numpy(), rt.probs_p)
    assert int(f["err_flag"].cpu()[0]) == 0
    for key in f:
        assert torch.equal(f[key], s[key]), f"{key}: fused differs from the four launches"
    _assert_counters_consistent(ws)


def test_router_route_repeated_calls_share_one_workspace():
    """Calls of several sizes in a row on one workspace (sized for the
    largest), and in one captured graph replayed twice: the counters the
    launch leaves at zero serve the next call."""
    dev = torch.device("cuda")
    E_all, k, E = 64, 4, 64
    ws = torch.zeros(mg.moe_router_route_workspace_size(9000, E_all, E), dtype=torch.uint8, device=dev)
    for i, T in enumerate((9000, 300, 9000, 1)):
        lg = _logits("biased", T, E_all, seed=100 + i)
        M_cap = T * k + E * 127
        f = _fused(torch.from_numpy(lg).to(dev), T, E_all, k, E, 0, M_cap, ws)
        torch.cuda.synchronize()
        oi, _ = om.router_topk(lg, k)
        rt = om.route(oi, f["probs"].cpu().numpy(), E, 0, M_cap)
        np.testing.assert_array_equal(f["row_id_map"].cpu().numpy(), rt.row_id_map)
        np.testing.assert_array_equal(f["row_src"].cpu().numpy(), rt.row_src)
        _assert_counters_consistent(ws)
    T = 5000
    lg_dev = torch.from_numpy(_logits("normal", T, E_all, seed=7)).to(dev)
    M_cap = T * k + E * 127
    b = _route_buffers(T, k, E, M_cap)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        mg.moe_router_route(T=T, E_total=E_all, k=k, E=E, M_cap=M_cap, logits=lg_dev,
                            workspace=ws, stream=s, **b)
        torch.cuda.synchronize()
        eager = {key: v.clone() for key, v in b.items()}
        with torch.cuda.graph(g, stream=s, capture_error_mode="global"):
            mg.moe_router_route(T=T, E_total=E_all, k=k, E=E, M_cap=M_cap, logits=lg_dev,
                                workspace=ws, stream=s, **b)
    for _ in range(2):
        for key, v in b.items():
            v.fill_(0 if key == "err_flag" else -3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in b:
            assert torch.equal(b[key], eager[key]), f"{key} differs on a replay"
        _assert_counters_consistent(ws)


def test_router_route_mcap_overflow_flags_and_stays_in_bounds():
    """M_cap below the padded row count: MOE_DEVERR_MCAP_OVERFLOW is set,
    rows past M_cap are dropped (row_id_map -1), every stored row is < M_cap
    and the kept rows agree with the oracle's layout."""
    T, E_all, k, E = 3000, 16, 2, 16
    lg = _logits("biased", T, E_all, seed=3)
    M_cap = 2048
    ws = torch.zeros(mg.moe_router_route_workspace_size(T, E_all, E), dtype=torch.uint8, device="cuda")
    f = _fused(torch.from_numpy(lg).cuda(), T, E_all, k, E, 0, M_cap, ws)
    torch.cuda.synchronize()
    assert int(f["err_flag"].cpu()[0]) & mg.DEVERR_MCAP_OVERFLOW
    oi, _ = om.router_topk(lg, k)
    rt = om.route(oi, f["probs"].cpu().numpy(), E, 0, T * k + E * 127)
    rmap = f["row_id_map"].cpu().numpy()
    full = rt.row_id_map
    np.testing.assert_array_equal(rmap, np.where(full < M_cap, full, -1))
    assert rmap.max() < M_cap
    np.testing.assert_array_equal(f["row_src"].cpu().numpy(), rt.row_src[:M_cap])


def test_graph_step_with_fused_routing_replays_match_eager():
    """The whole layer step with routing from logits in one launch
    (route_logits), FC1+GLU, FC2, combine, backward, captured in one graph
    (global mode) and replayed three times: bit-identical to eager."""
    from workloads import make_workload
    from .gpu_util import dev_bf16
    wl = make_workload("tiny", seed=12, E=8, T=1024, H=256, I=256)
    lg_dev = torch.from_numpy(_logits("normal", wl.T, wl.E, seed=12)).cuda()
    blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k)
    blk.load_weights(dev_bf16(wl.w1), dev_bf16(wl.w2))
    x, dout = dev_bf16(wl.x), dev_bf16(wl.dout)

    def step():
        blk.route_logits(lg_dev, x)
        blk.experts_forward()
        blk.combine(blk.yp, blk.out)
        blk.backward(dout)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    outs = (blk.out, blk.dx, blk.dprobs, blk.expert_idx, blk.probs, blk.row_id_map)
    eager = [t.clone() for t in outs]
    # the step from logits equals the step from the oracle router's ids
    oi, _ = om.router_topk(lg_dev.cpu().numpy(), wl.k)
    np.testing.assert_array_equal(blk.expert_idx.cpu().numpy(), oi)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="global"):
        step()
    for _ in range(3):
        for t in outs:
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outs, eager)):
            assert torch.equal(t, e), f"output {i} differs on a replay"
