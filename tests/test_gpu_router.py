"""Top-k router (moe_router_topk) against the oracle's router_topk through
the C ABI: expert ids bit-exact (the selection compares the fp32 logits on
both sides), kept probabilities within rtol 1e-5 of the float64 softmax."""

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
