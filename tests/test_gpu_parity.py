"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Routing, permutation and repack results must be bit-exact; bf16 tensors
must be within rtol 2e-2 / atol 1e-2 of the fp64 oracle (plus the
scale-aware check of gpu_util.assert_close).  Every call goes through the
C ABI (moe_grouped_mlp_amd.binding).
"""

import numpy as np
import pytest
import torch

import moe_grouped_mlp_amd as mg
from oracle import moe as om
from oracle import numerics as nu
from workloads import make_workload

from .gpu_util import (act_of, compare_layer, compare_routing, dev_bf16,
                       gemm_grid, host_bits, oracle_layer, run_gpu_layer,
                       tail_split_parts)

pytestmark = pytest.mark.gpu


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    mg.lib()  # fail loudly if the HIP library is not built


# ----------------------------------------------------------------- repack --
@pytest.mark.parametrize("E,I,H", [(3, 128, 96), (2, 2880, 64), (1, 64, 8)])
def test_repack_bit_exact(E, I, H):
    rng = np.random.default_rng(E * I + H)
    w = rng.integers(0, 2 ** 16, size=(E, 2 * I, H), dtype=np.uint16)
    src = dev_bf16(w)
    dst = torch.empty_like(src)
    mg.moe_weight_repack_interleave(src, dst, E, I, H)
    back = torch.empty_like(src)
    mg.moe_weight_repack_interleave(dst, back, E, I, H, inverse=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(dst), om.repack_interleave(w))
    np.testing.assert_array_equal(host_bits(back), w)


# ---------------------------------------------------------- route/permute --
def _routing_case(name):
    rng = np.random.default_rng(len(name))
    if name == "tiny":
        wl = make_workload("tiny", with_weights=False)
        return wl.expert_idx, wl.probs, wl.E, 0, wl.x
    if name == "gptoss_skew":
        wl = make_workload("gptoss", T=2048, H=64, with_weights=False)
        return wl.expert_idx, wl.probs, wl.E, 0, wl.x
    if name == "dsv3_zipf":
        wl = make_workload("dsv3", T=3000, H=64, with_weights=False)
        return wl.expert_idx, wl.probs, wl.E, 0, wl.x
    if name == "nonlocal":
        T, k = 300, 3
        idx = np.stack([rng.permutation(9)[:k] for _ in range(T)]).astype(np.int32)
        idx[5] = [7, 8, 0]                      # token with no local expert
        return idx, rng.random((T, k)).astype(np.float32), 3, 2, \
            rng.integers(0, 2 ** 16, (T, 32), dtype=np.uint16)
    if name == "one_token":
        return np.array([[2, 0]], np.int32), np.array([[0.6, 0.4]], np.float32), \
            4, 0, rng.integers(0, 2 ** 16, (1, 64), dtype=np.uint16)
    if name == "all_one_expert":
        T = 1000
        return np.zeros((T, 1), np.int32), rng.random((T, 1)).astype(np.float32), \
            4, 0, rng.integers(0, 2 ** 16, (T, 16), dtype=np.uint16)
    if name == "wide_ranks":
        # > 64 tokens per wave share experts; 8 slots; many chunks
        T, k, E = 5000, 8, 16
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        return idx, rng.random((T, k)).astype(np.float32), E, 0, \
            rng.integers(0, 2 ** 16, (T, 8), dtype=np.uint16)
    raise KeyError(name)


@pytest.mark.parametrize("case", ["tiny", "gptoss_skew", "dsv3_zipf", "nonlocal",
                                  "one_token", "all_one_expert", "wide_ranks"])
@pytest.mark.parametrize("tight", [False, True])
def test_route_and_permute_bit_exact(case, tight):
    idx, probs, E, first, x = _routing_case(case)
    T, k = idx.shape
    H = x.shape[1]
    rt_full = om.route(idx, probs, E, first)
    M_cap = int(rt_full.padded_offsets[-1]) if tight else T * k + E * 127 + 3
    M_cap = max(M_cap, 1)
    rt = om.route(idx, probs, E, first, M_cap)
    blk = mg.ExpertBlock(E, 64, 64, T, k, first_expert=first, M_cap=M_cap)
    blk.H = H
    blk.xp = torch.full((M_cap, H), -1.0, dtype=torch.bfloat16, device="cuda")
    blk.route(torch.from_numpy(idx).cuda(), torch.from_numpy(probs).cuda(),
              dev_bf16(x))
    torch.cuda.synchronize()
    compare_routing(blk, rt)
    mp = int(rt.padded_offsets[-1])
    xp = om.permute(x, rt.row_src)
    np.testing.assert_array_equal(host_bits(blk.xp)[:mp], xp[:mp])
    assert int(blk.err_flag.cpu()[0]) == 0


def test_route_flags_mcap_overflow_and_duplicates():
    idx = np.array([[0, 1], [1, 1], [2, 0]], np.int32)      # token 1 lists 1 twice
    probs = np.ones((3, 2), np.float32)
    blk = mg.ExpertBlock(4, 64, 64, 3, 2, M_cap=200)          # needs 3*128 rows
    blk.H = 8
    blk.xp = torch.zeros(200, 8, dtype=torch.bfloat16, device="cuda")
    blk.route(torch.from_numpy(idx).cuda(), torch.from_numpy(probs).cuda(),
              dev_bf16(np.ones((3, 8), np.uint16)))
    torch.cuda.synchronize()
    flag = int(blk.err_flag.cpu()[0])
    assert flag & 0x1 and flag & 0x2
    rmap = blk.row_id_map.cpu().numpy()
    assert np.all(rmap < 200)                                # nothing past M_cap


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_unpermute_of_permute_is_k_times_x(k):
    T, E, H = 777, 8, 192
    rng = np.random.default_rng(k)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = nu.f64_to_bf16_bits(nu.round_bf16(rng.standard_normal((T, H))))
    blk = mg.ExpertBlock(E, H, 64, T, k)
    blk.route(torch.from_numpy(idx).cuda(),
              torch.ones(T, k, device="cuda"), dev_bf16(x))
    blk.combine(blk.xp, blk.out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(nu.bf16_to_f64(host_bits(blk.out)),
                                  k * nu.bf16_to_f64(x))


# ------------------------------------------------------------- full layer --
LAYER_CASES = {
    "tiny": dict(name="tiny"),
    "multi_tile_ragged": dict(name="tiny", E=8, k=2, T=1024, H=640, I=320),
    # GPT-OSS activation (Swish slope 1.702, clamp +-7) at realistic scale
    "gptoss_act": dict(name="gptoss", T=512, H=128, I=192, E=16),
    # same code path with a clamp that binds often at this scale
    "clamp_binding": dict(name="gptoss", T=512, H=128, I=192, E=16, clamp=0.25),
    "geglu": dict(name="tiny", act="geglu", T=384, I=192),
    "srelu": dict(name="tiny", act="srelu", T=384, I=192),
    "dsv3_zipf_empty": dict(name="dsv3", T=2000, H=256, I=128),
}


@pytest.mark.parametrize("case", list(LAYER_CASES))
def test_layer_forward_backward_parity(case):
    kw = dict(LAYER_CASES[case])
    wl = make_workload(kw.pop("name"), seed=3, **kw)
    M_cap = wl.m_cap()
    blk = run_gpu_layer(wl, M_cap)
    fw, bw = oracle_layer(wl, M_cap)
    if case == "clamp_binding":
        # the clamp must bind on a good share of the FC1 outputs
        assert np.mean(np.abs(fw.z[fw.expert >= 0]) > 0.25) > 0.1
    if case == "dsv3_zipf_empty":
        assert fw.rt.split_sizes[0] == 0 and fw.rt.split_sizes[-1] == 0
    compare_layer(blk, wl, fw, bw)
    assert int(blk.err_flag.cpu()[0]) == 0


def test_layer_one_sided_clamp_and_linear_offset():
    """The other reading of the clamping option, at this scale's magnitudes:
    the gate half clamped from above only (at 0.15) and the linear half
    clamped to [-0.25, 0.25] with +1 added after the clamp (Swish slope
    1.702).  A linear offset takes the general SwiGLU kernel, not the
    unclamped one."""
    wl = make_workload("gptoss", seed=21, T=512, H=128, I=192, E=16)
    M_cap = wl.m_cap()
    kw = dict(gate_lo=-np.inf, gate_hi=0.15, lin_lo=-0.25, lin_hi=0.25, lin_offset=1.0)
    gp = mg.act_params(mg.ACT_SWIGLU, beta=wl.beta, **kw)
    op = om.ActParams(act="swiglu", beta=wl.beta, **kw)
    blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp, M_cap=M_cap)
    run_gpu_layer(wl, M_cap, block=blk)
    fw = om.forward(wl.x, wl.w1, wl.w2, wl.expert_idx, wl.probs, wl.E, op, M_cap=M_cap)
    bw = om.backward(fw, wl.dout, wl.w1, wl.w2, op)
    # both bounds bind on a good share of the FC1 outputs at this scale
    zv = fw.z[fw.expert >= 0]
    assert np.mean(zv[:, :wl.I] > 0.15) > 0.1
    assert np.mean(np.abs(zv[:, wl.I:]) > 0.25) > 0.1
    compare_layer(blk, wl, fw, bw)
    assert int(blk.err_flag.cpu()[0]) == 0


def test_layer_all_tokens_one_expert_and_empty_groups():
    wl = make_workload("tiny", seed=5, T=700)
    wl.expert_idx[:, 0] = 2
    wl.expert_idx[:, 1] = 1          # experts 0 and 3 empty, 1 and 2 full
    M_cap = wl.m_cap()
    blk = run_gpu_layer(wl, M_cap)
    fw, bw = oracle_layer(wl, M_cap)
    assert list(fw.rt.split_sizes) == [0, 700, 700, 0]
    compare_layer(blk, wl, fw, bw)


def test_layer_split_k_tail_parity():
    """A grid of 8 workgroups over 26 output tiles: FC2 and FC1 dgrad run
    three whole rounds, then split the last two tiles along K (partial tiles
    in the workspace, summed by the part that arrives last).  Results must
    match the oracle and repeat bit for bit."""
    wl = make_workload("tiny", seed=13, E=4, k=2, T=1536, H=512, I=512)
    M_cap = wl.m_cap()
    margin = torch.cuda.get_device_properties(0).multi_processor_count - 8
    G = gemm_grid(margin, M_cap, wl.E, wl.H)
    sizes = [int((wl.expert_idx == e).sum()) for e in range(wl.E)]
    assert G == 8
    assert tail_split_parts(sizes, wl.H, wl.I, G, 64) > 1          # FC2
    assert tail_split_parts(sizes, wl.H, 2 * wl.I, G, 64) > 1      # FC1 dgrad
    gp, _ = act_of(wl)
    blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp, M_cap=M_cap,
                         cu_margin=margin)
    run_gpu_layer(wl, M_cap, block=blk)
    r1 = [host_bits(t).copy() for t in (blk.yp, blk.dxp)]
    fw, bw = oracle_layer(wl, M_cap)
    compare_layer(blk, wl, fw, bw)
    run_gpu_layer(wl, M_cap, block=blk)
    for u, t in zip(r1, (blk.yp, blk.dxp)):
        np.testing.assert_array_equal(u, host_bits(t))
    assert int(blk.err_flag.cpu()[0]) == 0


def test_layer_is_deterministic():
    wl = make_workload("tiny", seed=7, E=8, T=1500, H=256, I=256)
    b1 = run_gpu_layer(wl)
    r1 = [host_bits(t).copy() for t in (b1.z, b1.a, b1.yp, b1.out, b1.dz,
                                        b1.dxp, b1.dx)]
    d1 = b1.dprobs.cpu().numpy().copy()
    b2 = run_gpu_layer(wl, block=b1)
    r2 = [host_bits(t) for t in (b2.z, b2.a, b2.yp, b2.out, b2.dz, b2.dxp, b2.dx)]
    for u, v in zip(r1, r2):
        np.testing.assert_array_equal(u, v)
    np.testing.assert_array_equal(d1, b2.dprobs.cpu().numpy())


def test_graph_capture_replays_match_eager():
    """The whole step (route, permute, FC1+GLU, FC2, unpermute, dOut gather,
    FC2 dgrad+dGLU, FC1 dgrad, unpermute + dprobs) captured into one HIP
    graph in global capture mode: any host sync or allocation inside the
    library would invalidate the capture."""
    wl = make_workload("tiny", seed=11, E=8, T=1024, H=256, I=256)
    gp, _ = act_of(wl)
    blk = mg.ExpertBlock(wl.E, wl.H, wl.I, wl.T, wl.k, act=gp)
    blk.load_weights(dev_bf16(wl.w1), dev_bf16(wl.w2))
    x = dev_bf16(wl.x)
    dout = dev_bf16(wl.dout)
    idx = torch.from_numpy(wl.expert_idx).cuda()
    probs = torch.from_numpy(wl.probs).cuda()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        blk.forward(x, idx, probs)
        blk.backward(dout)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    # z and dz are compared on the rows the kernels write (valid rows)
    valid = (blk.row_src >= 0).nonzero().squeeze(1)
    outs = (blk.out, blk.dx, blk.dprobs, blk.z, blk.dz)
    eager = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="global"):
        blk.forward(x, idx, probs)
        blk.backward(dout)
    for _ in range(3):
        for t in outs:
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outs, eager)):
            if i >= 3:
                t, e = t[valid], e[valid]
            assert torch.equal(t, e)
