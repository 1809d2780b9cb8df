"""Half-height tiles: an expert's last 128 rows or fewer run as a 128-row
tile (plain-store and GLU kernels with K-contiguous weights; the bf16
[K][N]-weight case here runs full tiles and checks that path on the same
sizes).  Group sizes chosen so that every case
appears: a group of 1..128 rows (one half tile), 129..256 (one full tile),
a full tile plus a half one, exactly 128 and 256 rows, and empty groups.
The plain grouped GEMM (bf16 [N][K] and [K][N] weights, MXFP8) against a
float32 product of the same operands, pad rows untouched; the fused layer
against the oracle, element by element."""

import numpy as np
import pytest
import torch

import moe_grouped_mlp_amd as mg
from oracle import numerics as nu
from workloads import make_workload

from .gpu_util import compare_layer, mx_scale_index, oracle_layer, run_gpu_layer
from .test_gpu_mx import compare_layer_mx

pytestmark = pytest.mark.gpu

SIZES = [100, 316, 128, 0, 129, 256, 641, 1, 384]


def _layout(sizes):
    pad = [0]
    for n in sizes:
        pad.append(pad[-1] + -(-n // mg.GROUP_ALIGN) * mg.GROUP_ALIGN)
    return pad


@pytest.mark.parametrize("b_kn", [False, True])
def test_plain_gemm_bf16_half_tiles(b_kn):
    dev = torch.device("cuda:0")
    pad = _layout(SIZES)
    E, N, K, M_cap = len(SIZES), 320, 448, pad[-1]
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    a = torch.randn(M_cap, K, generator=g, device=dev).to(torch.bfloat16)
    b = (torch.randn(E, N, K, generator=g, device=dev) * 0.05).to(torch.bfloat16)
    bw = b.transpose(1, 2).contiguous() if b_kn else b
    c = torch.full((M_cap, N), 5.0, dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(mg.moe_grouped_gemm_workspace_size(True), dtype=torch.uint8, device=dev)
    mg.moe_grouped_gemm(E=E, N=N, K=K, M_cap=M_cap,
                        split_sizes=torch.tensor(SIZES, dtype=torch.int32, device=dev),
                        padded_offsets=torch.tensor(pad, dtype=torch.int32, device=dev),
                        a=a, b=bw, c=c, b_kn=b_kn, workspace=ws)
    torch.cuda.synchronize()
    for e, n in enumerate(SIZES):
        r0 = pad[e]
        if n:
            ref = a[r0:r0 + n].float() @ b[e].float().T
            torch.testing.assert_close(c[r0:r0 + n].float(), ref, rtol=1e-2, atol=2e-2)
        assert (c[r0 + n:pad[e + 1]] == 5.0).all(), f"pad rows of group {e} written"


def test_plain_gemm_mxfp8_half_tiles():
    dev = torch.device("cuda:0")
    pad = _layout(SIZES)
    E, N, K, M_cap = len(SIZES), 256, 512, pad[-1]
    rng = np.random.default_rng(12)
    a = rng.standard_normal((M_cap, K))
    b = rng.standard_normal((E, N, K)) * 0.05
    u8 = dict(dtype=torch.uint8, device=dev)
    aq, as_ = nu.mx_quantize(a, axis=1)
    bq, bs = nu.mx_quantize(b.reshape(E * N, K), axis=1)
    # tiled scale layouts, as the quantize kernel writes them
    a_q = torch.from_numpy(aq).to(dev)
    b_q = torch.from_numpy(bq).to(dev)
    a_s = torch.empty(M_cap * K // 32, **u8)
    b_s = torch.empty(E * N * K // 32, **u8)
    idx_a = torch.from_numpy(mx_scale_index(M_cap, K).reshape(-1)).to(dev)
    idx_b = torch.from_numpy(mx_scale_index(N, K).reshape(-1)).to(dev)
    a_s[idx_a] = torch.from_numpy(as_.reshape(-1)).to(dev)
    for e in range(E):
        b_s[e * (N * K // 32) + idx_b] = torch.from_numpy(bs[e * N:(e + 1) * N].reshape(-1)).to(dev)
    c = torch.full((M_cap, N), 5.0, dtype=torch.bfloat16, device=dev)
    mg.moe_grouped_gemm(E=E, N=N, K=K, M_cap=M_cap,
                        split_sizes=torch.tensor(SIZES, dtype=torch.int32, device=dev),
                        padded_offsets=torch.tensor(pad, dtype=torch.int32, device=dev),
                        a=a_q, b=b_q, c=c, prec=mg.PREC_MXFP8, a_s=a_s, b_s=b_s)
    torch.cuda.synchronize()
    ad = nu.mx_dequantize(aq, as_, axis=1)
    bd = nu.mx_dequantize(bq, bs, axis=1).reshape(E, N, K)
    got = c.float().cpu().numpy()
    for e, n in enumerate(SIZES):
        r0 = pad[e]
        if n:
            ref = ad[r0:r0 + n] @ bd[e].T
            np.testing.assert_allclose(got[r0:r0 + n], ref, rtol=1e-2, atol=2e-2)
        assert (got[r0 + n:pad[e + 1]] == 5.0).all()


def _workload(seed, **kw):
    wl = make_workload("tiny", seed=seed, E=len(SIZES), k=1, T=sum(SIZES), **kw)
    rng = np.random.default_rng(seed)
    idx = np.repeat(np.arange(len(SIZES)), SIZES)[rng.permutation(sum(SIZES))]
    wl.expert_idx = idx.reshape(-1, 1).astype(np.int32)
    wl.probs = rng.random((sum(SIZES), 1)).astype(np.float32)
    assert wl.group_sizes().tolist() == SIZES
    return wl


@pytest.mark.parametrize("act", ["swiglu", "srelu"])
def test_layer_half_tiles_parity(act):
    wl = _workload(21, H=320, I=192, act=act)
    M_cap = wl.m_cap()
    blk = run_gpu_layer(wl, M_cap)
    fw, bw = oracle_layer(wl, M_cap)
    compare_layer(blk, wl, fw, bw)
    assert int(blk.err_flag.cpu()[0]) == 0


def test_layer_half_tiles_mx_parity():
    wl = _workload(22, H=256, I=192)
    M_cap = -(-wl.m_cap() // 128) * 128
    blk = run_gpu_layer(wl, M_cap, prec=mg.PREC_MXFP8)
    fw, bw = oracle_layer(wl, M_cap, mx=True)
    compare_layer_mx(blk, wl, fw, bw)
    assert int(blk.err_flag.cpu()[0]) == 0
