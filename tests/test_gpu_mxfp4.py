"""MXFP4 through the C ABI: moe_quantize_mxfp4 bit for bit against the
oracle's E2M1 / E8M0 encoding, and the MXFP4 grouped GEMM (gfx950's scaled
MFMA on E2M1 x E2M1) against the oracle's float64 contraction of the
MXFP4 operands it encodes itself from the same bf16 inputs."""

import numpy as np
import pytest
import torch

import moe_grouped_mlp_amd as mg
from oracle import numerics as nu

from .gpu_util import assert_close, dev_bf16, mx_scales_plain
from .test_gpu_mx import _hard_bf16

pytestmark = pytest.mark.gpu


def _unpack(q: np.ndarray) -> np.ndarray:
    """bytes [..., n] -> 4-bit codes [..., 2n], low nibble first."""
    out = np.empty(q.shape[:-1] + (2 * q.shape[-1],), np.uint8)
    out[..., 0::2] = q & 0xF
    out[..., 1::2] = q >> 4
    return out


def _with_ties(rng, bits, rows):
    """Rows whose blocks hold every E2M1 rounding midpoint (times a power of
    two; amax 6 fixes the scale) and their negatives."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    b = bits.copy()
    for r in range(0, rows, 9):
        k = int(rng.integers(-20, 20))
        row = np.resize(np.concatenate([mids, -mids]), b.shape[-1]) * 2.0 ** k
        b[..., r, :] = nu.f64_to_bf16_bits(row)
    return b


@pytest.mark.parametrize("mode", [mg.QUANT_ROW, mg.QUANT_COL])
@pytest.mark.parametrize("batch,rows,cols,pad", [(1, 32, 64, 0), (3, 128, 192, 0),
                                                 (2, 192, 2880, 40)])
def test_quantize_mxfp4_bit_exact(mode, batch, rows, cols, pad):
    rng = np.random.default_rng(rows + cols + 4)
    bits = _with_ties(rng, _hard_bf16(rng, (batch, rows, cols)), rows)
    stride = rows * cols + pad
    flat = np.zeros(batch * stride, np.uint16)
    for b in range(batch):
        flat[b * stride:b * stride + rows * cols] = bits[b].reshape(-1)
    x = dev_bf16(flat)
    q = torch.full((batch * rows * cols // 2,), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((batch * rows * cols // 32,), 0xAB, dtype=torch.uint8, device="cuda")
    if mode == mg.QUANT_COL and rows % 64:
        # the column mode takes rows in multiples of 64: rejected before any
        # launch, nothing written
        with pytest.raises(mg.MoeError) as ei:
            mg.moe_quantize_mxfp4(batch=batch, rows=rows, cols=cols, x=x, q=q, s=s, mode=mode,
                                  x_stride=stride if pad else 0)
        assert ei.value.status == mg.ERR_INVALID_ARG
        torch.cuda.synchronize()
        assert bool((q == 0xAB).all()) and bool((s == 0xAB).all())
        return
    mg.moe_quantize_mxfp4(batch=batch, rows=rows, cols=cols, x=x, q=q, s=s, mode=mode,
                          x_stride=stride if pad else 0)
    torch.cuda.synchronize()
    v = nu.bf16_to_f64(bits)
    R, K = (rows, cols) if mode == mg.QUANT_ROW else (cols, rows)
    qh = q.cpu().numpy().reshape(batch, R, K // 2)
    sh = s.cpu().numpy().reshape(batch, -1)
    for b in range(batch):
        src = v[b] if mode == mg.QUANT_ROW else v[b].T
        codes, scales = nu.mxfp4_quantize(src, axis=1)
        np.testing.assert_array_equal(_unpack(qh[b]), codes, f"codes, batch {b}")
        np.testing.assert_array_equal(qh[b], nu.pack_nibbles(codes))
        np.testing.assert_array_equal(mx_scales_plain(torch.from_numpy(sh[b]), R, K),
                                      scales, f"scales, batch {b}")


def _groups(sizes):
    pad = [0]
    for n in sizes:
        pad.append(pad[-1] + -(-n // mg.GROUP_ALIGN) * mg.GROUP_ALIGN)
    return pad


CASES = {
    # ragged groups (one empty), N not a multiple of the 256-wide tile,
    # K % 256 == 128 (the last stage half full)
    "ragged_k128": dict(sizes=[300, 0, 517, 129], N=384, K=640),
    # K % 256 == 64: the last stage holds one 64-deep step
    "ragged_k64": dict(sizes=[77, 640], N=256, K=576),
    "one_group_multi_tile": dict(sizes=[1000], N=768, K=1024),
}


@pytest.mark.parametrize("case", list(CASES))
def test_grouped_gemm_mxfp4_parity(case):
    c = CASES[case]
    sizes, N, K = c["sizes"], c["N"], c["K"]
    E = len(sizes)
    pad = _groups(sizes)
    M_cap = max(pad[-1], 128)
    rng = np.random.default_rng(sum(sizes) + N + K)
    a = rng.standard_normal((M_cap, K)) * np.exp2(rng.integers(-3, 4, (M_cap, 1)))
    b = rng.standard_normal((E, N, K)) * 0.05
    a_bits = nu.f64_to_bf16_bits(nu.round_bf16(a))
    b_bits = nu.f64_to_bf16_bits(nu.round_bf16(b))
    u8 = dict(dtype=torch.uint8, device="cuda")
    a_q, a_s = torch.empty(M_cap * K // 2, **u8), torch.empty(M_cap * K // 32, **u8)
    b_q, b_s = torch.empty(E * N * K // 2, **u8), torch.empty(E * N * K // 32, **u8)
    mg.moe_quantize_mxfp4(batch=1, rows=M_cap, cols=K, x=dev_bf16(a_bits.reshape(-1)),
                          q=a_q, s=a_s)
    mg.moe_quantize_mxfp4(batch=E, rows=N, cols=K, x=dev_bf16(b_bits.reshape(-1)), q=b_q,
                          s=b_s)
    out = torch.full((M_cap, N), -7.0, dtype=torch.bfloat16, device="cuda")
    split = torch.tensor(sizes, dtype=torch.int32, device="cuda")
    padded = torch.tensor(pad, dtype=torch.int32, device="cuda")
    mg.moe_grouped_gemm(E=E, N=N, K=K, M_cap=M_cap, split_sizes=split, padded_offsets=padded,
                        a=a_q, b=b_q, c=out, prec=mg.PREC_MXFP4, a_s=a_s, b_s=b_s)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    aq = nu.mxfp4_round(nu.bf16_to_f64(a_bits), axis=1)
    bq = nu.mxfp4_round(nu.bf16_to_f64(b_bits), axis=2)
    valid = np.zeros(M_cap, bool)
    for e in range(E):
        rows = slice(pad[e], pad[e] + sizes[e])
        valid[rows] = True
        ref = nu.round_bf16(aq[rows] @ bq[e].T)
        assert_close(got[rows], ref, f"expert {e}")
    # rows outside the groups are not written
    assert np.all(got[~valid] == -7.0)


@pytest.mark.timeout(600)
def test_mixtral_fc2_mxfp4_full_size_sampled():
    """The Mixtral-shaped FC2 GEMM at full size (E = 8, 16384 routed rows
    with the layer's group sizes, N = 4096, K = 14336), in the launch
    configuration bench.py --gemm times: sampled rows' codes and scales bit
    for bit, and 256 sampled outputs against the oracle's float64 dot
    products of its own MXFP4 encoding of the same bf16 rows."""
    from workloads.gen import CONFIGS, route_inputs
    cfg = dict(CONFIGS["mixtral"])
    E, k, T, N, K = cfg["E"], cfg["k"], cfg["T"], cfg["H"], cfg["I"]
    idx, _ = route_inputs(cfg, 0, T, E, k)
    flat = idx.reshape(-1)
    sizes = np.bincount(flat[(flat >= 0) & (flat < E)], minlength=E).tolist()
    pad = _groups(sizes)
    M_cap = pad[-1]
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    a = torch.randn(M_cap, K, generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn(E, N, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    u8 = dict(dtype=torch.uint8, device="cuda")
    a_q, a_s = torch.empty(M_cap, K // 2, **u8), torch.empty(M_cap * K // 32, **u8)
    b_q, b_s = torch.empty(E * N * K // 2, **u8), torch.empty(E * N * K // 32, **u8)
    mg.moe_quantize_mxfp4(batch=1, rows=M_cap, cols=K, x=a, q=a_q, s=a_s)
    mg.moe_quantize_mxfp4(batch=E, rows=N, cols=K, x=w, q=b_q, s=b_s)
    out = torch.empty(M_cap, N, dtype=torch.bfloat16, device="cuda")
    mg.moe_grouped_gemm(E=E, N=N, K=K, M_cap=M_cap,
                        split_sizes=torch.tensor(sizes, dtype=torch.int32, device="cuda"),
                        padded_offsets=torch.tensor(pad, dtype=torch.int32, device="cuda"),
                        a=a_q, b=b_q, c=out, prec=mg.PREC_MXFP4, a_s=a_s, b_s=b_s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    got, ref = [], []
    s_plain = mx_scales_plain(a_s, M_cap, K)
    for e in range(E):
        rows = pad[e] + rng.choice(sizes[e], 4, replace=False)
        cols = rng.choice(N, 8, replace=False)
        a_rows = nu.bf16_to_f64(a[rows].view(torch.int16).cpu().numpy().view(np.uint16))
        codes, scales = nu.mxfp4_quantize(a_rows, axis=1)
        np.testing.assert_array_equal(a_q[rows].cpu().numpy(), nu.pack_nibbles(codes))
        np.testing.assert_array_equal(s_plain[rows], scales)
        w_rows = nu.bf16_to_f64(w[e, cols].view(torch.int16).cpu().numpy().view(np.uint16))
        prod = nu.mxfp4_round(a_rows, axis=1) @ nu.mxfp4_round(w_rows, axis=1).T
        ref.append(nu.round_bf16(prod).reshape(-1))
        got.append(out[rows][:, cols].float().cpu().numpy().astype(np.float64).reshape(-1))
    assert_close(np.concatenate(got), np.concatenate(ref), "sampled outputs")
