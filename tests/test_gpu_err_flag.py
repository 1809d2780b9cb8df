"""Device-side checks of the grouped GEMMs: split_sizes / padded_offsets
that contradict each other (a negative size, a group running into the next
group's rows or past M_cap) OR MOE_DEVERR_BAD_OFFSETS into err_flag, and the
kernel still stays inside the caller's buffers (rows past M_cap are not
computed).  Consistent offsets leave the flag at 0 and give the plain
product on every routed row."""

import numpy as np
import pytest
import torch

import moe_grouped_mlp_amd as mg

pytestmark = pytest.mark.gpu

N, K = 256, 128


def _run(split, pad, M_cap):
    dev = torch.device("cuda:0")
    E = len(split)
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    a = torch.randn(M_cap, K, generator=g, device=dev).to(torch.bfloat16)
    b = (torch.randn(E, N, K, generator=g, device=dev) * 0.1).to(torch.bfloat16)
    c = torch.full((M_cap, N), 7.0, dtype=torch.bfloat16, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    mg.moe_grouped_gemm(E=E, N=N, K=K, M_cap=M_cap,
                        split_sizes=torch.tensor(split, dtype=torch.int32, device=dev),
                        padded_offsets=torch.tensor(pad, dtype=torch.int32, device=dev),
                        a=a, b=b, c=c, err_flag=err)
    torch.cuda.synchronize()
    return a, b, c, int(err.item())


def _expect_rows(a, b, c, e, r0, r1):
    ref = (a[r0:r1].float() @ b[e].float().T)
    got = c[r0:r1].float()
    assert torch.allclose(got, ref, rtol=2e-2, atol=2e-2)


def test_consistent_offsets_leave_the_flag_clear():
    a, b, c, err = _run([100, 50], [0, 128, 256], 256)
    assert err == 0
    _expect_rows(a, b, c, 0, 0, 100)
    _expect_rows(a, b, c, 1, 128, 178)
    assert (c[100:128] == 7.0).all() and (c[178:256] == 7.0).all()   # pad rows untouched


@pytest.mark.parametrize("split,pad,M_cap", [
    ([200, 50], [0, 128, 256], 384),     # group 0 runs into group 1's rows
    ([-5, 50], [0, 128, 256], 256),      # a negative size
    ([100, 300], [0, 128, 512], 256),    # group 1 runs past M_cap
])
def test_inconsistent_offsets_set_the_flag(split, pad, M_cap):
    a, b, c, err = _run(split, pad, M_cap)
    assert err == mg.DEVERR_BAD_OFFSETS
    if split[1] == 300:
        # the rows of group 1 inside M_cap are still computed
        _expect_rows(a, b, c, 1, 128, 256)
        _expect_rows(a, b, c, 0, 0, 100)
