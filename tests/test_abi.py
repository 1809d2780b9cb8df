"""Host-side checks of the C ABI (no GPU needed).

* the library loads and exports every function include/moe_gmlp.h declares;
* the ctypes structs of the binding have the header's layout (sizeof and
  offsetof of every field, read from a C program built with gcc);
* argument validation rejects bad calls before touching a device, and a
  valid call without a gfx950 device reports MOE_ERR_DEVICE.

The validation checks pass placeholder addresses (8, 16, 64) for device
buffers, so they run only where no HIP device is present: with one, a valid
call would launch kernels on those addresses.  The GPU tests cover valid
calls with real buffers.
"""

import ctypes
import os
import re
import shutil
import subprocess

import pytest

import moe_grouped_mlp_amd as m
from moe_grouped_mlp_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_gmlp.h")

INVALID, UNSUPPORTED, WORKSPACE, DEVICE = -1, -2, -3, -5


def _hip_device_present():
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return False
    n = ctypes.c_int(0)
    return hip.hipGetDeviceCount(ctypes.byref(n)) == 0 and n.value > 0


no_device = pytest.mark.skipif(
    _hip_device_present(),
    reason="placeholder device addresses: valid calls would launch on a present device")


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = m.lib()
    declared = _header_functions()
    assert set(declared) == set(B.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", m.lib_path],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_[a-z0-9_]+)", out))
    assert set(declared) <= exported


STRUCTS = {
    "moe_act_params": B.ActParams,
    "moe_permute_args": B.PermuteArgs,
    "moe_unpermute_args": B.UnpermuteArgs,
    "moe_quant_args": B.QuantArgs,
    "moe_fwd_args": B.FwdArgs,
    "moe_bwd_args": B.BwdArgs,
    "moe_wgrad_args": B.WgradArgs,
    "moe_router_args": B.RouterArgs,
    "moe_router_route_args": B.RouterRouteArgs,
    "moe_gemm_args": B.GemmArgs,
    "moe_glu_args": B.GluArgs,
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_ctypes_structs_match_header_layout(tmp_path):
    lines = ['#include <stdio.h>', '#include <stddef.h>',
             f'#include "{HEADER}"', "int main(void) {"]
    for cname, st in STRUCTS.items():
        lines.append(f'printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for fname, _ in st._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", '
                         f'offsetof({cname}, {fname}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-o", str(exe), str(src)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True,
                         check=True).stdout.split("\n")
    got = {}
    for line in out:
        if line:
            s, f, v = line.split()
            got[(s, f)] = int(v)
    for cname, st in STRUCTS.items():
        assert got[(cname, "sizeof")] == ctypes.sizeof(st), cname
        for fname, _ in st._fields_:
            assert got[(cname, fname)] == getattr(st, fname).offset, \
                (cname, fname)


def _call(fn, st):
    return getattr(m.lib(), fn)(ctypes.byref(st), None)


@no_device
def test_repack_validation():
    L = m.lib()
    assert L.moe_weight_repack_interleave(None, 8, 1, 64, 64, 64, 0, None) == INVALID
    assert L.moe_weight_repack_interleave(8, 8, 1, 64, 64, 64, 0, None) == INVALID   # alias
    assert L.moe_weight_repack_interleave(8, 16, 1, 96, 64, 64, 0, None) == INVALID  # I % 64
    assert L.moe_weight_repack_interleave(8, 16, 1, 64, 64, 32, 0, None) == INVALID  # block
    assert L.moe_weight_repack_interleave(8, 16, 1, 64, 60, 64, 0, None) == INVALID  # H % 8
    assert L.moe_weight_repack_interleave(8, 16, 1, 64, 64, 64, 0, None) == DEVICE


def _permute_args(**kw):
    a = B.PermuteArgs()
    a.flags, a.T, a.k, a.E, a.first_expert, a.H, a.M_cap = (
        B.PERMUTE_BUILD_MAP | B.PERMUTE_GATHER, 16, 2, 4, 0, 64, 16 * 2 + 4 * 127)
    for f in ("expert_idx", "probs", "split_sizes", "offsets", "padded_offsets",
              "row_id_map", "row_src", "probs_p", "x", "xp", "workspace"):
        setattr(a, f, 64)
    a.workspace_bytes = B.moe_permute_workspace_size(16, 4)
    for key, v in kw.items():
        setattr(a, key, v)
    return a


@no_device
def test_permute_validation():
    assert _call("moe_permute", _permute_args()) == DEVICE
    assert _call("moe_permute", _permute_args(flags=0)) == INVALID
    assert _call("moe_permute", _permute_args(flags=0x10)) == INVALID
    assert _call("moe_permute", _permute_args(k=9)) == INVALID
    assert _call("moe_permute", _permute_args(E=0)) == INVALID
    assert _call("moe_permute", _permute_args(E=1025)) == INVALID
    assert _call("moe_permute", _permute_args(row_src=None)) == INVALID
    assert _call("moe_permute", _permute_args(workspace=None)) == WORKSPACE
    assert _call("moe_permute", _permute_args(workspace_bytes=1)) == WORKSPACE
    assert _call("moe_permute", _permute_args(H=60)) == INVALID
    # gather only needs no workspace
    assert _call("moe_permute", _permute_args(flags=B.PERMUTE_GATHER,
                                              workspace=None)) == DEVICE
    assert B.moe_permute_workspace_size(257, 8) == 2 * 8 * 4


def _fwd_args(**kw):
    a = B.FwdArgs()
    a.E, a.H, a.I, a.M_cap, a.prec = 4, 128, 256, 1024, B.PREC_BF16
    a.act = B.act_params()
    for f in ("split_sizes", "padded_offsets", "probs_p", "xp", "w1i", "w2",
              "z", "a", "yp"):
        setattr(a, f, 64)
    for key, v in kw.items():
        setattr(a, key, v)
    return a


@no_device
def test_fwd_validation():
    assert _call("moe_grouped_mlp_fwd", _fwd_args()) == DEVICE
    assert _call("moe_grouped_mlp_fwd", _fwd_args(H=96)) == INVALID
    assert _call("moe_grouped_mlp_fwd", _fwd_args(I=100)) == INVALID
    assert _call("moe_grouped_mlp_fwd", _fwd_args(E=0)) == INVALID
    assert _call("moe_grouped_mlp_fwd", _fwd_args(a=None)) == INVALID
    assert _call("moe_grouped_mlp_fwd", _fwd_args(split_sizes=None)) == INVALID
    assert _call("moe_grouped_mlp_fwd", _fwd_args(prec=7)) == INVALID
    assert _call("moe_grouped_mlp_fwd", _fwd_args(cu_margin=-1)) == INVALID
    assert _call("moe_grouped_mlp_fwd",
                 _fwd_args(act=B.act_params(act=9))) == INVALID
    assert _call("moe_grouped_mlp_fwd",
                 _fwd_args(act=B.act_params(gate_lo=1.0, gate_hi=-1.0))) == INVALID
    assert _call("moe_grouped_mlp_fwd", _fwd_args(w1_stride=5)) == INVALID
    # z may be NULL (no backward follows)
    assert _call("moe_grouped_mlp_fwd", _fwd_args(z=None)) == DEVICE


@no_device
def test_unfused_baseline_validation():
    def gemm(**kw):
        a = B.GemmArgs(4, 256, 128, 1024, 0, 0, 64, 64, 64, 64, 0, 64, None, 0,
                       B.PREC_BF16, None, None, 0)
        for f, v in kw.items():
            setattr(a, f, v)
        return a
    assert _call("moe_grouped_gemm", gemm()) == DEVICE
    assert _call("moe_grouped_gemm", gemm(b_kn=1, b_stride=256 * 128)) == DEVICE
    mx = dict(prec=B.PREC_MXFP8, a_s=64, b_s=64)
    assert _call("moe_grouped_gemm", gemm(**mx)) == DEVICE
    f4 = dict(prec=B.PREC_MXFP4, a_s=64, b_s=64)
    assert _call("moe_grouped_gemm", gemm(**f4)) == DEVICE
    for bad in (dict(f4, b_kn=1), dict(f4, b_s=None), dict(f4, M_cap=1000),
                dict(f4, b_stride=256 * 128 + 1)):
        assert _call("moe_grouped_gemm", gemm(**bad)) == INVALID, bad
    for bad in (dict(N=100), dict(K=32), dict(E=0), dict(b_kn=2), dict(a=None),
                dict(c=None), dict(b_stride=5), dict(cu_margin=-1), dict(M_cap=0),
                dict(prec=9), dict(mx, b_kn=1), dict(mx, a_s=None),
                dict(mx, M_cap=1000), dict(mx, b_s_stride=3)):
        assert _call("moe_grouped_gemm", gemm(**bad)) == INVALID, bad

    def glu(**kw):
        a = B.GluArgs()
        a.direction, a.E, a.I, a.M_cap = 0, 4, 256, 1024
        a.act = B.act_params()
        for f in ("split_sizes", "padded_offsets", "probs_p", "z", "a", "da", "dz",
                  "dprobs_p"):
            setattr(a, f, 64)
        for f, v in kw.items():
            setattr(a, f, v)
        return a
    assert _call("moe_glu_unfused", glu()) == DEVICE
    assert _call("moe_glu_unfused", glu(direction=1, a=None)) == DEVICE
    for bad in (dict(direction=2), dict(I=96), dict(z=None), dict(a=None),
                dict(direction=1, dz=None), dict(direction=1, da=None),
                dict(act=B.act_params(gate_lo=1.0, gate_hi=-1.0))):
        assert _call("moe_glu_unfused", glu(**bad)) == INVALID, bad


@no_device
def test_router_validation():
    def args(**kw):
        a = B.RouterArgs(16, 8, 2, 64, 64, 64)
        for f, v in kw.items():
            setattr(a, f, v)
        return a
    assert _call("moe_router_topk", args()) == DEVICE
    assert _call("moe_router_topk", args(E=1024, k=8)) == DEVICE
    assert _call("moe_router_topk", args(E=3, k=3)) == DEVICE
    for bad in (dict(T=0), dict(E=0), dict(E=1025), dict(k=0), dict(k=9),
                dict(E=2, k=3), dict(logits=None), dict(expert_idx=None),
                dict(probs=None)):
        assert _call("moe_router_topk", args(**bad)) == INVALID, bad


@no_device
def test_wgrad_validation():
    def args(**kw):
        a = B.WgradArgs()
        a.E, a.H, a.I, a.gated, a.M_cap, a.prec = 4, 128, 256, 1, 1024, B.PREC_BF16
        for f in ("split_sizes", "padded_offsets", "dz", "xp", "dyp", "a",
                  "dw1", "dw2"):
            setattr(a, f, 64)
        for k, v in kw.items():
            setattr(a, k, v)
        return a
    assert _call("moe_grouped_mlp_wgrad", args()) == DEVICE
    assert _call("moe_grouped_mlp_wgrad", args(dw1=None, dz=None, xp=None)) == DEVICE
    assert _call("moe_grouped_mlp_wgrad", args(dw2=None, dyp=None, a=None)) == DEVICE
    assert _call("moe_grouped_mlp_wgrad", args(M_cap=1000)) == DEVICE   # bf16: any M_cap
    for bad in (dict(M_cap=0), dict(M_cap=1 << 23), dict(H=96), dict(I=32),
                dict(E=0), dict(gated=2), dict(prec=7), dict(cu_margin=-1),
                dict(split_sizes=None), dict(padded_offsets=None), dict(a=None),
                dict(xp=None), dict(prec=B.PREC_MXFP8),
                # bf16 addresses a whole [M_cap][n] activation with 32-bit offsets
                dict(M_cap=1 << 17, I=16384)):
        assert _call("moe_grouped_mlp_wgrad", args(**bad)) == INVALID, bad
    # MXFP8 reads the transposed copies and needs the scales of every one
    mx = dict(prec=B.PREC_MXFP8, dz=None, xp=None, dyp=None, a=None,
              dzT_q=64, dzT_s=64, xpT_q=64, xpT_s=64, dypT_q=64, dypT_s=64,
              aT_q=64, aT_s=64)
    assert _call("moe_grouped_mlp_wgrad", args(**mx)) == DEVICE
    assert _call("moe_grouped_mlp_wgrad", args(**{**mx, "aT_s": None})) == INVALID
    assert _call("moe_grouped_mlp_wgrad", args(**{**mx, "xpT_q": None})) == INVALID
    assert _call("moe_grouped_mlp_wgrad", args(**{**mx, "M_cap": 1000})) == INVALID
    # MXFP4 the same way
    f4 = {**mx, "prec": B.PREC_MXFP4}
    assert _call("moe_grouped_mlp_wgrad", args(**f4)) == DEVICE
    assert _call("moe_grouped_mlp_wgrad", args(**{**f4, "dzT_s": None})) == INVALID
    assert _call("moe_grouped_mlp_wgrad", args(**{**f4, "M_cap": 1000})) == INVALID


@no_device
def test_bwd_validation():
    a = B.BwdArgs()
    a.E, a.H, a.I, a.M_cap, a.prec = 4, 128, 256, 1024, B.PREC_BF16
    a.act = B.act_params()
    for f in ("split_sizes", "padded_offsets", "probs_p", "dyp", "w2", "z",
              "w1i", "dz", "dprobs_p", "dxp", "workspace"):
        setattr(a, f, 64)
    # the dprobs partials (one per 256-column tile of I) are required; the
    # full size adds the split-K area (one fp32 256 x 256 tile and a counter
    # per workgroup of a one-per-CU grid; 256 CUs assumed without a device,
    # rounded up to 256 bytes) and the work counters of dynamic tile
    # scheduling (8 XCDs x 64 bytes for each of the two GEMMs)
    need = 1024 * 1 * 4
    full = B.moe_grouped_mlp_workspace_size(4, 128, 256, 1024)
    split = -(-256 * (256 * 256 * 4 + 4) // 256) * 256
    assert full == need + split + 2 * 8 * 64
    assert B.moe_grouped_gemm_workspace_size(False) == split
    assert B.moe_grouped_gemm_workspace_size(True) == split + 8 * 64
    a.workspace_bytes = full
    assert _call("moe_grouped_mlp_bwd", a) == DEVICE
    a.workspace_bytes = need
    assert _call("moe_grouped_mlp_bwd", a) == DEVICE
    a.workspace_bytes = need - 1
    assert _call("moe_grouped_mlp_bwd", a) == WORKSPACE
    a.workspace_bytes = need
    a.z = None
    assert _call("moe_grouped_mlp_bwd", a) == INVALID


@no_device
def test_router_route_validation():
    a = B.RouterRouteArgs()
    a.T, a.E_total, a.k, a.E, a.first_expert, a.M_cap = 1000, 64, 4, 32, 0, 5000
    for f in ("logits", "expert_idx", "probs", "split_sizes", "padded_offsets",
              "row_id_map", "row_src", "probs_p", "workspace"):
        setattr(a, f, 64)
    need = B.moe_router_route_workspace_size(1000, 64, 32)
    assert need == 4096 + 16 * 4 * 32        # counters + [ceil(T / 64)][E] counts
    assert B.moe_router_route_workspace_size(1000, 32, 32) == 4096 + 4 * 4 * 32
    a.workspace_bytes = need
    assert _call("moe_router_route", a) == DEVICE
    a.workspace_bytes = need - 1
    assert _call("moe_router_route", a) == WORKSPACE
    a.workspace_bytes = need
    for field, bad in (("k", 9), ("k", 0), ("E_total", 1025), ("E", 0), ("T", 0),
                       ("first_expert", -1), ("M_cap", 0)):
        old = getattr(a, field)
        setattr(a, field, bad)
        assert _call("moe_router_route", a) == INVALID, field
        setattr(a, field, old)
    a.k, a.E_total = 8, 6                       # k > E_total
    assert _call("moe_router_route", a) == INVALID
    a.k, a.E_total = 4, 64
    a.row_src = None
    assert _call("moe_router_route", a) == INVALID
    a.row_src = 64
    a.offsets = None                            # optional
    assert _call("moe_router_route", a) == DEVICE


@no_device
def test_bwd_noalloc_validation():
    """The backward without a workspace argument: the same host checks
    first, then the fixed scratch size (MOE_ERR_UNSUPPORTED past it), then
    the device; the workspace fields are ignored."""
    a = B.BwdArgs()
    a.E, a.H, a.I, a.M_cap, a.prec = 4, 128, 256, 1024, B.PREC_BF16
    a.act = B.act_params()
    for f in ("split_sizes", "padded_offsets", "probs_p", "dyp", "w2", "z",
              "w1i", "dz", "dprobs_p", "dxp"):
        setattr(a, f, 64)
    a.workspace, a.workspace_bytes = None, 0
    assert _call("moe_grouped_mlp_bwd_noalloc", a) == DEVICE
    a.z = None
    assert _call("moe_grouped_mlp_bwd_noalloc", a) == INVALID
    a.z = 64
    # fp32 partials of M_cap rows x ceil(I / 256) tiles past 16 MiB
    a.I = 1024
    a.M_cap = B.NOALLOC_SCRATCH_BYTES // (4 * 4)
    assert _call("moe_grouped_mlp_bwd_noalloc", a) == DEVICE
    a.M_cap += 128
    assert _call("moe_grouped_mlp_bwd_noalloc", a) == UNSUPPORTED
    assert m.lib().moe_grouped_mlp_bwd_noalloc(None, None) == INVALID


@no_device
def test_unpermute_validation():
    a = B.UnpermuteArgs(8, 2, 64, 100, 64, 64, 64, None, None)
    assert _call("moe_unpermute", a) == DEVICE
    a.dprobs = 64          # dprobs without dprobs_p
    assert _call("moe_unpermute", a) == INVALID
    a.dprobs, a.H = None, 12
    assert _call("moe_unpermute", a) == INVALID


@no_device
def test_bench_occupy_validation():
    L = m.lib()
    assert L.moe_bench_occupy(0, 1000, None) == INVALID
    assert L.moe_bench_occupy(1025, 1000, None) == INVALID
    assert L.moe_bench_occupy(8, 0, None) == INVALID
    assert L.moe_bench_occupy(8, 100000001, None) == INVALID


@no_device
def test_gemm_clock_trace_validation():
    L = m.lib()
    assert L.moe_gemm_clock_trace(64, 0) == INVALID
    assert L.moe_gemm_clock_trace(64, 65) == INVALID
    assert L.moe_gemm_clock_trace(None, 0) == 0      # clearing needs no slots
    assert L.moe_gemm_clock_trace(None, 5) == 0


def test_status_strings():
    L = m.lib()
    for code in (0, -1, -2, -3, -4, -5):
        assert L.moe_status_string(code)
    assert L.moe_status_string(-99) == b"unknown status"


# ------------------------------------------------------------------ MXFP8 --
def test_mx_scale_offset_is_the_documented_tiled_layout():
    """Byte of (row r, K-block b) of an [R][K] operand: a bijection onto
    [0, R*K/32), and each 32-row x 64-column unit owns one 64-byte run."""
    for R, K in ((32, 64), (96, 192), (128, 2880), (64, 4096)):
        offs = [[B.moe_mx_scale_offset(r, b, K) for b in range(K // 32)]
                for r in range(R)]
        flat = sorted(o for row in offs for o in row)
        assert flat == list(range(R * K // 32))
        for r in range(R):
            for b in range(K // 32):
                o = offs[r][b]
                unit = (r // 32) * (K // 64) + b // 2
                assert o // 64 == unit
                assert o % 64 == (b % 2) * 32 + r % 32


def _quant_args(**kw):
    a = B.QuantArgs(B.QUANT_ROW, 2, 128, 192, 0, 64, 64, 64, None)
    for key, v in kw.items():
        setattr(a, key, v)
    return a


@no_device
def test_quantize_validation():
    assert _call("moe_quantize_mxfp8", _quant_args()) == DEVICE
    assert _call("moe_quantize_mxfp8", _quant_args(mode=B.QUANT_COL)) == DEVICE
    # BOTH needs the COL destination as well
    assert _call("moe_quantize_mxfp8", _quant_args(mode=B.QUANT_BOTH)) == INVALID
    assert _call("moe_quantize_mxfp8", _quant_args(mode=B.QUANT_BOTH, qT=64)) == INVALID
    assert _call("moe_quantize_mxfp8", _quant_args(mode=B.QUANT_BOTH, qT=64, sT=64)) == DEVICE
    assert _call("moe_quantize_mxfp8", _quant_args(mode=3)) == INVALID
    assert _call("moe_quantize_mxfp8", _quant_args(rows=96)) == INVALID    # % 64
    assert _call("moe_quantize_mxfp8", _quant_args(cols=160)) == INVALID   # % 64
    assert _call("moe_quantize_mxfp8", _quant_args(batch=-1)) == INVALID
    assert _call("moe_quantize_mxfp8", _quant_args(x=None)) == INVALID
    assert _call("moe_quantize_mxfp8", _quant_args(s=None)) == INVALID
    assert _call("moe_quantize_mxfp8", _quant_args(x_stride=128 * 192 - 8)) == INVALID
    assert _call("moe_quantize_mxfp8", _quant_args(x_stride=128 * 192 + 4)) == INVALID
    assert _call("moe_quantize_mxfp8", _quant_args(x_stride=128 * 192 + 8)) == DEVICE


@no_device
def test_quantize_mxfp4_validation():
    assert _call("moe_quantize_mxfp4", _quant_args()) == DEVICE
    assert _call("moe_quantize_mxfp4", _quant_args(rows=96)) == DEVICE      # % 32 is enough
    assert _call("moe_quantize_mxfp4", _quant_args(mode=B.QUANT_COL)) == DEVICE
    assert _call("moe_quantize_mxfp4", _quant_args(mode=B.QUANT_COL, rows=96)) == INVALID
    assert _call("moe_quantize_mxfp4", _quant_args(mode=B.QUANT_BOTH)) == INVALID
    assert _call("moe_quantize_mxfp4", _quant_args(mode=B.QUANT_BOTH, qT=64, sT=64)) == DEVICE
    assert _call("moe_quantize_mxfp4",
                 _quant_args(mode=B.QUANT_BOTH, qT=64, sT=64, rows=96)) == INVALID   # % 64
    assert _call("moe_quantize_mxfp4", _quant_args(mode=3)) == INVALID
    assert _call("moe_quantize_mxfp4", _quant_args(rows=80)) == INVALID     # % 32
    assert _call("moe_quantize_mxfp4", _quant_args(cols=160)) == INVALID    # % 64
    assert _call("moe_quantize_mxfp4", _quant_args(amax=64)) == INVALID
    assert _call("moe_quantize_mxfp4", _quant_args(q=None)) == INVALID
    assert _call("moe_quantize_mxfp4", _quant_args(x_stride=128 * 192 + 4)) == INVALID


@no_device
def test_permute_write_mx_validation():
    mx = B.PERMUTE_BUILD_MAP | B.PERMUTE_GATHER | B.PERMUTE_WRITE_MX
    ok = dict(flags=mx, xp_q=64, xp_s=64, M_cap=640)
    assert _call("moe_permute", _permute_args(**ok)) == DEVICE
    assert _call("moe_permute", _permute_args(**{**ok, "xp": None})) == DEVICE
    assert _call("moe_permute", _permute_args(**{**ok, "xp_s": None})) == INVALID
    assert _call("moe_permute", _permute_args(**{**ok, "M_cap": 600})) == INVALID
    assert _call("moe_permute", _permute_args(**{**ok, "H": 96})) == INVALID
    # WRITE_MX modifies a gather
    assert _call("moe_permute", _permute_args(
        **{**ok, "flags": B.PERMUTE_BUILD_MAP | B.PERMUTE_WRITE_MX})) == INVALID


@no_device
def test_fwd_bwd_mx_validation():
    mx_fwd = ("xp_q", "xp_s", "w1_q", "w1_s", "w2_q", "w2_s", "a_q", "a_s")
    base = {f: 64 for f in mx_fwd}
    base.update(prec=B.PREC_MXFP8, xp=None, w1i=None, w2=None, a=None)
    assert _call("moe_grouped_mlp_fwd", _fwd_args(**base)) == DEVICE
    for f in mx_fwd:
        assert _call("moe_grouped_mlp_fwd", _fwd_args(**{**base, f: None})) == INVALID, f
    assert _call("moe_grouped_mlp_fwd", _fwd_args(**{**base, "aT_q": 64})) == INVALID
    assert _call("moe_grouped_mlp_fwd",
                 _fwd_args(**{**base, "aT_q": 64, "aT_s": 64})) == DEVICE
    assert _call("moe_grouped_mlp_fwd", _fwd_args(**{**base, "M_cap": 1000})) == INVALID

    a = B.BwdArgs()
    a.E, a.H, a.I, a.M_cap, a.prec = 4, 128, 256, 1024, B.PREC_MXFP8
    a.act = B.act_params()
    mx_bwd = ("dyp_q", "dyp_s", "w2t_q", "w2t_s", "w1t_q", "w1t_s", "dz_q", "dz_s")
    for f in ("split_sizes", "padded_offsets", "probs_p", "z", "dprobs_p",
              "dxp", "workspace") + mx_bwd:
        setattr(a, f, 64)
    a.workspace_bytes = B.moe_grouped_mlp_workspace_size(4, 128, 256, 1024,
                                                         B.PREC_MXFP8)
    assert _call("moe_grouped_mlp_bwd", a) == DEVICE      # dz (bf16) optional
    for f in mx_bwd:
        setattr(a, f, None)
        assert _call("moe_grouped_mlp_bwd", a) == INVALID, f
        setattr(a, f, 64)
    a.dzT_s = 64
    assert _call("moe_grouped_mlp_bwd", a) == INVALID


@no_device
def test_permute_write_mx4_validation():
    mx4 = B.PERMUTE_BUILD_MAP | B.PERMUTE_GATHER | B.PERMUTE_WRITE_MX4
    ok = dict(flags=mx4, xp_q=64, xp_s=64, M_cap=640)
    assert _call("moe_permute", _permute_args(**ok)) == DEVICE
    assert _call("moe_permute", _permute_args(**{**ok, "xp": None})) == DEVICE
    assert _call("moe_permute", _permute_args(**{**ok, "xp_q": None})) == INVALID
    assert _call("moe_permute", _permute_args(**{**ok, "M_cap": 600})) == INVALID
    assert _call("moe_permute", _permute_args(**{**ok, "H": 96})) == INVALID
    # one MX format per call, and only with a gather
    assert _call("moe_permute", _permute_args(
        **{**ok, "flags": mx4 | B.PERMUTE_WRITE_MX})) == INVALID
    assert _call("moe_permute", _permute_args(
        **{**ok, "flags": B.PERMUTE_BUILD_MAP | B.PERMUTE_WRITE_MX4})) == INVALID


@no_device
def test_fwd_bwd_mxfp4_validation():
    mx_fwd = ("xp_q", "xp_s", "w1_q", "w1_s", "w2_q", "w2_s", "a_q", "a_s")
    base = {f: 64 for f in mx_fwd}
    base.update(prec=B.PREC_MXFP4, xp=None, w1i=None, w2=None, a=None)
    assert _call("moe_grouped_mlp_fwd", _fwd_args(**base)) == DEVICE
    for f in mx_fwd:
        assert _call("moe_grouped_mlp_fwd", _fwd_args(**{**base, f: None})) == INVALID, f
    # the transposed copy is optional (both pointers or neither); no bias
    assert _call("moe_grouped_mlp_fwd",
                 _fwd_args(**{**base, "aT_q": 64, "aT_s": 64})) == DEVICE
    assert _call("moe_grouped_mlp_fwd", _fwd_args(**{**base, "aT_q": 64})) == INVALID
    assert _call("moe_grouped_mlp_fwd", _fwd_args(**{**base, "bias1": 64})) == INVALID
    assert _call("moe_grouped_mlp_fwd", _fwd_args(**{**base, "M_cap": 1000})) == INVALID
    # the MXFP4 epilogues' 32-bit lane offsets: M_cap up to 2^27, I up to 2^26
    assert _call("moe_grouped_mlp_fwd",
                 _fwd_args(**{**base, "M_cap": (1 << 27) + 128})) == UNSUPPORTED
    assert _call("moe_grouped_mlp_fwd", _fwd_args(**{**base, "I": (1 << 26) + 64})) == UNSUPPORTED

    a = B.BwdArgs()
    a.E, a.H, a.I, a.M_cap, a.prec = 4, 128, 256, 1024, B.PREC_MXFP4
    a.act = B.act_params()
    mx_bwd = ("dyp_q", "dyp_s", "w2t_q", "w2t_s", "w1t_q", "w1t_s", "dz_q", "dz_s")
    for f in ("split_sizes", "padded_offsets", "probs_p", "z", "dprobs_p",
              "dxp", "workspace") + mx_bwd:
        setattr(a, f, 64)
    a.workspace_bytes = B.moe_grouped_mlp_workspace_size(4, 128, 256, 1024,
                                                         B.PREC_MXFP4)
    assert _call("moe_grouped_mlp_bwd", a) == DEVICE
    for f in mx_bwd:
        setattr(a, f, None)
        assert _call("moe_grouped_mlp_bwd", a) == INVALID, f
        setattr(a, f, 64)
    a.dzT_q, a.dzT_s = 64, 64
    assert _call("moe_grouped_mlp_bwd", a) == DEVICE
    a.dzT_s = None
    assert _call("moe_grouped_mlp_bwd", a) == INVALID
    a.dzT_q = None
    a.bias1 = 64
    assert _call("moe_grouped_mlp_bwd", a) == INVALID
