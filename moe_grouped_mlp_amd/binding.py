"""ctypes binding of libmoe_gmlp.so: one Python function per C entry point,
with the same name and arguments.  Tensors are passed as device pointers
(``tensor.data_ptr()``) and the stream defaults to torch's current stream.
The functions only marshal arguments; all work runs in the HIP kernels.
"""

from __future__ import annotations

import ctypes
import math
import os
from ctypes import c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(HERE, "libmoe_gmlp.so")

# ---- constants mirrored from include/moe_gmlp.h ---------------------------
ACT_SWIGLU, ACT_GEGLU, ACT_SRELU = 0, 1, 2
PREC_BF16, PREC_MXFP8, PREC_MXFP4 = 0, 1, 2
PERMUTE_BUILD_MAP, PERMUTE_GATHER, PERMUTE_WRITE_MX = 0x1, 0x2, 0x4
PERMUTE_WRITE_MX4 = 0x8
QUANT_ROW, QUANT_COL, QUANT_BOTH = 0, 1, 2
GROUP_ALIGN = 128
INTERLEAVE = 64
MX_BLOCK = 32
DEVERR_MCAP_OVERFLOW, DEVERR_DUP_EXPERT, DEVERR_SYNC_TIMEOUT = 0x1, 0x2, 0x4
DEVERR_BAD_OFFSETS = 0x8
NOALLOC_SCRATCH_BYTES = 16 << 20
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_LAUNCH, ERR_DEVICE = 0, -1, -2, -3, -4, -5

EXPORTED_SYMBOLS = (
    "moe_weight_repack_interleave", "moe_permute_workspace_size",
    "moe_permute", "moe_unpermute", "moe_quantize_mxfp8", "moe_quantize_mxfp4",
    "moe_grouped_mlp_fwd", "moe_grouped_mlp_bwd", "moe_grouped_mlp_wgrad",
    "moe_router_topk", "moe_grouped_gemm", "moe_glu_unfused",
    "moe_grouped_mlp_workspace_size", "moe_status_string", "moe_gmlp_version",
    "moe_mx_scale_offset", "moe_grouped_mlp_bwd_noalloc", "moe_router_route",
    "moe_router_route_workspace_size", "moe_clock_tick_rate_hz",
    "moe_gemm_clock_trace", "moe_bench_occupy", "moe_grouped_gemm_workspace_size",
)


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {text} (status {status})")
        self.status = status


# ---- argument structs (layout of include/moe_gmlp.h) ----------------------
class ActParams(ctypes.Structure):
    _fields_ = [("act", c_int32), ("beta", c_float), ("gate_lo", c_float),
                ("gate_hi", c_float), ("lin_lo", c_float), ("lin_hi", c_float),
                ("lin_offset", c_float)]


class PermuteArgs(ctypes.Structure):
    _fields_ = [("flags", c_int32), ("T", c_int32), ("k", c_int32),
                ("E", c_int32), ("first_expert", c_int32), ("H", c_int32),
                ("M_cap", c_int64),
                ("expert_idx", c_void_p), ("probs", c_void_p),
                ("split_sizes", c_void_p), ("offsets", c_void_p),
                ("padded_offsets", c_void_p), ("row_id_map", c_void_p),
                ("row_src", c_void_p), ("probs_p", c_void_p),
                ("x", c_void_p), ("xp", c_void_p), ("xp_q", c_void_p),
                ("xp_s", c_void_p), ("err_flag", c_void_p),
                ("workspace", c_void_p), ("workspace_bytes", c_size_t)]


class UnpermuteArgs(ctypes.Structure):
    _fields_ = [("T", c_int32), ("k", c_int32), ("H", c_int32),
                ("M_cap", c_int64), ("row_id_map", c_void_p), ("yp", c_void_p),
                ("out", c_void_p), ("dprobs_p", c_void_p),
                ("dprobs", c_void_p)]


class QuantArgs(ctypes.Structure):
    _fields_ = [("mode", c_int32), ("batch", c_int32), ("rows", c_int32),
                ("cols", c_int32), ("x_stride", c_int64), ("x", c_void_p),
                ("q", c_void_p), ("s", c_void_p), ("amax", c_void_p),
                ("qT", c_void_p), ("sT", c_void_p), ("live", c_void_p)]


class FwdArgs(ctypes.Structure):
    _fields_ = [("E", c_int32), ("H", c_int32), ("I", c_int32),
                ("M_cap", c_int64), ("prec", c_int32), ("act", ActParams),
                ("cu_margin", c_int32), ("split_sizes", c_void_p),
                ("padded_offsets", c_void_p), ("probs_p", c_void_p),
                ("xp", c_void_p), ("w1i", c_void_p), ("w2", c_void_p),
                ("w1_stride", c_int64), ("w2_stride", c_int64),
                ("z", c_void_p), ("a", c_void_p), ("amax", c_void_p),
                ("yp", c_void_p), ("err_flag", c_void_p),
                ("timing_events", c_void_p * 3),
                ("xp_q", c_void_p), ("xp_s", c_void_p),
                ("w1_q", c_void_p), ("w1_s", c_void_p),
                ("w2_q", c_void_p), ("w2_s", c_void_p),
                ("a_q", c_void_p), ("a_s", c_void_p),
                ("aT_q", c_void_p), ("aT_s", c_void_p),
                ("workspace", c_void_p), ("workspace_bytes", c_size_t),
                ("bias1", c_void_p)]


class BwdArgs(ctypes.Structure):
    _fields_ = [("E", c_int32), ("H", c_int32), ("I", c_int32),
                ("M_cap", c_int64), ("prec", c_int32), ("act", ActParams),
                ("cu_margin", c_int32), ("split_sizes", c_void_p),
                ("padded_offsets", c_void_p), ("probs_p", c_void_p),
                ("dyp", c_void_p), ("w2", c_void_p), ("z", c_void_p),
                ("w1i", c_void_p), ("w1_stride", c_int64),
                ("w2_stride", c_int64), ("dz", c_void_p),
                ("dprobs_p", c_void_p), ("dxp", c_void_p),
                ("err_flag", c_void_p), ("workspace", c_void_p),
                ("workspace_bytes", c_size_t),
                ("timing_events", c_void_p * 3),
                ("dyp_q", c_void_p), ("dyp_s", c_void_p),
                ("w2t_q", c_void_p), ("w2t_s", c_void_p),
                ("w1t_q", c_void_p), ("w1t_s", c_void_p),
                ("dz_q", c_void_p), ("dz_s", c_void_p),
                ("dzT_q", c_void_p), ("dzT_s", c_void_p), ("bias1", c_void_p)]


class GemmArgs(ctypes.Structure):
    _fields_ = [("E", c_int32), ("N", c_int32), ("K", c_int32),
                ("M_cap", c_int64), ("b_kn", c_int32), ("cu_margin", c_int32),
                ("split_sizes", c_void_p), ("padded_offsets", c_void_p),
                ("a", c_void_p), ("b", c_void_p), ("b_stride", c_int64),
                ("c", c_void_p), ("workspace", c_void_p),
                ("workspace_bytes", c_size_t), ("prec", c_int32),
                ("a_s", c_void_p), ("b_s", c_void_p), ("b_s_stride", c_int64),
                ("err_flag", c_void_p)]


class GluArgs(ctypes.Structure):
    _fields_ = [("direction", c_int32), ("E", c_int32), ("I", c_int32),
                ("M_cap", c_int64), ("act", ActParams),
                ("split_sizes", c_void_p), ("padded_offsets", c_void_p),
                ("probs_p", c_void_p), ("z", c_void_p), ("a", c_void_p),
                ("amax", c_void_p), ("da", c_void_p), ("dz", c_void_p),
                ("dprobs_p", c_void_p)]


class RouterArgs(ctypes.Structure):
    _fields_ = [("T", c_int32), ("E", c_int32), ("k", c_int32),
                ("logits", c_void_p), ("expert_idx", c_void_p),
                ("probs", c_void_p)]


class RouterRouteArgs(ctypes.Structure):
    _fields_ = [("T", c_int32), ("E_total", c_int32), ("k", c_int32),
                ("E", c_int32), ("first_expert", c_int32), ("M_cap", c_int64),
                ("logits", c_void_p), ("expert_idx", c_void_p), ("probs", c_void_p),
                ("split_sizes", c_void_p), ("offsets", c_void_p),
                ("padded_offsets", c_void_p), ("row_id_map", c_void_p),
                ("row_src", c_void_p), ("probs_p", c_void_p), ("err_flag", c_void_p),
                ("workspace", c_void_p), ("workspace_bytes", c_size_t)]


class WgradArgs(ctypes.Structure):
    _fields_ = [("E", c_int32), ("H", c_int32), ("I", c_int32),
                ("gated", c_int32), ("M_cap", c_int64), ("prec", c_int32),
                ("cu_margin", c_int32), ("split_sizes", c_void_p),
                ("padded_offsets", c_void_p),
                ("dz", c_void_p), ("xp", c_void_p), ("dyp", c_void_p),
                ("a", c_void_p),
                ("dzT_q", c_void_p), ("dzT_s", c_void_p),
                ("xpT_q", c_void_p), ("xpT_s", c_void_p),
                ("dypT_q", c_void_p), ("dypT_s", c_void_p),
                ("aT_q", c_void_p), ("aT_s", c_void_p),
                ("dw1", c_void_p), ("dw2", c_void_p),
                ("timing_events", c_void_p * 3), ("err_flag", c_void_p)]


# ---- library loading ------------------------------------------------------
_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library.  Raises if it is not built: there is no
    other implementation to fall back to."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(lib_path):
            raise ImportError(
                f"{lib_path} is missing: build it with "
                "`python -m moe_grouped_mlp_amd.build`")
        L = ctypes.CDLL(lib_path)
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [c_int]
        L.moe_gmlp_version.restype = c_int
        L.moe_weight_repack_interleave.restype = c_int
        L.moe_weight_repack_interleave.argtypes = [
            c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, c_void_p]
        L.moe_permute_workspace_size.restype = c_size_t
        L.moe_permute_workspace_size.argtypes = [c_int, c_int]
        L.moe_router_route_workspace_size.restype = c_size_t
        L.moe_router_route_workspace_size.argtypes = [c_int, c_int, c_int]
        L.moe_mx_scale_offset.restype = c_int64
        L.moe_mx_scale_offset.argtypes = [c_int64, c_int64, c_int64]
        L.moe_clock_tick_rate_hz.restype = c_int64
        L.moe_clock_tick_rate_hz.argtypes = []
        L.moe_gemm_clock_trace.restype = c_int
        L.moe_gemm_clock_trace.argtypes = [c_void_p, c_int]
        L.moe_bench_occupy.restype = c_int
        L.moe_bench_occupy.argtypes = [c_int, c_int64, c_void_p]
        L.moe_grouped_gemm_workspace_size.restype = c_size_t
        L.moe_grouped_gemm_workspace_size.argtypes = [c_int]
        L.moe_grouped_mlp_workspace_size.restype = c_size_t
        L.moe_grouped_mlp_workspace_size.argtypes = [
            c_int, c_int, c_int, c_int64, c_int, c_int]
        for name, st in (("moe_permute", PermuteArgs),
                         ("moe_unpermute", UnpermuteArgs),
                         ("moe_quantize_mxfp8", QuantArgs),
                         ("moe_quantize_mxfp4", QuantArgs),
                         ("moe_grouped_mlp_fwd", FwdArgs),
                         ("moe_grouped_mlp_bwd", BwdArgs),
                         ("moe_grouped_mlp_bwd_noalloc", BwdArgs),
                         ("moe_grouped_mlp_wgrad", WgradArgs),
                         ("moe_router_topk", RouterArgs),
                         ("moe_router_route", RouterRouteArgs),
                         ("moe_grouped_gemm", GemmArgs),
                         ("moe_glu_unfused", GluArgs)):
            f = getattr(L, name)
            f.restype = c_int
            f.argtypes = [ctypes.POINTER(st), c_void_p]
        _LIB = L
    return _LIB


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MoeError(fn, status, lib().moe_status_string(status).decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _events(evs):
    arr = (c_void_p * 3)()
    for i, e in enumerate(evs or ()):
        if e is not None:
            arr[i] = e if isinstance(e, int) else e.cuda_event
    return arr


def act_params(act: int = ACT_SWIGLU, beta: float = 1.0,
               clamp: float | None = None, gate_lo: float = -math.inf,
               gate_hi: float = math.inf, lin_lo: float = -math.inf,
               lin_hi: float = math.inf, lin_offset: float = 0.0) -> ActParams:
    if clamp is not None:
        gate_lo, gate_hi, lin_lo, lin_hi = -clamp, clamp, -clamp, clamp
    return ActParams(act, beta, gate_lo, gate_hi, lin_lo, lin_hi, lin_offset)


# ---- entry points ---------------------------------------------------------
def moe_weight_repack_interleave(w1, w1i, E, I, H, block=INTERLEAVE,
                                 inverse=False, stream=None):
    _check("moe_weight_repack_interleave",
           lib().moe_weight_repack_interleave(_ptr(w1), _ptr(w1i), E, I, H,
                                              block, int(bool(inverse)),
                                              _stream(stream)))


def moe_permute_workspace_size(T, E) -> int:
    return lib().moe_permute_workspace_size(T, E)


def moe_permute(*, flags, T, k, E, H, M_cap, split_sizes, padded_offsets,
                row_id_map, first_expert=0, expert_idx=None, probs=None,
                offsets=None, row_src=None, probs_p=None, x=None, xp=None,
                xp_q=None, xp_s=None, err_flag=None, workspace=None,
                stream=None):
    a = PermuteArgs(flags, T, k, E, first_expert, H, M_cap, _ptr(expert_idx),
                    _ptr(probs), _ptr(split_sizes), _ptr(offsets),
                    _ptr(padded_offsets), _ptr(row_id_map), _ptr(row_src),
                    _ptr(probs_p), _ptr(x), _ptr(xp), _ptr(xp_q), _ptr(xp_s),
                    _ptr(err_flag), _ptr(workspace), _nbytes(workspace))
    _check("moe_permute", lib().moe_permute(ctypes.byref(a), _stream(stream)))


def moe_unpermute(*, T, k, H, M_cap, row_id_map, yp, out, dprobs_p=None,
                  dprobs=None, stream=None):
    a = UnpermuteArgs(T, k, H, M_cap, _ptr(row_id_map), _ptr(yp), _ptr(out),
                      _ptr(dprobs_p), _ptr(dprobs))
    _check("moe_unpermute",
           lib().moe_unpermute(ctypes.byref(a), _stream(stream)))


def moe_quantize_mxfp8(*, mode, batch, rows, cols, x, q, s, x_stride=0,
                       amax=None, qT=None, sT=None, live=None, stream=None):
    a = QuantArgs(mode, batch, rows, cols, x_stride, _ptr(x), _ptr(q), _ptr(s),
                  _ptr(amax), _ptr(qT), _ptr(sT), _ptr(live))
    _check("moe_quantize_mxfp8",
           lib().moe_quantize_mxfp8(ctypes.byref(a), _stream(stream)))


def moe_quantize_mxfp4(*, batch, rows, cols, x, q, s, mode=QUANT_ROW, x_stride=0,
                       qT=None, sT=None, live=None, stream=None):
    a = QuantArgs(mode, batch, rows, cols, x_stride, _ptr(x), _ptr(q), _ptr(s), None,
                  _ptr(qT), _ptr(sT), _ptr(live))
    _check("moe_quantize_mxfp4",
           lib().moe_quantize_mxfp4(ctypes.byref(a), _stream(stream)))


def moe_grouped_mlp_workspace_size(E, H, I, M_cap, prec=PREC_BF16,
                                   act=ACT_SWIGLU) -> int:
    return lib().moe_grouped_mlp_workspace_size(E, H, I, M_cap, prec, act)


def moe_mx_scale_offset(r, b, K) -> int:
    return lib().moe_mx_scale_offset(r, b, K)


def moe_grouped_mlp_fwd(*, E, H, I, M_cap, split_sizes, padded_offsets,
                        probs_p, yp, xp=None, w1i=None, w2=None, a=None,
                        z=None, amax=None, act=None, prec=PREC_BF16,
                        cu_margin=0, w1_stride=0, w2_stride=0, err_flag=None,
                        timing_events=None, xp_q=None, xp_s=None, w1_q=None,
                        w1_s=None, w2_q=None, w2_s=None, a_q=None, a_s=None,
                        aT_q=None, aT_s=None, workspace=None, bias1=None, stream=None):
    args = FwdArgs(E, H, I, M_cap, prec, act or act_params(), cu_margin,
                   _ptr(split_sizes), _ptr(padded_offsets), _ptr(probs_p),
                   _ptr(xp), _ptr(w1i), _ptr(w2), w1_stride, w2_stride,
                   _ptr(z), _ptr(a), _ptr(amax), _ptr(yp), _ptr(err_flag),
                   _events(timing_events), _ptr(xp_q), _ptr(xp_s), _ptr(w1_q),
                   _ptr(w1_s), _ptr(w2_q), _ptr(w2_s), _ptr(a_q), _ptr(a_s),
                   _ptr(aT_q), _ptr(aT_s), _ptr(workspace), _nbytes(workspace),
                   _ptr(bias1))
    _check("moe_grouped_mlp_fwd",
           lib().moe_grouped_mlp_fwd(ctypes.byref(args), _stream(stream)))


def moe_grouped_mlp_bwd(*, E, H, I, M_cap, split_sizes, padded_offsets,
                        probs_p, z, dprobs_p, dxp, workspace, dyp=None,
                        w2=None, w1i=None, dz=None, act=None, prec=PREC_BF16,
                        cu_margin=0, w1_stride=0, w2_stride=0, err_flag=None,
                        timing_events=None, dyp_q=None, dyp_s=None,
                        w2t_q=None, w2t_s=None, w1t_q=None, w1t_s=None,
                        dz_q=None, dz_s=None, dzT_q=None, dzT_s=None,
                        bias1=None, stream=None):
    args = BwdArgs(E, H, I, M_cap, prec, act or act_params(), cu_margin,
                   _ptr(split_sizes), _ptr(padded_offsets), _ptr(probs_p),
                   _ptr(dyp), _ptr(w2), _ptr(z), _ptr(w1i), w1_stride,
                   w2_stride, _ptr(dz), _ptr(dprobs_p), _ptr(dxp),
                   _ptr(err_flag), _ptr(workspace), _nbytes(workspace),
                   _events(timing_events), _ptr(dyp_q), _ptr(dyp_s),
                   _ptr(w2t_q), _ptr(w2t_s), _ptr(w1t_q), _ptr(w1t_s),
                   _ptr(dz_q), _ptr(dz_s), _ptr(dzT_q), _ptr(dzT_s), _ptr(bias1))
    _check("moe_grouped_mlp_bwd",
           lib().moe_grouped_mlp_bwd(ctypes.byref(args), _stream(stream)))


def moe_grouped_mlp_bwd_noalloc(*, E, H, I, M_cap, split_sizes, padded_offsets,
                                probs_p, z, dprobs_p, dxp, dyp=None, w2=None, w1i=None,
                                dz=None, act=None, prec=PREC_BF16, cu_margin=0,
                                w1_stride=0, w2_stride=0, err_flag=None,
                                timing_events=None, dyp_q=None, dyp_s=None,
                                w2t_q=None, w2t_s=None, w1t_q=None, w1t_s=None,
                                dz_q=None, dz_s=None, dzT_q=None, dzT_s=None,
                                bias1=None, stream=None):
    """moe_grouped_mlp_bwd without a workspace argument: the library's fixed
    per-device scratch array serves as the workspace (for callers that
    cannot allocate)."""
    args = BwdArgs(E, H, I, M_cap, prec, act or act_params(), cu_margin,
                   _ptr(split_sizes), _ptr(padded_offsets), _ptr(probs_p),
                   _ptr(dyp), _ptr(w2), _ptr(z), _ptr(w1i), w1_stride,
                   w2_stride, _ptr(dz), _ptr(dprobs_p), _ptr(dxp),
                   _ptr(err_flag), None, 0,
                   _events(timing_events), _ptr(dyp_q), _ptr(dyp_s),
                   _ptr(w2t_q), _ptr(w2t_s), _ptr(w1t_q), _ptr(w1t_s),
                   _ptr(dz_q), _ptr(dz_s), _ptr(dzT_q), _ptr(dzT_s), _ptr(bias1))
    _check("moe_grouped_mlp_bwd_noalloc",
           lib().moe_grouped_mlp_bwd_noalloc(ctypes.byref(args), _stream(stream)))


def moe_grouped_mlp_wgrad(*, E, H, I, M_cap, split_sizes, padded_offsets,
                          gated=True, prec=PREC_BF16, cu_margin=0, dz=None,
                          xp=None, dyp=None, a=None, dzT_q=None, dzT_s=None,
                          xpT_q=None, xpT_s=None, dypT_q=None, dypT_s=None,
                          aT_q=None, aT_s=None, dw1=None, dw2=None,
                          timing_events=None, err_flag=None, stream=None):
    args = WgradArgs(E, H, I, int(bool(gated)), M_cap, prec, cu_margin,
                     _ptr(split_sizes), _ptr(padded_offsets), _ptr(dz),
                     _ptr(xp), _ptr(dyp), _ptr(a), _ptr(dzT_q), _ptr(dzT_s),
                     _ptr(xpT_q), _ptr(xpT_s), _ptr(dypT_q), _ptr(dypT_s),
                     _ptr(aT_q), _ptr(aT_s), _ptr(dw1), _ptr(dw2),
                     _events(timing_events), _ptr(err_flag))
    _check("moe_grouped_mlp_wgrad",
           lib().moe_grouped_mlp_wgrad(ctypes.byref(args), _stream(stream)))


def moe_router_topk(*, T, E, k, logits, expert_idx, probs, stream=None):
    args = RouterArgs(T, E, k, _ptr(logits), _ptr(expert_idx), _ptr(probs))
    _check("moe_router_topk", lib().moe_router_topk(ctypes.byref(args), _stream(stream)))


def moe_router_route_workspace_size(T, E_total, E) -> int:
    return lib().moe_router_route_workspace_size(T, E_total, E)


def moe_router_route(*, T, E_total, k, E, M_cap, logits, expert_idx, probs, split_sizes,
                     padded_offsets, row_id_map, row_src, probs_p, workspace, offsets=None,
                     first_expert=0, err_flag=None, stream=None):
    """Router and routing metadata in one launch; the workspace's first 4096
    bytes must be zero before the first call (each call leaves them as the
    next call expects)."""
    args = RouterRouteArgs(T, E_total, k, E, first_expert, M_cap, _ptr(logits),
                           _ptr(expert_idx), _ptr(probs), _ptr(split_sizes), _ptr(offsets),
                           _ptr(padded_offsets), _ptr(row_id_map), _ptr(row_src),
                           _ptr(probs_p), _ptr(err_flag), _ptr(workspace), _nbytes(workspace))
    _check("moe_router_route", lib().moe_router_route(ctypes.byref(args), _stream(stream)))


def moe_clock_tick_rate_hz() -> int:
    return lib().moe_clock_tick_rate_hz()


CLOCK_MAX_WORKGROUPS = 1024


def moe_gemm_clock_trace(records=None, slots=1):
    """Grouped-GEMM launches that follow write per-workgroup {cycles, ticks}
    into records (device int64 [slots][CLOCK_MAX_WORKGROUPS][2]) in turn;
    records=None clears the trace."""
    _check("moe_gemm_clock_trace", lib().moe_gemm_clock_trace(_ptr(records), slots))


def moe_bench_occupy(*, workgroups, ticks, stream=None):
    """Hold `workgroups` CUs busy for `ticks` of the constant-rate counter."""
    _check("moe_bench_occupy", lib().moe_bench_occupy(workgroups, ticks, _stream(stream)))


def moe_grouped_gemm_workspace_size(dynamic=True) -> int:
    return lib().moe_grouped_gemm_workspace_size(int(bool(dynamic)))


def moe_grouped_gemm(*, E, N, K, M_cap, split_sizes, padded_offsets, a, b, c,
                     b_kn=False, b_stride=0, cu_margin=0, workspace=None,
                     prec=PREC_BF16, a_s=None, b_s=None, b_s_stride=0,
                     err_flag=None, stream=None):
    args = GemmArgs(E, N, K, M_cap, int(bool(b_kn)), cu_margin,
                    _ptr(split_sizes), _ptr(padded_offsets), _ptr(a), _ptr(b),
                    b_stride, _ptr(c), _ptr(workspace), _nbytes(workspace), prec,
                    _ptr(a_s), _ptr(b_s), b_s_stride, _ptr(err_flag))
    _check("moe_grouped_gemm", lib().moe_grouped_gemm(ctypes.byref(args), _stream(stream)))


def moe_glu_unfused(*, direction, E, I, M_cap, split_sizes, padded_offsets,
                    probs_p, z, act=None, a=None, amax=None, da=None, dz=None,
                    dprobs_p=None, stream=None):
    args = GluArgs(direction, E, I, M_cap, act or act_params(), _ptr(split_sizes),
                   _ptr(padded_offsets), _ptr(probs_p), _ptr(z), _ptr(a),
                   _ptr(amax), _ptr(da), _ptr(dz), _ptr(dprobs_p))
    _check("moe_glu_unfused", lib().moe_glu_unfused(ctypes.byref(args), _stream(stream)))
