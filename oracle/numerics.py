"""Storage formats of the expert block, written out from their definitions.

TEST INFRASTRUCTURE ONLY: part of the CPU oracle. Nothing in the product
path may import it.

Formats (sources):
  * bf16: 1 sign, 8 exponent, 7 mantissa bits -- TE + BioNeMo Mixtral
    tutorial ("NVIDIA Transformer Engine 优化 MoE 生物基础模型训练"),
    § "Challenge 2: model size and activation memory", Fig. 3.
  * MXFP8: E4M3 elements with one shared E8M0 scale per 32 contiguous
    values -- same section and figure.  The E4M3 element is the OCP
    "E4M3FN" encoding: exponent bias 7, 3 mantissa bits, subnormals m*2^-9,
    no infinities, S.1111.111 is NaN, largest finite 448 = 1.75 * 2^8.
  * Scale rule (the pages only say "one scale per 32 values"; the rule
    taken is 2^(floor(log2 amax) - 8), 8 being the exponent of E4M3's
    largest finite value), clamped to E8M0's range 2^-127 .. 2^127.
  * MXFP4: E2M1 elements with one E8M0 scale per 32 values -- the 4-bit
    member of the same microscaling family, the MI355X counterpart of the
    NVFP4 recipe of the fusion-kernels blog ("Boosting MoE Training
    Throughput with Advanced Fusion Kernels", § "Fused MXFP8 and NVFP4
    quantization"), which names the format but not its rules.  E2M1:
    exponent bias 1, 1 mantissa bit, subnormals m * 0.5, no infinities or
    NaN, largest value 6 = 1.5 * 2^2.  Scale 2^(floor(log2 amax) - 2) (2
    being the exponent of 6); scaled values in (6, 8) saturate to 6.

Every conversion here works on exponents taken from the floating-point
representation (numpy.frexp / numpy.ldexp), never on a floating log2, and
rounds with numpy.rint (round half to even on float64), so each result is
the exact round-to-nearest-even of the float64 input.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- bf16 ----
BF16_MIN_EXP = -126        # smallest normal exponent
BF16_MANT_BITS = 7
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):     # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def f32_to_f64(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _round_to_grid(x: np.ndarray, sig_bits: int, min_exp: int) -> np.ndarray:
    """Round float64 x to `sig_bits` significant bits (RNE), with gradual
    underflow below 2^min_exp.  No overflow handling."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                 # |x| in [2^(e-1), 2^e)
    # quantum of the binade of x, floored at the subnormal quantum
    q = np.maximum(e - sig_bits, min_exp - (sig_bits - 1))
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), returned as float64.

    Values whose rounded magnitude reaches 2^128 become +-inf; NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        r = _round_to_grid(x, BF16_MANT_BITS + 1, BF16_MIN_EXP)
        r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)
        r = np.where(np.isfinite(x), r, x)
    return r


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 values ALREADY on the bf16 grid -> uint16 bit patterns."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------- E4M3 ----
E4M3_MAX = 448.0
E4M3_EMAX = 8              # exponent of the largest finite value
E4M3_MIN_EXP = -6          # smallest normal exponent
E4M3_MANT_BITS = 3


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 E4M3 codes -> float64 (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(ef == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, ef - 7))
    mag = np.where((ef == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float64 -> E4M3 code, round to nearest even, saturating at +-448.

    The sign is kept (so -0 and negative values that round to zero give
    0x80).  NaN and +-inf inputs give NaN codes (0x7F / 0xFF).
    """
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.abs(v)
    with np.errstate(invalid="ignore", over="ignore"):
        r = _round_to_grid(a, E4M3_MANT_BITS + 1, E4M3_MIN_EXP)
        r = np.minimum(r, E4M3_MAX)
    finite = np.isfinite(a)
    r = np.where(finite, r, 0.0)
    _, e = np.frexp(r)
    e2 = e - 1                              # r in [2^e2, 2^(e2+1))
    sub = r < 2.0 ** E4M3_MIN_EXP
    m_sub = np.ldexp(r, 9)                  # r / 2^-9, integer 0..7
    m_norm = np.ldexp(r, -e2) * 8.0 - 8.0   # mantissa 0..7
    code = np.where(sub, m_sub, ((e2 + 7) << 3) + m_norm)
    code = code.astype(np.int64)
    code = np.where(finite, code, 0x7F)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


# ---------------------------------------------------------------- MXFP8 ---
MX_BLOCK = 32


def e8m0_exponent(amax: np.ndarray) -> np.ndarray:
    """Shared-scale exponent for blocks with absolute maximum `amax`:
    floor(log2 amax) - 8, clamped to [-127, 127]; 0 -> -127.

    floor(log2 amax) is read from the float64 exponent field via frexp.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)                   # amax in [2^(e-1), 2^e)
    ex = (e - 1) - E4M3_EMAX
    ex = np.where(amax > 0, ex, -127)
    return np.clip(ex, -127, 127).astype(np.int64)


def mx_quantize(x: np.ndarray, axis: int = -1, block: int = MX_BLOCK):
    """MXFP8-encode float64 `x` in blocks of `block` along `axis`.

    Returns (codes uint8, same shape as x; scales uint8 E8M0 codes, shape of
    x with that axis divided by `block`).  A block holding NaN or inf gets
    scale code 0xFF and NaN element codes.
    """
    x = np.asarray(x, dtype=np.float64)
    xm = np.moveaxis(x, axis, -1)
    n = xm.shape[-1]
    if n % block:
        raise ValueError(f"axis length {n} is not a multiple of {block}")
    blk = xm.reshape(xm.shape[:-1] + (n // block, block))
    amax = np.max(np.abs(blk), axis=-1)
    bad = ~np.isfinite(amax)
    ex = e8m0_exponent(np.where(bad, 0.0, amax))
    scaled = np.ldexp(blk, -ex[..., None])
    codes = e4m3_encode(scaled)
    codes = np.where(bad[..., None], codes | 0x7F, codes).astype(np.uint8)
    scales = np.where(bad, 0xFF, ex + 127).astype(np.uint8)
    codes = np.moveaxis(codes.reshape(xm.shape), -1, axis)
    scales = np.moveaxis(scales, -1, axis)
    return codes, scales


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, axis: int = -1,
                  block: int = MX_BLOCK) -> np.ndarray:
    """Inverse of mx_quantize (exact, float64)."""
    cm = np.moveaxis(np.asarray(codes, dtype=np.uint8), axis, -1)
    sm = np.moveaxis(np.asarray(scales, dtype=np.uint8), axis, -1)
    n = cm.shape[-1]
    vals = e4m3_decode(cm).reshape(cm.shape[:-1] + (n // block, block))
    ex = sm.astype(np.int64) - 127
    out = np.ldexp(vals, ex[..., None])
    out = np.where((sm == 0xFF)[..., None], np.nan, out)
    return np.moveaxis(out.reshape(cm.shape), -1, axis)


def mx_round(x: np.ndarray, axis: int = -1) -> np.ndarray:
    """dequant(quant(x)): the values an MXFP8 operand carries."""
    c, s = mx_quantize(x, axis)
    return mx_dequantize(c, s, axis)


# ---------------------------------------------------------------- MXFP4 ---
E2M1_MAX = 6.0
E2M1_EMAX = 2              # exponent of the largest value
E2M1_MIN_EXP = 0           # smallest normal exponent (1.0)
E2M1_MANT_BITS = 1


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit E2M1 codes (0..15, in any integer array) -> float64."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    ef = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(ef == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, ef - 1))
    return sign * mag


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """float64 -> E2M1 code (uint8 0..15), round to nearest even,
    saturating at +-6; the sign is kept (-0 gives 0x8).  Inputs must be
    finite."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("E2M1 has no encoding for NaN or inf")
    neg = np.signbit(v)
    r = _round_to_grid(np.abs(v), E2M1_MANT_BITS + 1, E2M1_MIN_EXP)
    r = np.minimum(r, E2M1_MAX)
    _, e = np.frexp(r)
    e2 = e - 1                              # r in [2^e2, 2^(e2+1))
    sub = r < 1.0
    m_sub = r * 2.0                         # 0 or 1 (0.5 steps)
    m_norm = np.ldexp(r, -e2) * 2.0 - 2.0   # mantissa bit
    code = np.where(sub, m_sub, ((e2 + 1) << 1) + m_norm).astype(np.int64)
    return (code | np.where(neg, 0x8, 0)).astype(np.uint8)


def mxfp4_quantize(x: np.ndarray, axis: int = -1, block: int = MX_BLOCK):
    """MXFP4-encode finite float64 `x` in blocks of `block` along `axis`.

    Returns (codes uint8 0..15, one per value, same shape as x; scales
    uint8 E8M0 codes, that axis divided by `block`).  The scale exponent is
    floor(log2 amax) - 2, clamped to [-127, 127]; an all-zero block gets
    scale code 0 and zero codes."""
    x = np.asarray(x, dtype=np.float64)
    xm = np.moveaxis(x, axis, -1)
    n = xm.shape[-1]
    if n % block:
        raise ValueError(f"axis length {n} is not a multiple of {block}")
    blk = xm.reshape(xm.shape[:-1] + (n // block, block))
    amax = np.max(np.abs(blk), axis=-1)
    _, e = np.frexp(amax)                   # amax in [2^(e-1), 2^e)
    ex = np.where(amax > 0, (e - 1) - E2M1_EMAX, -127)
    ex = np.clip(ex, -127, 127).astype(np.int64)
    codes = e2m1_encode(np.ldexp(blk, -ex[..., None]))
    scales = (ex + 127).astype(np.uint8)
    codes = np.moveaxis(codes.reshape(xm.shape), -1, axis)
    return codes, np.moveaxis(scales, -1, axis)


def mxfp4_dequantize(codes: np.ndarray, scales: np.ndarray, axis: int = -1,
                     block: int = MX_BLOCK) -> np.ndarray:
    """Inverse of mxfp4_quantize (exact, float64)."""
    cm = np.moveaxis(np.asarray(codes), axis, -1)
    sm = np.moveaxis(np.asarray(scales, dtype=np.uint8), axis, -1)
    n = cm.shape[-1]
    vals = e2m1_decode(cm).reshape(cm.shape[:-1] + (n // block, block))
    out = np.ldexp(vals, (sm.astype(np.int64) - 127)[..., None])
    return np.moveaxis(out.reshape(cm.shape), -1, axis)


def mxfp4_round(x: np.ndarray, axis: int = -1) -> np.ndarray:
    """dequant(quant(x)): the values an MXFP4 operand carries."""
    c, s = mxfp4_quantize(x, axis)
    return mxfp4_dequantize(c, s, axis)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """4-bit codes along the last axis -> bytes, element 2i in the low
    nibble of byte i."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
