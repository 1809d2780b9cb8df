"""Pins of the oracle's storage formats (bf16, E4M3, E8M0 / MXFP8).

Each check compares the oracle with something other than itself: torch's own
casts (an independent library), hand-derived vectors from the format
definition (tests/golden), or a brute-force nearest-value search over a
decode table built here from the bit-field definition.
"""

import os

import numpy as np
import pytest
import torch

from oracle import numerics as nu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ bf16 --
def _torch_bf16_bits(f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_round_matches_torch_cast_on_fp32_inputs():
    rng = np.random.default_rng(11)
    # random bit patterns cover every exponent, subnormals and ties
    bits = rng.integers(0, 2 ** 32, size=400_000, dtype=np.uint64)
    f = bits.astype(np.uint32).view(np.float32)
    f = f[np.isfinite(f)]
    # add exact ties (lower 16 bits = 0x8000) and near-max values
    ties = (rng.integers(0, 2 ** 16, 5000, dtype=np.uint32) << 16) | 0x8000
    f = np.concatenate([f, ties.view(np.float32), np.float32([3.3e38, -3.4e38,
                                                              1e-45, -0.0])])
    f = f[np.isfinite(f)]
    ref = _torch_bf16_bits(f)
    got = nu.round_bf16(f.astype(np.float64))
    got_bits = nu.f64_to_bf16_bits(got)
    np.testing.assert_array_equal(got_bits, ref)


def test_bf16_round_is_direct_not_double_rounded():
    # 1 + 2^-8 + 2^-30 lies just above the bf16 tie 1 + 2^-8; a detour
    # through fp32 would land exactly on the tie and round down to 1.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert nu.round_bf16(np.float64(x)) == 1.0 + 2.0 ** -7
    assert nu.round_bf16(np.float64(1.0 + 2.0 ** -8)) == 1.0     # tie -> even
    assert nu.round_bf16(np.float64(1.0 + 3 * 2.0 ** -8)) == 1.0 + 2 ** -6
    assert np.isinf(nu.round_bf16(np.float64(2.0 ** 128 * 0.99999)))
    assert nu.round_bf16(np.float64(2.0 ** -134)) == 0.0          # tie -> 0
    assert nu.round_bf16(np.float64(3 * 2.0 ** -134)) == 2.0 ** -132


def test_bf16_decode_widening():
    bits = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    v = nu.bf16_to_f64(bits)
    fin = np.isfinite(v)
    np.testing.assert_array_equal(nu.f64_to_bf16_bits(v[fin]), bits[fin])
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double()
    np.testing.assert_array_equal(t.numpy()[fin], v[fin])


# ------------------------------------------------------------ E4M3 / MX --
def _e4m3_table():
    """All 256 E4M3FN codes decoded from the bit fields, written here
    independently of the oracle."""
    vals = []
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        E = (c >> 3) & 0xF
        m = c & 7
        if E == 15 and m == 7:
            vals.append(np.nan)
        elif E == 0:
            vals.append(s * m * 2.0 ** -9)
        else:
            vals.append(s * (1 + m / 8) * 2.0 ** (E - 7))
    return np.array(vals)


def _brute_scale_exp(amax: float) -> int:
    """floor(log2 amax) - 8 by walking powers of two, clamped to E8M0."""
    if amax == 0:
        return -127
    e = 0
    while 2.0 ** e > amax:
        e -= 1
    while 2.0 ** (e + 1) <= amax:
        e += 1
    return max(-127, min(127, e - 8))


def _brute_code(q: float, table: np.ndarray) -> int:
    """Nearest positive E4M3 code to |q| (ties to even mantissa), saturating
    at 448, with the sign of q."""
    pos = np.arange(0, 127)               # 0x00..0x7E, finite non-negative
    if abs(q) >= 448:
        c = 0x7E
    else:
        d = np.abs(table[pos] - abs(q))
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:
            best = [b for b in best if b % 2 == 0]
        c = int(pos[best[0]])
    return c | (0x80 if np.signbit(q) else 0)


def test_mx_golden_vectors():
    path = os.path.join(GOLDEN, "mxfp8_e4m3_vectors.txt")
    n = 0
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        amax_s, v_s, sc_s, c_s = line.split()
        amax, v = float.fromhex(amax_s), float.fromhex(v_s)
        blk = np.zeros(32)
        blk[0] = v
        if abs(v) != amax:
            blk[1] = amax
        codes, scales = nu.mx_quantize(blk[None, :], axis=1)
        assert scales[0, 0] == int(sc_s, 16), line
        assert codes[0, 0] == int(c_s, 16), line
        n += 1
    assert n >= 15


def test_e4m3_decode_matches_bitfield_table():
    tab = _e4m3_table()
    got = nu.e4m3_decode(np.arange(256, dtype=np.uint8))
    np.testing.assert_array_equal(np.isnan(got), np.isnan(tab))
    ok = ~np.isnan(tab)
    np.testing.assert_array_equal(got[ok], tab[ok])


@pytest.mark.parametrize("block_amax", [1.0, 2.0 ** -100, 2.0 ** 90])
def test_mx_exhaustive_bf16_vs_brute_force(block_amax):
    """Every finite bf16 value, placed in a block whose other element is
    +block_amax, against a brute-force search over the decode table."""
    tab = _e4m3_table()
    bits = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    v = nu.bf16_to_f64(bits)
    v = v[np.isfinite(v)]
    blk = np.zeros((v.size, 32))
    blk[:, 0] = v
    blk[:, 1] = block_amax
    codes, scales = nu.mx_quantize(blk, axis=1)
    amax = np.maximum(np.abs(v), block_amax)
    # brute force per distinct amax (most rows share block_amax)
    uniq, inv = np.unique(amax, return_inverse=True)
    exps = np.array([_brute_scale_exp(a) for a in uniq])[inv]
    np.testing.assert_array_equal(scales[:, 0].astype(np.int64), exps + 127)
    q = v / 2.0 ** exps.astype(np.float64)
    # vectorised brute force: nearest of the 127 non-negative finite codes
    pos = tab[:127]
    d = np.abs(np.abs(q)[:, None] - pos[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    even = cand & (np.arange(127)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    pick = np.where(np.abs(q) >= 448, 0x7E, pick)
    want = pick | np.where(np.signbit(q), 0x80, 0)
    np.testing.assert_array_equal(codes[:, 0].astype(np.int64), want)
    # spot-check the vectorised brute force against the scalar one
    rng = np.random.default_rng(3)
    for i in rng.integers(0, v.size, 300):
        assert _brute_code(q[i], tab) == want[i]


def test_e4m3_encode_matches_torch_float8_in_range():
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-448, 448, 200_000),
                        rng.standard_normal(100_000) * 2.0 ** -7,
                        rng.standard_normal(100_000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8)
    got = nu.e4m3_encode(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref.numpy())


def test_mx_roundtrip_and_nonfinite_blocks():
    rng = np.random.default_rng(9)
    x = nu.round_bf16(rng.standard_normal((64, 96)) * 3)
    c, s = nu.mx_quantize(x, axis=1)
    y = nu.mx_dequantize(c, s, axis=1)
    # E4M3 with a power-of-two block scale X: half a mantissa step (2^-4 of
    # the value) or half the smallest subnormal step (2^-10 X); values with
    # |v|/X above 448 saturate, losing at most 1/8 of their magnitude
    X = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)
    sat = np.abs(x) / X > 448
    bound = np.where(sat, np.abs(x) / 8, np.maximum(np.abs(x) * 2.0 ** -4,
                                                    X * 2.0 ** -10))
    assert np.all(np.abs(y - x) <= bound)
    assert np.all(np.abs(y[sat]) == 448 * X[sat])
    # along axis 0 gives the transpose of along axis 1 of x.T
    c0, s0 = nu.mx_quantize(x, axis=0)
    c1, s1 = nu.mx_quantize(x.T, axis=1)
    np.testing.assert_array_equal(c0, c1.T)
    np.testing.assert_array_equal(s0, s1.T)
    bad = np.zeros((1, 32))
    bad[0, 5] = np.nan
    c, s = nu.mx_quantize(bad, axis=1)
    assert s[0, 0] == 0xFF and np.all((c & 0x7F) == 0x7F)


# ---------------------------------------------------------------- MXFP4 ---
# E2M1 magnitudes of codes 0..7 as the OCP microscaling format lists them
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_matches_value_table():
    vals = nu.e2m1_decode(np.arange(16))
    np.testing.assert_array_equal(vals[:8], E2M1_TABLE)
    np.testing.assert_array_equal(vals[8:], [-v for v in E2M1_TABLE])
    assert np.signbit(vals[8])


def _e2m1_brute(v):
    """Nearest of the 16 codes by search; ties to the code whose mantissa
    bit is 0; magnitudes past 6 saturate."""
    out = []
    for x in v:
        a = min(abs(x), 6.0)
        d = [abs(a - t) for t in E2M1_TABLE]
        best = min(d)
        cands = [c for c in range(8) if d[c] == best]
        c = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        out.append(c | (8 if np.signbit(x) else 0))
    return np.array(out, dtype=np.uint8)


def test_e2m1_encode_matches_brute_force():
    rng = np.random.default_rng(0)
    mids = [(a + b) / 2 for a, b in zip(E2M1_TABLE, E2M1_TABLE[1:])]
    v = np.concatenate([rng.uniform(-9, 9, 4000), mids, [-m for m in mids],
                        E2M1_TABLE, [7.0, 8.0, 100.0, -0.0, 1e-9]])
    np.testing.assert_array_equal(nu.e2m1_encode(v), _e2m1_brute(v))


@pytest.mark.parametrize("k", [-130, -20, 0, 5, 120])
def test_mxfp4_scale_rule_closed_form(k):
    """A block whose largest magnitude lies in [4, 8) * 2^k gets scale 2^k
    (clamped to E8M0's range), and values on the E2M1 grid times that scale
    come back exactly."""
    rng = np.random.default_rng(k + 200)
    kc = max(k, -127)
    codes = rng.integers(0, 16, size=(3, 64)).astype(np.uint8)
    codes[:, 0] = 0x7          # 6: amax in every block
    codes[:, 32] = 0xE         # -4
    x = np.ldexp(nu.e2m1_decode(codes), kc)
    q, s = nu.mxfp4_quantize(x, axis=1)
    assert np.all(s == kc + 127)
    np.testing.assert_array_equal(nu.mxfp4_dequantize(q, s, axis=1), x)
    # amax 7.9 * 2^k still takes scale 2^k and saturates to 6
    y = x.copy()
    y[:, 0] = np.ldexp(7.9, kc)
    q2, s2 = nu.mxfp4_quantize(y, axis=1)
    assert np.all(s2 == kc + 127) and np.all(q2[:, 0] == 0x7)


def test_mxfp4_zero_block_and_blocks_along_axis():
    x = np.zeros((64, 2))
    x[33, 1] = 3.0
    q, s = nu.mxfp4_quantize(x, axis=0)
    assert s.shape == (2, 2) and s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0
    assert s[1, 1] == 126      # amax 3: 2^(floor(log2 3) - 2) = 2^-1
    np.testing.assert_array_equal(nu.mxfp4_dequantize(q, s, axis=0), x)


def test_pack_nibbles_low_first():
    c = np.array([[1, 2, 3, 15]], dtype=np.uint8)
    np.testing.assert_array_equal(nu.pack_nibbles(c), [[0x21, 0xF3]])
