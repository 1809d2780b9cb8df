// Microscaling encoding helpers: MXFP8 (E4M3 values) and MXFP4 (E2M1
// values), one E8M0 scale per 32 values.
//
// The MXFP8 block rule: e = clamp(floor(log2 max|v|) - 8, -127, 127) (-127
// for an all-zero block), scale code e + 127, code = E4M3 round-to-nearest-
// even of v / 2^e saturated to +-448 (TE + BioNeMo Mixtral tutorial,
// § "Challenge 2: model size and activation memory", Fig. 3).  MXFP4 takes
// e = floor(log2 max|v|) - 2 (2 being the exponent of E2M1's largest value,
// 6) and the E2M1 round-to-nearest-even value of v / 2^e, saturated to +-6.
// The inputs are always bf16 values, so v / 2^e is exact and the only
// rounding is the conversion's: gfx950's scaled conversions of packed bf16
// words (v_cvt_scalef32_pk_{fp8,fp4}_bf16), which divide by a power-of-two
// scale and round to nearest even.  They were checked against the block
// rule on every finite bf16 value at every scale exponent: the FP4 one
// matches it, the FP8 one except that it gives NaN where the rule saturates
// (mx_codes4_bf16 corrects that).
#pragma once

#include "common.h"

namespace moe {

// e for a block whose largest magnitude is `amax` (a bf16 value, >= 0):
// floor(log2 amax) read from the exponent field; a zero or subnormal amax
// gives -127 after the clamp (the largest bf16 gives 119, so no upper clamp
// is ever reached).
MOE_DEV int mx_exponent(float amax) {
  const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu) - 127 - 8;
  return e < -127 ? -127 : e;
}

// The MXFP4 block exponent (see above), at least -127.
MOE_DEV int mx4_exponent(float amax) {
  const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu) - 127 - 2;
  return e < -127 ? -127 : e;
}

MOE_DEV uint8_t mx_scale_code(int e) { return static_cast<uint8_t>(e + 127); }

// 2^e as an fp32, exactly (2^-127 as the subnormal it is): the scale
// operand of the scaled conversions, which divide by it.
MOE_DEV float mx_scale_f32(int e) {
  return e > -127 ? __uint_as_float(static_cast<uint32_t>(e + 127) << 23)
                  : __uint_as_float(0x00400000u);
}

// Four bf16 values (two packed words, value 0 in the low half of w.x)
// divided by 2^e (scale = 2^e) -> four E4M3 codes, little-endian:
// v_cvt_scalef32_pk_fp8_bf16 divides by the scale and rounds to nearest
// even, but turns magnitudes past 464 (whose rounding would pass the
// largest code) into NaN, 0x7f / 0xff, where the block rule saturates at
// 448, 0x7e / 0xfe: those bytes are moved one code down.  The block
// exponent keeps |v| / 2^e below 512, so nothing else can come out as NaN.
typedef short short2_t __attribute__((ext_vector_type(2)));
MOE_DEV uint32_t mx_codes4_bf16(uint2 w, float scale) {
  short2_t r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, w.x), scale,
                                                false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, w.y), scale,
                                                true);
  const uint32_t c = __builtin_bit_cast(uint32_t, r);
  const uint32_t nan = ((c & 0x7f7f7f7fu) + 0x01010101u) & 0x80808080u;
  return c - (nan >> 7);
}

// Four bf16 values (two packed words, value 0 in the low half of w.x)
// divided by 2^e -> four E2M1 codes in the low 16 bits, value i in nibble
// i: v_cvt_scalef32_pk_fp4_bf16, which divides by the scale, rounds to
// nearest even and saturates at +-6 with the sign kept, the block rule.
MOE_DEV uint32_t mx4_codes4_bf16(uint2 w, float scale) {
  const uint32_t c =
      __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(bf16x2_t, w.x), scale, 0);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(bf16x2_t, w.y), scale,
                                                   1);
}

// The largest of a quad's four values (lanes 4 i .. 4 i + 3, every lane
// active): DPP quad permutations [1 0 3 2] and [2 3 0 1], no LDS traffic.
MOE_DEV uint32_t mx_quad_max(uint32_t m) {
  m = max(m, static_cast<uint32_t>(
                 __builtin_amdgcn_mov_dpp(static_cast<int>(m), 0xB1, 0xF, 0xF, false)));
  m = max(m, static_cast<uint32_t>(
                 __builtin_amdgcn_mov_dpp(static_cast<int>(m), 0x4E, 0xF, 0xF, false)));
  return m;
}

// |v| of a bf16 pattern as an ordered integer (bf16 magnitudes compare like
// their bit patterns).
MOE_DEV uint32_t bf16_abs_bits(uint32_t b) { return b & 0x7fffu; }

// Byte offset of the scale of row r, K-block b in the tiled scale layout of
// an [R][K] operand (see MOE_MX_BLOCK in moe_gmlp.h).
MOE_DEV int64_t mx_scale_off(int64_t r, int64_t b, int64_t K) {
  return ((r >> 5) * (K >> 6) + (b >> 1)) * 64 + (b & 1) * 32 + (r & 31);
}

}  // namespace moe
