// Shared device helpers for the gfx950 kernels of the MoE expert block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_gmlp.h"

#define MOE_DEV __device__ __forceinline__

typedef uint16_t bf16_t;  // bf16 bit pattern
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies

// ---------------------------------------------------------------- bf16 ---
MOE_DEV float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even done on the bit pattern with integer
// VALU operations (NaN kept quiet).  Same results as pack_bf16x2 for every
// finite value; the plain-store epilogue uses it because with it the register
// allocator keeps the MXFP8 K loop free of spill reloads.
MOE_DEV bf16_t f32_to_bf16_sw(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

MOE_DEV uint32_t pack_bf16x2_sw(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16_sw(lo)) |
         (static_cast<uint32_t>(f32_to_bf16_sw(hi)) << 16);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (lo in bits 0..15), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.  The kernels run with fp32 denormals enabled,
// so denormal inputs round like any other value; NaN stays NaN.
MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ---------------------------------------------------------------- waves --
MOE_DEV int lane_id() { return __lane_id(); }

MOE_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Wave maximum with no lane-address registers: xor 1 .. 16 inside each half
// wave by ds_swizzle (bit-mask mode: and 0x1f, xor m, an immediate pattern)
// and xor 32 by v_permlane32_swap.  Used in epilogues, where the address
// registers of a ds_bpermute-based shuffle would be kept across the K loop
// (spilled and reloaded after the stores).
MOE_DEV float wave_max_imm(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1f | (1 << 10))));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1f | (2 << 10))));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1f | (4 << 10))));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1f | (8 << 10))));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1f | (16 << 10))));
  // one of the two swapped words is the partner half's value, the other ours
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(v, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

MOE_DEV int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Raise *dst to max(*dst, v) for non-negative v: the IEEE order of
// non-negative floats equals the order of their bit patterns, so an integer
// atomicMax is exact and independent of arrival order.
MOE_DEV void atomic_max_nonneg(float* dst, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(dst), __float_as_uint(v));
}

MOE_DEV void set_err(int32_t* flag, int32_t bit) {
  if (flag) atomicOr(flag, bit);
}
