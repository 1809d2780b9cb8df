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

// fp32 -> bf16, round to nearest even on the bit pattern (NaN kept quiet).
MOE_DEV bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) |
         (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// ---------------------------------------------------------------- waves --
MOE_DEV int lane_id() { return __lane_id(); }

MOE_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
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
