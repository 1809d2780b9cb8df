// Gated activations and their derivatives, as the fused epilogues and the
// unfused activation kernels evaluate them ("Boosting MoE Training
// Throughput with Advanced Fusion Kernels", § "Optimizing GLU activations
// with fused GEMM epilogues", eq. SwiGLU; GeGLU and the clamp option from
// the list of supported activation patterns).
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

// 1 / (1 + e^-x) with the hardware reciprocal (v_rcp_f32, about 1 ulp)
// instead of an IEEE division: the result is rounded to bf16 or feeds
// products that are, so the few-ulp fp32 error never shows.
MOE_DEV float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// SwiGLU with no clamp and no linear offset (gate_lo = lin_lo = -inf,
// gate_hi = lin_hi = +inf, lin_offset = 0): an internal activation code with
// its own kernel instantiation that skips the clamps and range flags.
constexpr int kActSwigluFree = 0x100;
// flag on a GEMM kernel's activation parameter: the layer has an FC1 bias
constexpr int kActBias = 0x200;
// flag on an MXFP4 GLU / dGLU kernel's activation parameter: the epilogue
// also writes the transposed MXFP4 copy (the instantiation without it keeps
// that code, and its registers and LDS, out of the kernel)
constexpr int kActTr = 0x400;
inline bool act_unclamped(const ActP& p) {
  return p.glo == -__builtin_inff() && p.llo == -__builtin_inff() &&
         p.ghi == __builtin_inff() && p.lhi == __builtin_inff() && p.loff == 0.0f;
}

// Unscaled gated activation s and its partial derivatives.
struct GluVal {
  float s;     // act(g) * u
  float f;     // act(g)
  float df;    // act'(g)
  float u;     // clamped linear half (+ offset)
  bool g_in, u_in;
};

template <int ACT>
MOE_DEV GluVal glu_eval(float g_pre, float u_pre, const ActP& p) {
  GluVal r;
  if constexpr (ACT == kActSwigluFree) {
    const float sg = sigmoid_f(p.beta * g_pre);
    r.f = g_pre * sg;
    r.df = sg * (1.0f + p.beta * g_pre * (1.0f - sg));
    r.u = u_pre;
    r.g_in = r.u_in = true;
    r.s = r.f * r.u;
    return r;
  }
  // a finite input lies inside [lo, hi] (bounds included) exactly when
  // clamping leaves it unchanged: one compare instead of two and an and
  float g = fminf(fmaxf(g_pre, p.glo), p.ghi);
  const float uc = fminf(fmaxf(u_pre, p.llo), p.lhi);
  r.u = uc + p.loff;
  r.g_in = g == g_pre;
  r.u_in = uc == u_pre;
  if constexpr (ACT == MOE_ACT_GEGLU) {
    const float kInvSqrt2 = 0.70710678118654752f;
    const float kInvSqrt2Pi = 0.39894228040143268f;
    float cdf = 0.5f * (1.0f + erff(g * kInvSqrt2));
    r.f = g * cdf;
    r.df = cdf + g * kInvSqrt2Pi * __expf(-0.5f * g * g);
  } else {
    float sg = sigmoid_f(p.beta * g);
    r.f = g * sg;
    r.df = sg * (1.0f + p.beta * g * (1.0f - sg));
  }
  r.s = r.f * r.u;
  return r;
}

}  // namespace moe
