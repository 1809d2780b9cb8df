// The top-k router of one token (TE + BioNeMo Mixtral tutorial, Fig. 1: the
// sparse MoE block's router sends each token to k of E experts; the layer's
// configs route by "softmax then top-k").
//
// p = softmax(logits) over all E experts in fp32; the k largest logits are
// kept, in descending order, ties to the lower expert id, with probability
// p[e] (no renormalisation).  Softmax is monotone, so the selection compares
// the logits themselves and is exact.
//
// A token takes GS lanes (1, or 4 for wider routers), lane g of the group
// reading its share of the logits in ascending id order: with VEC the
// 4-logit blocks q = g, g + GS, ..., else logits g, g + GS, ....  Each lane
// takes the maximum and the sum of exp(logit - m) over its share (a
// fixed-order fp32 sum) and inserts every logit into a sorted list of KP
// entries (KP = k rounded up to 1, 2, 4 or 8; slots k .. KP-1 hold +inf so
// nothing is inserted there).  With GS = 4 the group then combines: maximum
// and sum by a butterfly over the quad (DPP quad permutes; a + b and b + a
// are equal, so every lane holds the same bits), and the k picks by k
// rounds in which the largest list head of the quad (ties to the lower id)
// is taken and popped from its lane's list.
#pragma once

#include "common.h"

namespace moe {

template <int KP>
struct RouterPicks {
  int32_t id[KP];   // every lane of the token's group holds all k picks
  float p[KP];
};

// One insertion step: a value arriving in ascending id order (within the
// lane) goes in front of the first entry it is larger than, and the entries
// from there on move down one slot (the last one drops out), so an equal
// value stays behind the earlier (lower) id.  Each slot is computed from
// the old values of itself and the slot above, bottom slot first.
template <int KP>
MOE_DEV void topk_insert(float (&bv)[KP], int (&bi)[KP], float v, int e) {
#pragma unroll
  for (int j = KP - 1; j >= 0; --j) {
    const bool gt = v > bv[j];
    const bool gt_above = j > 0 && v > bv[j > 0 ? j - 1 : 0];
    const float nv = gt_above ? bv[j > 0 ? j - 1 : 0] : v;
    const int ni = gt_above ? bi[j > 0 ? j - 1 : 0] : e;
    bv[j] = gt ? nv : bv[j];
    bi[j] = gt ? ni : bi[j];
  }
}

// Value of lane (l ^ 1) or (l ^ 2) inside the quad, by a DPP quad permute.
template <int X>
MOE_DEV int quad_xor(int v) {
  static_assert(X == 1 || X == 2, "quad xor");
  constexpr int ctrl = X == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] / [2,3,0,1]
  return __builtin_amdgcn_update_dpp(v, v, ctrl, 0xF, 0xF, false);
}
template <int X>
MOE_DEV float quad_xor(float v) {
  return __int_as_float(quad_xor<X>(__float_as_int(v)));
}

// row: the token's E logits (finite); g: the lane's index in its group;
// VEC: row is 16-byte aligned and E % 4 == 0.
template <int KP, int GS, bool VEC>
MOE_DEV RouterPicks<KP> router_token(const float* __restrict__ row, int E, int k, int g) {
  static_assert(GS == 1 || GS == 4, "lanes per token");
  float m = -__builtin_inff();
  if constexpr (VEC) {
    const float4* r4 = reinterpret_cast<const float4*>(row);
    for (int q = g; q < E / 4; q += GS) {
      const float4 v = r4[q];
      m = fmaxf(m, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
    }
  } else {
    for (int e = g; e < E; e += GS) m = fmaxf(m, row[e]);
  }
  if constexpr (GS == 4) {
    m = fmaxf(m, quad_xor<1>(m));
    m = fmaxf(m, quad_xor<2>(m));
  }
  float bv[KP];
  int bi[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    bv[j] = j < k ? -__builtin_inff() : __builtin_inff();
    bi[j] = 0x7fffffff;
  }
  float s = 0.0f;
  if constexpr (VEC) {
    const float4* r4 = reinterpret_cast<const float4*>(row);
    for (int q = g; q < E / 4; q += GS) {
      const float4 v = r4[q];
      s += __expf(v.x - m);
      s += __expf(v.y - m);
      s += __expf(v.z - m);
      s += __expf(v.w - m);
      topk_insert<KP>(bv, bi, v.x, 4 * q);
      topk_insert<KP>(bv, bi, v.y, 4 * q + 1);
      topk_insert<KP>(bv, bi, v.z, 4 * q + 2);
      topk_insert<KP>(bv, bi, v.w, 4 * q + 3);
    }
  } else {
    for (int e = g; e < E; e += GS) {
      const float v = row[e];
      s += __expf(v - m);
      topk_insert<KP>(bv, bi, v, e);
    }
  }
  RouterPicks<KP> r;
  if constexpr (GS == 1) {
    const float inv = 1.0f / s;
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      r.id[j] = bi[j];
      r.p[j] = __expf(bv[j] - m) * inv;
    }
  } else {
    s = s + quad_xor<1>(s);
    s = s + quad_xor<2>(s);
    const float inv = 1.0f / s;
    // k rounds: the largest head of the quad's four lists, ties to the
    // lower id, is taken and popped from its list.  A lane with fewer than
    // k logits keeps -inf heads, which never win while finite ones remain.
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      if (j < k) {
        float v = bv[0];
        int i = bi[0];
        {
          const float v2 = quad_xor<1>(v);
          const int i2 = quad_xor<1>(i);
          const bool take = v2 > v || (v2 == v && i2 < i);
          v = take ? v2 : v;
          i = take ? i2 : i;
        }
        {
          const float v2 = quad_xor<2>(v);
          const int i2 = quad_xor<2>(i);
          const bool take = v2 > v || (v2 == v && i2 < i);
          v = take ? v2 : v;
          i = take ? i2 : i;
        }
        r.id[j] = i;
        r.p[j] = __expf(v - m) * inv;
        const bool pop = bi[0] == i;
#pragma unroll
        for (int q = 0; q < KP; ++q) {
          const float nv = q + 1 < KP ? bv[q + 1 < KP ? q + 1 : q] : -__builtin_inff();
          const int ni = q + 1 < KP ? bi[q + 1 < KP ? q + 1 : q] : 0x7fffffff;
          bv[q] = pop ? nv : bv[q];
          bi[q] = pop ? ni : bi[q];
        }
      }
    }
  }
  return r;
}

// KP for k (1 <= k <= 8)
inline int router_kp(int k) { return k <= 1 ? 1 : k <= 2 ? 2 : k <= 4 ? 4 : 8; }
// lanes per token: one for up to 32 experts, four beyond
inline int router_gs(int E) { return E <= 32 ? 1 : 4; }

}  // namespace moe
