// attn_common.h -- split-K decode attention pieces shared by the rewrite kernel (which
// attends the view rows while it copies them) and the tier attention kernel.
//
// Layout: a wavefront holds 4 rows at a time, 16 lanes per row, 8 head dims per lane.
// Logits are kept in base 2 (queries pre-scaled by log2(e) / sqrt(D)); each 16-lane row
// group runs its own online softmax; at the end the four groups of a wavefront and the
// four wavefronts of the workgroup are merged into one partial (m, l, acc[128]) per
// query, which a combine kernel reduces across partials.
#pragma once

#include "hardkv_internal.h"

namespace hardkv {

template <int G>
struct AttnState {
  float m[G], l[G], acc[G][8];
  HK_DEV void init() {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;
    }
  }
};

HK_DEV float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// one row (the same row in all 16 lanes of the group); logit = (q . k) * kscale + bias,
// value v.  Called by every lane of the wavefront; rows with act == false add nothing.
template <int G>
HK_DEV void attn_row(AttnState<G> &st, const float (&qs)[G][8], const float (&k)[8],
                     const float (&v)[8], float kscale, float bias, bool act) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float d = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) d = __builtin_fmaf(qs[g][i], k[i], d);
    d += dpp<DPP_XOR1>(d);
    d += dpp<DPP_XOR2>(d);
    d += dpp<DPP_HALF_MIRROR>(d);
    d += dpp<DPP_MIRROR>(d);
    const float lg = act ? __builtin_fmaf(d, kscale, bias) : -INFINITY;
    const float mn = fmaxf(st.m[g], lg);
    const float sc = (st.m[g] == mn) ? 1.0f : exp2_fast(st.m[g] - mn);
    const float p = act ? exp2_fast(lg - mn) : 0.0f;
    st.l[g] = __builtin_fmaf(st.l[g], sc, p);
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[g][i] = __builtin_fmaf(p, v[i], st.acc[g][i] * sc);
    st.m[g] = mn;
  }
}

HK_DEV float merge_factor(float m, float mn) { return (m == -INFINITY) ? 0.0f : exp2_fast(m - mn); }

// merge the four 16-lane groups of each wavefront, then the four wavefronts; write the
// partial [G][2 + HD] = (m, l, acc) to dst.  Must be reached by all threads.
template <int G>
HK_DEV void attn_write_partial(AttnState<G> &st, float *dst, float (*s_part)[G][2 + HD]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, sub = lane & 15;
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float m2 = __shfl_xor(st.m[g], off);
      const float l2 = __shfl_xor(st.l[g], off);
      const float mn = fmaxf(st.m[g], m2);
      const float f1 = merge_factor(st.m[g], mn), f2 = merge_factor(m2, mn);
      st.l[g] = st.l[g] * f1 + l2 * f2;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float a2 = __shfl_xor(st.acc[g][i], off);
        st.acc[g][i] = st.acc[g][i] * f1 + a2 * f2;
      }
      st.m[g] = mn;
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (sub == 0) {
        s_part[wave][g][0] = st.m[g];
        s_part[wave][g][1] = st.l[g];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) s_part[wave][g][2 + sub * 8 + i] = st.acc[g][i];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * HD; idx += NTHREADS) {
    const int g = idx / HD, d = idx - g * HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_part[w][g][0]);
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = merge_factor(s_part[w][g][0], M);
      L += s_part[w][g][1] * f;
      A += s_part[w][g][2 + d] * f;
    }
    float *o = dst + (size_t)g * (2 + HD);
    o[2 + d] = A;
    if (d == 0) {
      o[0] = M;
      o[1] = L;
    }
  }
}

// queries of KV head h, scaled to base-2 logits
template <typename T, int G>
HK_DEV void load_q_scaled(const Args &a, int b, int h, int sub, float (&qs)[G][8]) {
  constexpr int EB = Elem<T>::bytes;
  const char *qb = (const char *)a.q + (((int64_t)b * a.Hq + (int64_t)h * G) * HD + sub * 8) * EB;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    load8(qb + (size_t)g * HD * EB, qs[g], T{});
#pragma unroll
    for (int i = 0; i < 8; ++i) qs[g][i] *= a.att_scale;
  }
}

}  // namespace hardkv
