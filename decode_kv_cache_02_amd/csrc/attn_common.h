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


// one row (the same row in all 16 lanes of the group); logit = (q . k) * kscale + bias,
// value v.  Called by every lane of the wavefront; rows with act == false add nothing.
// (The condensed slots, which carry a scale and a bias per slot, take this form.)
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

// NR rows per 16-lane group at once (one from each load of a batch), in two phases so
// that a caller can release the key registers before the values are needed:
// attn_keys forms the NR logits, rescales the accumulators once to the new running
// maximum and leaves the rows' probabilities in p; attn_values adds the NR value rows.
template <typename T, int G, int NR>
HK_DEV void attn_keys(AttnState<G> &st, const float (&qs)[G][8], const Raw8<T> (&kr)[NR],
                      const bool (&act)[NR], float (&p)[G][NR]) {
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    float kf[8];
    raw_to_f(kr[j], kf);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float d = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) d = __builtin_fmaf(qs[g][i], kf[i], d);
      d += dpp<DPP_XOR1>(d);
      d += dpp<DPP_XOR2>(d);
      d += dpp<DPP_HALF_MIRROR>(d);
      d += dpp<DPP_MIRROR>(d);
      p[g][j] = act[j] ? d : -INFINITY;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mx = p[g][0];
#pragma unroll
    for (int j = 1; j < NR; ++j) mx = fmaxf(mx, p[g][j]);
    const float mn = fmaxf(st.m[g], mx);
    const float sc = (st.m[g] == mn) ? 1.0f : exp2_fast(st.m[g] - mn);
    float ps = 0.0f;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      p[g][j] = act[j] ? exp2_fast(p[g][j] - mn) : 0.0f;
      ps += p[g][j];
    }
    st.l[g] = __builtin_fmaf(st.l[g], sc, ps);
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[g][i] *= sc;
    st.m[g] = mn;
  }
}

// inactive rows must hold finite values (zeros): their probability is 0
template <typename T, int G, int NR>
HK_DEV void attn_values(AttnState<G> &st, const float (&p)[G][NR], const Raw8<T> (&vr)[NR]) {
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    float vf[8];
    raw_to_f(vr[j], vf);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) st.acc[g][i] = __builtin_fmaf(p[g][j], vf[i], st.acc[g][i]);
  }
}

template <typename T, int G, int NR>
HK_DEV void attn_rows(AttnState<G> &st, const float (&qs)[G][8], const Raw8<T> (&kr)[NR],
                      const Raw8<T> (&vr)[NR], const bool (&act)[NR]) {
  float p[G][NR];
  attn_keys<T, G, NR>(st, qs, kr, act, p);
  attn_values<T, G, NR>(st, p, vr);
}

// merge the four 16-lane groups of each wavefront, then the four wavefronts; write the
// partial [G][2 + HD] = (m, l, acc) to dst (only (m, l) = (-inf, 0) for a query that saw
// no row: the combine never reads that accumulator).  Must be reached by all threads.
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
    if (d == 0) {
      o[0] = M;
      o[1] = L;
    }
    if (L > 0.0f) o[2 + d] = A;  // a partial with l = 0 carries no accumulator
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

// Attention partial of segment `seg` of a head's tiers, written to its partial slot.
// Segments [0, nv_att) are view rows (rv_att each, up to k*), then nc_att segments of
// condensed slots (rc_att each, slots with n > 0 only), then nd_att segments of dense
// positions (rd_att each, positions [max(S, t - W), t)), then ns_att segments of sink
// positions (rs_att each, [0, min(S, t))), then (a step without selection) nt_att segments
// of the pool positions that arrived after the last selection, [pool end at t_plan, pool
// end at t), each taking every nt_att-th piece of rt_att of them.  A merged slot holding n tokens
// enters with key Kn/Omega, value Vn/Omega and logit bias ln n (log2 n in base 2).
template <typename T, int G>
HK_DEV void attend_segment(const Args &a, int bh, int seg, float (*s_part)[G][2 + HD]) {
  constexpr int EB = Elem<T>::bytes;
  constexpr size_t ROWB = (size_t)HD * EB;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane & 15, grp = lane >> 4;
  const int rloc = wave * 4 + grp;  // row of this lane group inside a batch of 16

  const int64_t t = a.seq_len[b];
  AttnState<G> st;
  st.init();
  float qs[G][8];
  load_q_scaled<T, G>(a, b, h, sub, qs);

  int slot;
  if (seg < a.nv_att) {  // view rows
    slot = seg;
    // a head that was not rewritten this step has no valid view (its kept rows are
    // attended from the pool by the rewrite kernel instead)
    const int64_t voff = a.head[bh].voff;
    const int64_t vcap = a.view_sum ? max((int64_t)0, a.view_rows - voff) : (int64_t)a.V_cap;
    const int64_t kst = a.head[bh].rw ? min((int64_t)a.budget[bh], vcap) : 0;
    const int64_t r0 = (int64_t)seg * a.rv_att, r1 = min(r0 + (int64_t)a.rv_att, kst);
    if (r0 < r1) {  // uniform
      // the head's view rows [0, r1) through buffer resources: a row past r1 gets an
      // offset outside the range (the load returns zeros, with no branch around it), and
      // the next batch's loads are in flight while the current one is attended
      const BufRes vk = make_buf((const char *)a.view_k + (size_t)voff * ROWB, (uint64_t)r1 * ROWB);
      const BufRes vv = make_buf((const char *)a.view_v + (size_t)voff * ROWB, (uint64_t)r1 * ROWB);
      const uint32_t lane_b = (uint32_t)(sub * 8 * EB);
      constexpr int VB = EB == 2 ? 4 : 2;  // rows per 16-lane group in a batch (fp32 rows: registers)
      auto issue = [&](Raw8<T> (&kr)[VB], Raw8<T> (&vr)[VB], int64_t base) {
#pragma unroll
        for (int j = 0; j < VB; ++j) {
          const int64_t r = base + j * 16 + rloc;
          const uint32_t off = r < r1 ? (uint32_t)((size_t)r * ROWB) + lane_b : BUF_SKIP;
          buf_load_nt(vk, off, kr[j]);
          buf_load_nt(vv, off, vr[j]);
        }
      };
      auto consume = [&](const Raw8<T> (&kr)[VB], const Raw8<T> (&vr)[VB], int64_t base) {
        bool act[VB];
#pragma unroll
        for (int j = 0; j < VB; ++j) act[j] = base + j * 16 + rloc < r1;
        attn_rows<T, G, VB>(st, qs, kr, vr, act);
      };
      // (the scheduling barriers keep each batch's loads ahead of the other batch's
      // arithmetic, where the compiler would otherwise sink them)
      Raw8<T> kA[VB], vA[VB], kB[VB], vB[VB];
      const int nb = (int)((r1 - r0 + 16 * VB - 1) / (16 * VB));
      int64_t base = r0;
      issue(kA, vA, base);
      for (int i = 0; i + 2 <= nb; i += 2) {
        issue(kB, vB, base + 16 * VB);
        __builtin_amdgcn_sched_barrier(0);
        consume(kA, vA, base);
        __builtin_amdgcn_sched_barrier(0);
        issue(kA, vA, base + 32 * VB);
        __builtin_amdgcn_sched_barrier(0);
        consume(kB, vB, base + 16 * VB);
        __builtin_amdgcn_sched_barrier(0);
        base += 32 * VB;
      }
      if (nb & 1) consume(kA, vA, base);
    }
  } else if (seg < a.nv_att + a.nc_att) {  // condensed slots
    const int xc = seg - a.nv_att;
    slot = a.part_cd_base + xc;
    const int s0 = xc * a.rc_att, s1 = min(s0 + a.rc_att, a.C);
    const size_t cb = (size_t)bh * a.C;
    for (int base = s0; base < s1; base += 16) {
      const int sg = base + rloc;
      const int n = sg < s1 ? a.cond_n[cb + sg] : 0;
      const bool act = n > 0;
      float kf[8], vf[8];
      float inv = 0.0f, bias = 0.0f;
      if (act) {
        load8(a.cond_kn + (cb + sg) * HD + sub * 8, kf, F32{});
        load8(a.cond_vn + (cb + sg) * HD + sub * 8, vf, F32{});
        inv = 1.0f / a.cond_omega[cb + sg];
        bias = a.merge_bias ? log2f((float)n) : 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) vf[i] *= inv;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) kf[i] = vf[i] = 0.0f;
      }
      attn_row<G>(st, qs, kf, vf, inv, bias, act);
    }
  } else if (seg < a.nv_att + a.nc_att + a.nd_att) {  // dense positions
    const int xd = seg - a.nv_att - a.nc_att;
    slot = a.part_cd_base + a.nc_att + xd;
    const int64_t lo = dense_lo_of(t, a.W, a.S);
    const int64_t p0 = lo + (int64_t)xd * a.rd_att, p1 = min(p0 + (int64_t)a.rd_att, t);
    const char *dk = (const char *)a.dense_k + (size_t)bh * a.W * ROWB + sub * 8 * EB;
    const char *dv = (const char *)a.dense_v + (size_t)bh * a.W * ROWB + sub * 8 * EB;
    for (int64_t base = p0; base < p1; base += 32) {
      Raw8<T> kr[2], vr[2];
      bool act[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t p = base + j * 16 + rloc;
        act[j] = p < p1;
        if (act[j]) {
          const size_t row = (size_t)(p % a.W);
          raw_load_nt(dk + row * ROWB, kr[j]);
          raw_load_nt(dv + row * ROWB, vr[j]);
        } else {
          kr[j] = Raw8<T>{};
          vr[j] = Raw8<T>{};
        }
      }
      attn_rows<T, G, 2>(st, qs, kr, vr, act);
    }
  } else if (seg < a.nv_att + a.nc_att + a.nd_att + a.ns_att) {  // sink positions [0, min(S, t)), row p
    const int xs = seg - a.nv_att - a.nc_att - a.nd_att;
    slot = a.part_cd_base + a.nc_att + a.nd_att + xs;
    const int64_t p0 = (int64_t)xs * a.rs_att, p1 = min(min(p0 + (int64_t)a.rs_att, (int64_t)a.S), t);
    const char *sk = (const char *)a.sink_k + (size_t)bh * a.S * ROWB + sub * 8 * EB;
    const char *sv = (const char *)a.sink_v + (size_t)bh * a.S * ROWB + sub * 8 * EB;
    for (int64_t base = p0; base < p1; base += 32) {
      Raw8<T> kr[2], vr[2];
      bool act[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t p = base + j * 16 + rloc;
        act[j] = p < p1;
        if (act[j]) {
          raw_load_nt(sk + (size_t)p * ROWB, kr[j]);
          raw_load_nt(sv + (size_t)p * ROWB, vr[j]);
        } else {
          kr[j] = Raw8<T>{};
          vr[j] = Raw8<T>{};
        }
      }
      attn_rows<T, G, 2>(st, qs, kr, vr, act);
    }
  } else {  // pool positions since the last selection
    const int xt = seg - a.nv_att - a.nc_att - a.nd_att - a.ns_att;
    slot = a.part_cd_base + a.nc_att + a.nd_att + a.ns_att + xt;
    const int64_t lo = pool_end(a.head[bh].t_plan, a.W, a.S), hi = pool_end(t, a.W, a.S);
    const char *pk = (const char *)a.pool_k + sub * 8 * EB;
    const char *pv = (const char *)a.pool_v + sub * 8 * EB;
    for (int64_t q0 = lo + (int64_t)xt * a.rt_att; q0 < hi; q0 += (int64_t)a.nt_att * a.rt_att) {
      const int64_t q1 = min(q0 + (int64_t)a.rt_att, hi);
      for (int64_t base = q0; base < q1; base += 32) {
        Raw8<T> kr[2], vr[2];
        bool act[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t p = base + j * 16 + rloc;
          act[j] = p < q1;
          if (act[j]) {
            const size_t row = pool_row0(a, bh, (int)((p / BK) % a.P)) + (size_t)(p % BK);
            raw_load_nt(pk + row * ROWB, kr[j]);
            raw_load_nt(pv + row * ROWB, vr[j]);
          } else {
            kr[j] = Raw8<T>{};
            vr[j] = Raw8<T>{};
          }
        }
        attn_rows<T, G, 2>(st, qs, kr, vr, act);
      }
    }
  }
  attn_write_partial<G>(st, a.part + ((size_t)bh * a.npart + slot) * G * (2 + HD), s_part);
}

}  // namespace hardkv
