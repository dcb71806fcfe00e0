// k_attend.hip -- decode attention over the three tiers, and the split-K combine.
//
// HARD-KV explainer, technical summary 2.A: the dense tier keeps the most recent tokens,
// the sparse tier the kept tokens (here already rewritten into the head's view), and the
// condensed tier constant-size merged slots.  Each query attends to all three.  A merged
// slot holding n tokens enters with key Kn/Omega, value Vn/Omega and logit bias ln n, so
// that n identical tokens merged into one slot weigh exactly as the n tokens did.
//
// Grid (segments, B*Hkv), 256 threads.  Segment x selects a range of one tier: view
// rows (standalone call only; in the fused step the rewrite kernel already attended
// them), condensed slots, or dense positions.  Each workgroup writes one partial; the
// combine kernel (one workgroup per head) merges them into the fp32 output.
#include "attn_common.h"

namespace hardkv {

namespace {


template <typename T, int G>
__global__ __launch_bounds__(NTHREADS) void hardkv_attend_tiers(Args a, int seg_offset) {
  constexpr int EB = Elem<T>::bytes;
  constexpr size_t ROWB = (size_t)HD * EB;
  const int bh = blockIdx.y, x = blockIdx.x + seg_offset;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane & 15, grp = lane >> 4;
  const int rloc = wave * 4 + grp;  // row of this lane group inside a batch of 16

  __shared__ float s_part[4][G][2 + HD];

  const int64_t t = a.seq_len[b];
  AttnState<G> st;
  st.init();
  float qs[G][8];
  load_q_scaled<T, G>(a, b, h, sub, qs);

  int slot;
  if (x < a.nv_att) {  // view rows [x*rv, min(x*rv + rv, k*))
    slot = x;
    const int64_t kst = min((int64_t)a.budget[bh], (int64_t)a.V_cap);
    const int64_t r0 = (int64_t)x * a.rv_att, r1 = min(r0 + (int64_t)a.rv_att, kst);
    const char *vk = (const char *)a.view_k + (size_t)bh * a.V_cap * ROWB + sub * 8 * EB;
    const char *vv = (const char *)a.view_v + (size_t)bh * a.V_cap * ROWB + sub * 8 * EB;
    for (int64_t base = r0; base < r1; base += 32) {
      Raw8<T> kr[2], vr[2];
      bool act[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t r = base + j * 16 + rloc;
        act[j] = r < r1;
        if (act[j]) {
          raw_load(vk + (size_t)r * ROWB, kr[j]);
          raw_load(vv + (size_t)r * ROWB, vr[j]);
        } else {
          kr[j] = Raw8<T>{};
          vr[j] = Raw8<T>{};
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float kf[8], vf[8];
        raw_to_f(kr[j], kf);
        raw_to_f(vr[j], vf);
        attn_row<G>(st, qs, kf, vf, 1.0f, 0.0f, act[j]);
      }
    }
  } else if (x < a.nv_att + a.nc_att) {  // condensed slots
    const int xc = x - a.nv_att;
    slot = a.part_cd_base + xc;
    const int s0 = xc * a.rc_att, s1 = min(s0 + a.rc_att, a.C);
    const size_t cb = (size_t)bh * a.C;
    for (int base = s0; base < s1; base += 16) {
      const int sg = base + rloc;
      const bool inr = sg < s1;
      const int n = inr ? a.cond_n[cb + sg] : 0;
      const bool act = n > 0;
      float kf[8], vf[8];
      float inv = 0.0f, bias = 0.0f;
      if (act) {
        load8(a.cond_kn + (cb + sg) * HD + sub * 8, kf, F32{});
        load8(a.cond_vn + (cb + sg) * HD + sub * 8, vf, F32{});
        inv = 1.0f / a.cond_omega[cb + sg];
        bias = a.merge_bias ? __log2f((float)n) : 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) vf[i] *= inv;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) kf[i] = vf[i] = 0.0f;
      }
      attn_row<G>(st, qs, kf, vf, inv, bias, act);
    }
  } else {  // dense positions [max(0, t - W), t)
    const int xd = x - a.nv_att - a.nc_att;
    slot = a.part_cd_base + a.nc_att + xd;
    const int64_t lo = t > a.W ? t - a.W : 0;
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
          raw_load(dk + row * ROWB, kr[j]);
          raw_load(dv + row * ROWB, vr[j]);
        } else {
          kr[j] = Raw8<T>{};
          vr[j] = Raw8<T>{};
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float kf[8], vf[8];
        raw_to_f(kr[j], kf);
        raw_to_f(vr[j], vf);
        attn_row<G>(st, qs, kf, vf, 1.0f, 0.0f, act[j]);
      }
    }
  }
  attn_write_partial<G>(st, a.part + ((size_t)bh * a.npart + slot) * G * (2 + HD), s_part);
}

template <int G>
__global__ __launch_bounds__(NTHREADS) void hardkv_combine(Args a) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  const float *base = a.part + (size_t)bh * a.npart * G * (2 + HD);
  const int ncd = a.nc_att + a.nd_att;
  for (int idx = threadIdx.x; idx < G * HD; idx += NTHREADS) {
    const int g = idx / HD, d = idx - g * HD;
    float M = -INFINITY;
    for (int i = 0; i < a.nvp + ncd; ++i) {
      const int s = i < a.nvp ? i : a.part_cd_base + (i - a.nvp);
      const float *ps = base + ((size_t)s * G + g) * (2 + HD);
      if (ps[1] > 0.0f) M = fmaxf(M, ps[0]);
    }
    float L = 0.0f, A = 0.0f;
    for (int i = 0; i < a.nvp + ncd; ++i) {
      const int s = i < a.nvp ? i : a.part_cd_base + (i - a.nvp);
      const float *ps = base + ((size_t)s * G + g) * (2 + HD);
      if (ps[1] > 0.0f) {
        const float f = exp2_fast(ps[0] - M);
        L += ps[1] * f;
        A += ps[2 + d] * f;
      }
    }
    a.out[((size_t)b * a.Hq + (size_t)h * G + g) * HD + d] = A / L;
  }
}

template <typename T>
hipError_t launch_tiers(const Args &a, hipStream_t s, bool with_view) {
  const int off = with_view ? 0 : a.nv_att;
  dim3 grid((with_view ? a.nv_att : 0) + a.nc_att + a.nd_att, a.B * a.Hkv);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((hardkv_attend_tiers<T, 1>), grid, dim3(NTHREADS), 0, s, a, off); break;
    case 2: hipLaunchKernelGGL((hardkv_attend_tiers<T, 2>), grid, dim3(NTHREADS), 0, s, a, off); break;
    case 4: hipLaunchKernelGGL((hardkv_attend_tiers<T, 4>), grid, dim3(NTHREADS), 0, s, a, off); break;
    case 8: hipLaunchKernelGGL((hardkv_attend_tiers<T, 8>), grid, dim3(NTHREADS), 0, s, a, off); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend(const Args &a, hipStream_t s, bool bf16, bool with_view) {
  return bf16 ? launch_tiers<BF16>(a, s, with_view) : launch_tiers<F32>(a, s, with_view);
}

hipError_t launch_combine(const Args &a, hipStream_t s) {
  dim3 grid(a.B * a.Hkv);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((hardkv_combine<1>), grid, dim3(NTHREADS), 0, s, a); break;
    case 2: hipLaunchKernelGGL((hardkv_combine<2>), grid, dim3(NTHREADS), 0, s, a); break;
    case 4: hipLaunchKernelGGL((hardkv_combine<4>), grid, dim3(NTHREADS), 0, s, a); break;
    case 8: hipLaunchKernelGGL((hardkv_combine<8>), grid, dim3(NTHREADS), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hardkv
