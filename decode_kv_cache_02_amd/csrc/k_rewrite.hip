// k_rewrite.hip -- stage 3 of the decode step: Index Regularization by Rewrite Cache.
//
// HARD-KV explainer, technical summary 2.C: the tokens the top-p mask keeps are moved
// into contiguous ranges, each head owning a fixed-capacity view (the max-length form
// of Flatten Index), so that attention reads static, contiguous, fixed-stride blocks.
//
// Grid (chunks, B*Hkv), 256 threads.  A wavefront takes one 64-row pool block at a
// time: the mask word (one bit per row) gives the kept rows; their rank inside the word
// (mbcnt) plus the block's view offset (from the select stage's scan) gives each row's
// view row, so the order of positions is preserved.  The kept rows are copied as 16-byte
// pieces, 16 lanes per row, 16 rows in flight per wavefront.  In the fused step the
// same kernel also runs the attention of the group's queries over the rows it copies
// and writes one split-K partial per workgroup, so the view is never read back.
#include "attn_common.h"

namespace hardkv {

namespace {

template <typename T, int G, bool ATTN>
__global__ __launch_bounds__(NTHREADS) void hardkv_rewrite(Args a) {
  constexpr int EB = Elem<T>::bytes;
  constexpr size_t ROWB = (size_t)HD * EB;
  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane & 15, grp = lane >> 4;
  const int P = a.P, V = a.V_cap;

  __shared__ uint8_t s_list[4][64];
  __shared__ float s_part[ATTN ? 4 : 1][G][2 + HD];

  const int64_t t = a.seq_len[b];
  const int64_t c = a.pool_head[bh];
  const int64_t pend = pool_end(t, a.W);
  const int64_t E = plan_E(pend - c, a.mode, a.S_cap);
  const int64_t ub_lo = (c + (int64_t)BK * E) / BK, blk_hi = (pend + BK - 1) / BK;
  const int64_t L0 = ub_lo + (int64_t)chunk * a.cb_reg;
  const int64_t L1 = min(L0 + (int64_t)a.cb_reg, blk_hi);

  AttnState<G> st;
  float qs[G][8];
  if (ATTN) {
    st.init();
    load_q_scaled<T, G>(a, b, h, sub, qs);
  }
  const char *pk = (const char *)a.pool_k + (size_t)bh * P * BK * ROWB + sub * 8 * EB;
  const char *pv = (const char *)a.pool_v + (size_t)bh * P * BK * ROWB + sub * 8 * EB;
  char *vk = (char *)a.view_k + (size_t)bh * V * ROWB + sub * 8 * EB;
  char *vv = (char *)a.view_v + (size_t)bh * V * ROWB + sub * 8 * EB;
  int32_t *vpos = a.view_pos + (size_t)bh * V;

  const int nl = (int)(L1 - L0);
  const int pb0 = L0 < L1 ? (int)(L0 % P) : 0;
  for (int i = wave; i < nl; i += 4) {
    const int64_t L = L0 + i;
    const size_t pb = (size_t)(pb0 + i >= P ? pb0 + i - P : pb0 + i);
    const uint64_t mw = a.mask[(size_t)bh * P + pb];
    if (mw == 0) continue;  // wave-uniform
    const uint32_t vo = a.viewoff[(size_t)bh * P + pb];
    const bool sel = (mw >> lane) & 1ull;
    const uint32_t idx = popc_below(mw);
    if (sel) {
      s_list[wave][idx] = (uint8_t)lane;
      if (vo + idx < (uint32_t)V) vpos[vo + idx] = (int32_t)(L * BK + lane);
    }
    wave_sync();
    const int ns = __popcll(mw);
    const char *pkb = pk + pb * BK * ROWB, *pvb = pv + pb * BK * ROWB;
    for (int it = 0; it < ns; it += 16) {
      Raw8<T> kr[4], vr[4];
      bool act[4];
      uint32_t dst[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = it + j * 4 + grp;
        dst[j] = vo + (uint32_t)k;
        act[j] = k < ns && dst[j] < (uint32_t)V;
        const int row = s_list[wave][k < ns ? k : 0];
        if (act[j]) {
          raw_load(pkb + (size_t)row * ROWB, kr[j]);
          raw_load(pvb + (size_t)row * ROWB, vr[j]);
        } else {
          kr[j] = Raw8<T>{};
          vr[j] = Raw8<T>{};
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (act[j]) {
          raw_store(vk + (size_t)dst[j] * ROWB, kr[j]);
          raw_store(vv + (size_t)dst[j] * ROWB, vr[j]);
        }
      }
      if (ATTN) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float kf[8], vf[8];
          raw_to_f(kr[j], kf);
          raw_to_f(vr[j], vf);
          attn_row<G>(st, qs, kf, vf, 1.0f, 0.0f, act[j]);
        }
      }
    }
    wave_sync();
  }
  if (ATTN) attn_write_partial<G>(st, a.part + ((size_t)bh * a.npart + chunk) * G * (2 + HD), s_part);
}

template <typename T, bool ATTN>
hipError_t launch_g(const Args &a, hipStream_t s) {
  dim3 grid(a.nch_reg, a.B * a.Hkv);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((hardkv_rewrite<T, 1, ATTN>), grid, dim3(NTHREADS), 0, s, a); break;
    case 2: hipLaunchKernelGGL((hardkv_rewrite<T, 2, ATTN>), grid, dim3(NTHREADS), 0, s, a); break;
    case 4: hipLaunchKernelGGL((hardkv_rewrite<T, 4, ATTN>), grid, dim3(NTHREADS), 0, s, a); break;
    case 8: hipLaunchKernelGGL((hardkv_rewrite<T, 8, ATTN>), grid, dim3(NTHREADS), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_regularize(const Args &a, hipStream_t s, bool bf16, bool attend) {
  if (bf16) return attend ? launch_g<BF16, true>(a, s) : launch_g<BF16, false>(a, s);
  return attend ? launch_g<F32, true>(a, s) : launch_g<F32, false>(a, s);
}

}  // namespace hardkv
