// k_condense.hip -- stage 4 of the decode step: eviction or weighted merging of the
// oldest pool blocks into the constant-size condensed tier.
//
// HARD-KV explainer, technical summary 2.A (tier 3): to keep memory within hard limits
// the oldest blocks are compressed further, by eviction or weighted merging, into
// storage of constant size.  Here each condensed block goes to the next slot of a ring
// of C slots; MERGE adds its tokens with weights w_j / W_all (the calibrated probability
// of the select stage) to the slot's numerators, EVICT drops it.  The pool head
// advances by the condensed blocks either way.
//
// Grid (slots touched, B*Hkv), 256 threads.  Workgroup i owns ring slot (cursor + i)
// mod C and folds in, in age order, every condensed block that lands there (blocks i,
// i + C, ...), so the result does not depend on scheduling.  Every workgroup reads the
// pool head, the cursor and E from the plan the select kernel saved, so workgroup 0 can
// advance the state's pool head and cursor without waiting for the others.
#include "hardkv_internal.h"

namespace hardkv {

namespace {

template <typename T>
__global__ __launch_bounds__(NTHREADS) void hardkv_condense(Args a) {
  constexpr int EB = Elem<T>::bytes;
  constexpr size_t ROWB = (size_t)HD * EB;
  const int bh = blockIdx.y, i = blockIdx.x;
  const int tid = threadIdx.x, rg = tid >> 4, sub = tid & 15;
  const int P = a.P, C = a.C;

  __shared__ float s_k[16][HD];
  __shared__ float s_v[16][HD];
  __shared__ unsigned long long s_w[16];

  const HeadInfo *hd = a.head + bh;
  const int64_t c = hd->c_plan;
  const int64_t E = hd->E;
  const int32_t nu = hd->nu_plan;

  if (a.mode == HARDKV_COND_MERGE && i < E) {
    float ak[8], av[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) ak[k] = av[k] = 0.0f;
    unsigned long long wsum = 0;
    int nblk = 0;
    for (int64_t e = i; e < E; e += C) {
      ++nblk;
      const size_t pb = (size_t)((c / BK + e) % P);
      const char *kb = (const char *)a.pool_k + ((size_t)bh * P + pb) * BK * ROWB + sub * 8 * EB;
      const char *vb = (const char *)a.pool_v + ((size_t)bh * P + pb) * BK * ROWB + sub * 8 * EB;
      const uint32_t *wb = a.weights + ((size_t)bh * P + pb) * BK;
#pragma unroll
      for (int rr = 0; rr < BK; rr += 16) {
        const int row = rr + rg;
        const uint32_t w = wb[row];
        const float wf = (float)w;
        float kf[8], vf[8];
        load8(kb + (size_t)row * ROWB, kf, T{});
        load8(vb + (size_t)row * ROWB, vf, T{});
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          ak[k] = __builtin_fmaf(wf, kf[k], ak[k]);
          av[k] = __builtin_fmaf(wf, vf[k], av[k]);
        }
        if (sub == 0) wsum += w;
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      s_k[rg][sub * 8 + k] = ak[k];
      s_v[rg][sub * 8 + k] = av[k];
    }
    if (sub == 0) s_w[rg] = wsum;
    __syncthreads();
    const double w_all = (double)hd->w_all;
    const float inv = (float)(1.0 / w_all);
    const size_t sg = (size_t)bh * C + (size_t)((nu + i) % C);
    if (tid < HD) {
      float sk = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) sk += s_k[r][tid];
      a.cond_kn[sg * HD + tid] += sk * inv;
    } else {
      const int d = tid - HD;
      float sv = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) sv += s_v[r][d];
      a.cond_vn[sg * HD + d] += sv * inv;
    }
    if (tid == 0) {
      unsigned long long ws = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) ws += s_w[r];
      a.cond_omega[sg] += (float)((double)ws / w_all);
      a.cond_n[sg] += BK * nblk;
    }
  }

  if (i == 0 && tid == 0) {
    if (a.mode == HARDKV_COND_MERGE) a.cond_cursor[bh] = (int32_t)((nu + E) % C);
    a.pool_head[bh] = c + (int64_t)BK * E;
  }
}

}  // namespace

hipError_t launch_condense(const Args &a, hipStream_t s, bool bf16) {
  dim3 grid(a.ncs, a.B * a.Hkv);
  if (bf16)
    hipLaunchKernelGGL((hardkv_condense<BF16>), grid, dim3(NTHREADS), 0, s, a);
  else
    hipLaunchKernelGGL((hardkv_condense<F32>), grid, dim3(NTHREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace hardkv
