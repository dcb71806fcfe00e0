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
// Grid (ceil(slots touched / 4), B*Hkv), 256 threads.  Each wavefront owns one ring slot
// (cursor + i) mod C and folds in, in age order, every condensed block that lands there
// (blocks i, i + C, ...), so the result does not depend on scheduling.  Inside a block,
// 16 lanes hold one row (8 head dims each) and a load covers 4 rows; each lane
// accumulates w * k and w * v for its dims over its rows, the four row groups are then
// summed by lane exchanges, and 16 lanes update the slot.  Every wavefront reads the pool
// head, the cursor and E from the plan the select kernel saved, so one of them can
// advance the state's pool head and cursor without waiting for the others.
#include "hardkv_internal.h"

namespace hardkv {

namespace {

template <typename T>
__global__ __launch_bounds__(NTHREADS) void hardkv_condense(Args a) {
  constexpr int EB = Elem<T>::bytes;
  constexpr size_t ROWB = (size_t)HD * EB;
  const int bh = a.bh0 + blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane & 15, grp = lane >> 4;
  const int i = blockIdx.x * 4 + wave;  // slot offset from the cursor
  const int P = a.P, C = a.C;

  const HeadInfo *hd = a.head + bh;
  const int64_t c = hd->c_plan;
  const int64_t E = hd->E;
  const int32_t nu = hd->nu_plan;

  if (a.mode == HARDKV_COND_MERGE && i < E && i < C) {  // chain heads: blocks 0 .. min(E, C) - 1
    float ak[8], av[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) ak[k] = av[k] = 0.0f;
    uint64_t wsum = 0;
    int nblk = 0;
    for (int64_t e = i; e < E; e += C) {
      ++nblk;
      const size_t pb = (size_t)((c / BK + e) % P);
      const char *kb = (const char *)a.pool_k + ((size_t)bh * P + pb) * BK * ROWB + sub * 8 * EB;
      const char *vb = (const char *)a.pool_v + ((size_t)bh * P + pb) * BK * ROWB + sub * 8 * EB;
      const uint32_t wl = a.weights[((size_t)bh * P + pb) * BK + lane];  // weight of row `lane`
      wsum += wl;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        Raw8<T> kr[8], vr[8];
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int row = (half * 8 + it) * 4 + grp;
          raw_load_nt(kb + (size_t)row * ROWB, kr[it]);
          raw_load_nt(vb + (size_t)row * ROWB, vr[it]);
        }
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int row = (half * 8 + it) * 4 + grp;
          const float wf = (float)(uint32_t)__shfl((int)wl, row);
          float kf[8], vf[8];
          raw_to_f(kr[it], kf);
          raw_to_f(vr[it], vf);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            ak[k] = __builtin_fmaf(wf, kf[k], ak[k]);
            av[k] = __builtin_fmaf(wf, vf[k], av[k]);
          }
        }
      }
    }
    // sum the four row groups (lanes sub, sub + 16, sub + 32, sub + 48)
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        ak[k] += __shfl_xor(ak[k], off);
        av[k] += __shfl_xor(av[k], off);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)wsum, off), hi = __shfl_xor((uint32_t)(wsum >> 32), off);
      wsum += ((uint64_t)hi << 32) | lo;
    }
    const double w_all = (double)hd->w_all;
    const float inv = (float)(1.0 / w_all);
    const size_t sg = (size_t)bh * C + (size_t)((nu + i) % C);
    if (lane < 16) {
      float4 *kn = reinterpret_cast<float4 *>(a.cond_kn + sg * HD + sub * 8);
      float4 *vn = reinterpret_cast<float4 *>(a.cond_vn + sg * HD + sub * 8);
      float4 k0 = kn[0], k1 = kn[1], v0 = vn[0], v1 = vn[1];
      k0.x += ak[0] * inv; k0.y += ak[1] * inv; k0.z += ak[2] * inv; k0.w += ak[3] * inv;
      k1.x += ak[4] * inv; k1.y += ak[5] * inv; k1.z += ak[6] * inv; k1.w += ak[7] * inv;
      v0.x += av[0] * inv; v0.y += av[1] * inv; v0.z += av[2] * inv; v0.w += av[3] * inv;
      v1.x += av[4] * inv; v1.y += av[5] * inv; v1.z += av[6] * inv; v1.w += av[7] * inv;
      kn[0] = k0; kn[1] = k1; vn[0] = v0; vn[1] = v1;
    }
    if (lane == 0) {
      a.cond_omega[sg] += (float)((double)wsum / w_all);
      a.cond_n[sg] += BK * nblk;
    }
  }

  if (i == 0 && lane == 0) {
    if (a.mode == HARDKV_COND_MERGE) a.cond_cursor[bh] = (int32_t)((nu + E) % C);
    a.pool_head[bh] = c + (int64_t)BK * E;
  }
}

}  // namespace

hipError_t launch_condense(const Args &a, hipStream_t s, bool bf16) {
  dim3 grid((a.ncs + 3) / 4, a.nbh);
  if (bf16)
    hipLaunchKernelGGL((hardkv_condense<BF16>), grid, dim3(NTHREADS), 0, s, a);
  else
    hipLaunchKernelGGL((hardkv_condense<F32>), grid, dim3(NTHREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace hardkv
