// condense_common.h -- the condensation of one ring slot, shared by the condense kernel and
// by the select kernels that condense in the same launch when few blocks can condense.
//
// HARD-KV explainer, technical summary 2.A (tier 3): the oldest blocks are evicted or
// merged by weight into storage of constant size.  Condensed block e (of the E oldest,
// from pool head c) goes to ring slot (nu + e) mod C; MERGE adds its tokens with weights
// w_j / W_all to the slot's numerators.
#pragma once
#include "hardkv_internal.h"

namespace hardkv {

// One wavefront folds into ring slot (nu + i) mod C, in age order, every condensing block
// that lands there (blocks i, i + C, ...).  Inside a block, 16 lanes hold one row (8 head
// dims each) and a load covers 4 rows; NB loads of keys and NB of values per lane are in
// flight per batch.  Each lane accumulates w k and w v for its dims over its rows, the
// four row groups are summed by lane exchanges, and 16 lanes update the slot.  LEAN: the
// batches one after another (no later batch's loads hoisted into an earlier one), for a
// caller with fewer registers to spare.
template <typename T, int NB, bool LEAN = false>
HK_DEV void condense_chain(const Args &a, int bh, int i, int64_t c, int64_t E, int32_t nu, uint64_t w_all) {
  constexpr int EB = Elem<T>::bytes;
  constexpr size_t ROWB = (size_t)HD * EB;
  static_assert(16 % NB == 0, "batches of NB row groups cover the 16 of a block");
  const int lane = threadIdx.x & 63;
  const int sub = lane & 15, grp = lane >> 4;
  const int P = a.P, C = a.C;
  const size_t sg = (size_t)bh * C + (size_t)((nu + i) % C);
  // an empty slot (n = 0, as every slot is after a prefill) holds zeros: it is written
  // without being read back
  const bool fresh = a.cond_n[sg] == 0;
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
    constexpr int UNB = LEAN ? 1 : 16 / NB;
#pragma unroll UNB
    for (int bt = 0; bt < 16 / NB; ++bt) {
      Raw8<T> kr[NB], vr[NB];
#pragma unroll
      for (int it = 0; it < NB; ++it) {
        const int row = (bt * NB + it) * 4 + grp;
        raw_load_nt(kb + (size_t)row * ROWB, kr[it]);
        raw_load_nt(vb + (size_t)row * ROWB, vr[it]);
      }
#pragma unroll
      for (int it = 0; it < NB; ++it) {
        const int row = (bt * NB + it) * 4 + grp;
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
  const double wa = (double)w_all;
  const float inv = (float)(1.0 / wa);
  if (lane < 16) {
    float4 *kn = reinterpret_cast<float4 *>(a.cond_kn + sg * HD + sub * 8);
    float4 *vn = reinterpret_cast<float4 *>(a.cond_vn + sg * HD + sub * 8);
    const float4 z = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float4 k0 = z, k1 = z, v0 = z, v1 = z;
    if (!fresh) {
      k0 = kn[0];
      k1 = kn[1];
      v0 = vn[0];
      v1 = vn[1];
    }
    k0.x += ak[0] * inv; k0.y += ak[1] * inv; k0.z += ak[2] * inv; k0.w += ak[3] * inv;
    k1.x += ak[4] * inv; k1.y += ak[5] * inv; k1.z += ak[6] * inv; k1.w += ak[7] * inv;
    v0.x += av[0] * inv; v0.y += av[1] * inv; v0.z += av[2] * inv; v0.w += av[3] * inv;
    v1.x += av[4] * inv; v1.y += av[5] * inv; v1.z += av[6] * inv; v1.w += av[7] * inv;
    kn[0] = k0; kn[1] = k1; vn[0] = v0; vn[1] = v1;
  }
  if (lane == 0) {
    a.cond_omega[sg] = (fresh ? 0.0f : a.cond_omega[sg]) + (float)((double)wsum / wa);
    a.cond_n[sg] += BK * nblk;
  }
}

// After the slots: the cursor (MERGE) and the pool head move past the E condensed blocks.
HK_DEV void condense_advance(const Args &a, int bh, int64_t c, int64_t E, int32_t nu) {
  if (a.mode == HARDKV_COND_MERGE) a.cond_cursor[bh] = (int32_t)((nu + E) % a.C);
  a.pool_head[bh] = c + (int64_t)BK * E;
}

}  // namespace hardkv
