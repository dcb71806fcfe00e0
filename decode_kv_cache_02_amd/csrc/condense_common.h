// condense_common.h -- the condensation of one ring slot (the condense kernel) and the
// advance of the pool head past the condensed blocks (also taken by the select kernels that
// condense in the same launch when few blocks can condense).
//
// HARD-KV explainer, technical summary 2.A (tier 3): the oldest blocks are evicted or
// merged by weight into storage of constant size.  Condensed block e (of the E oldest,
// from pool head c) goes to ring slot (nu + e) mod C; MERGE adds its tokens with weights
// w_j / W_all to the slot's numerators.
#pragma once
#include "hardkv_internal.h"

namespace hardkv {

// The buffer resources over a ring block's rows (K and V) and the block's first row inside
// them: the unit's own ring, or in the shared pool the 1 GB segment that holds the block's
// physical block (one resource reaches 2 GB; the pool can be larger).  Wave-uniform.
template <typename T>
struct BlockRows {
  BufRes k, v;
  uint32_t row0;
};
template <typename T>
HK_DEV BlockRows<T> block_rows(const Args &a, int bh, int pb) {
  constexpr uint32_t ROWB = (uint32_t)(HD * Elem<T>::bytes);
  constexpr uint64_t BLKB = (uint64_t)BK * ROWB;
  BlockRows<T> r;
  if (a.pool_shared) {
    constexpr uint32_t SEGB = (uint32_t)((1ull << 30) / BLKB);  // blocks per segment
    const int32_t ph = a.btab[(size_t)bh * a.P + pb];
    const uint32_t phys = ph < 0 ? 0u : (uint32_t)ph;
    const uint32_t seg = phys / SEGB;
    const size_t base = (size_t)seg * SEGB * BLKB;
    const uint64_t bytes = (uint64_t)min((uint32_t)a.NB - seg * SEGB, SEGB) * BLKB;
    r.k = make_buf((const char *)a.pool_k + base, bytes);
    r.v = make_buf((const char *)a.pool_v + base, bytes);
    r.row0 = (phys % SEGB) * BK;
  } else {
    const size_t base = (size_t)bh * a.P * BLKB;
    r.k = make_buf((const char *)a.pool_k + base, (uint64_t)a.P * BLKB);
    r.v = make_buf((const char *)a.pool_v + base, (uint64_t)a.P * BLKB);
    r.row0 = (uint32_t)pb * BK;
  }
  return r;
}

// One wavefront folds into ring slot (nu + i) mod C, in age order, every condensing block
// that lands there (blocks i, i + C, ...).  Inside a block, 16 lanes hold one row (8 head
// dims each) and a load covers 4 rows, through the block's buffer resources; NB loads of
// keys and NB of values per lane are in flight per batch.  Each lane accumulates w k and w v for its dims over its rows, the
// four row groups are summed by lane exchanges, and 16 lanes update the slot.
template <typename T, int NB>
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
  int nlive = 0;  // rows merged: those with a weight (all 64 of a block unless dropped)
  for (int64_t e = i; e < E; e += C) {
    const size_t pb = (size_t)((c / BK + e) % P);
    const BlockRows<T> br = block_rows<T>(a, bh, (int)pb);
    const uint32_t lane_off = br.row0 * (uint32_t)ROWB + (uint32_t)(sub * 8 * EB);
    const uint32_t wl = a.weights[((size_t)bh * P + pb) * BK + lane];  // weight of row `lane`
    wsum += wl;
    nlive += __popcll(ballot(wl != 0u));
#pragma unroll
    for (int bt = 0; bt < 16 / NB; ++bt) {
      Raw8<T> kr[NB], vr[NB];
#pragma unroll
      for (int it = 0; it < NB; ++it) {
        const int row = (bt * NB + it) * 4 + grp;
        buf_load_nt(br.k, lane_off + (uint32_t)(row * ROWB), kr[it]);
        buf_load_nt(br.v, lane_off + (uint32_t)(row * ROWB), vr[it]);
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
  const float inv = w_all ? (float)(1.0 / wa) : 0.0f;  // (no mass: every row dropped, nothing merged)
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
    a.cond_omega[sg] = (fresh ? 0.0f : a.cond_omega[sg]) + (w_all ? (float)((double)wsum / wa) : 0.0f);
    a.cond_n[sg] += nlive;
  }
}

// After the slots: the cursor (MERGE) and the pool head move past the E condensed blocks.
// In the shared pool the condensed blocks go back to the free list (their table entries
// stay: nothing reads a ring block outside the pool, and the append that reuses the ring
// block sets it again).  Called by all 64 lanes of one wavefront: lane 0 moves the counters,
// the lanes return the blocks 64 at a time.
HK_DEV void condense_advance(const Args &a, int bh, int64_t c, int64_t E, int32_t nu) {
  const int lane = threadIdx.x & 63;
  if (lane == 0) {
    if (a.mode == HARDKV_COND_MERGE) a.cond_cursor[bh] = (int32_t)((nu + E) % a.C);
    a.pool_head[bh] = c + (int64_t)BK * E;
  }
  if (a.pool_shared && E > 0) {
    // (a block the pool never got, after an overflow, has no entry to return)
    const int32_t *tb = a.btab + (size_t)bh * a.P;
    const int64_t blk0 = c / BK;
    int32_t n = 0;
    for (int64_t e0 = 0; e0 < E; e0 += 64) {
      const int64_t e = e0 + lane;
      const int32_t ph = e < E ? tb[(blk0 + e) % a.P] : -1;
      n += __popcll(ballot(ph >= 0));
    }
    int32_t at = 0;
    if (lane == 0) at = atomicAdd(a.free_top, n);
    at = __shfl(at, 0);
    int32_t k = 0;
    for (int64_t e0 = 0; e0 < E; e0 += 64) {
      const int64_t e = e0 + lane;
      const int32_t ph = e < E ? tb[(blk0 + e) % a.P] : -1;
      const uint64_t m = ballot(ph >= 0);
      const int32_t slot = at + k + (int32_t)popc_below(m);
      if (ph >= 0 && slot < a.NB) a.free_list[slot] = ph;
      k += __popcll(m);
    }
  }
}

}  // namespace hardkv
