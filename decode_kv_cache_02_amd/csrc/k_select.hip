// k_select.hip -- stage 2 of the decode step: max-pooled scores, logits calibration and
// calibrated top-p for every (sequence, KV head).
//
// HARD-KV explainer, technical summary 2.A (tier 2: calibrated top-p gives each head
// its own budget) and 2.B (max-pooled logits as the importance metric; calibration maps
// the scores to one softmax by a temperature, keeping their order).
//
// Kernel boundaries are the only synchronization between workgroups (no cross-workgroup
// flags: on MI355X each agent-scope release/acquire writes back or invalidates a whole
// XCD's L2).
//
// hardkv_score, grid (chunks, B*Hkv), 256 threads (units interleaved over the XCDs): streams a chunk of the head's pool
//   keys with 16-byte loads; 16 lanes hold one 256-byte bf16 row (8 elements each), a
//   wavefront covers 4 rows per load.  Each lane forms the pairwise sum of its 8
//   products in registers (tree levels 1-3); levels 4-7 are DPP exchanges inside the
//   16-lane row, so every lane ends with the exact root.  The score is the max over the
//   group queries.  Writes the scores and the chunk's maximum.  With 16-bit elements
//   every product is exact unless an element is tiny or huge; while the head's pool
//   holds no such key and the queries none either, a level-1 node is one fused
//   multiply-add (the same value, a fifth fewer vector instructions per row).  Under
//   destructive selection the chunk first lists its rows in play in LDS (the last
//   selection's kept rows and the arrivals since) and streams only those: the pass costs
//   what the selection keeps, not what the pool holds.
//
// hardkv_select, grid (B*Hkv), 1024 threads: one workgroup per head.  Pass A turns the
//   scores into integer weights and builds a mass histogram of the survivors on the top
//   bits of the weight's float encoding; the bucket that holds the cut is found by a
//   suffix scan.  Pass B counts, per 64-row block, the weights above that bucket and
//   gathers the bucket's tokens into LDS, where two more histogram levels give the
//   exact threshold weight w_th and the number r of ties at w_th that are kept (ties go
//   to the lowest positions).  A scan over blocks gives each block its first view row
//   and its ties-before count; the rewrite kernel derives the mask bits from them.  The
//   select kernel clears all the head's mask words; the rewrite writes the survivors'.
//
// For rings of SEL_SPLIT_MIN or more slices of SEL_SLICE_BLOCKS blocks, one workgroup per
//   head would spend most of the stage streaming its pool through one CU, so the two
//   passes run over the slices in parallel: hardkv_sel_weigh (pass A per slice, its
//   histogram and masses to memory), hardkv_sel_cut (per head: the cut bucket),
//   hardkv_sel_count (pass B per slice: per-block counts, the bucket's tokens through a
//   counter) and hardkv_sel_finish (per head: the same ending as the one-workgroup kernel).
#include <mutex>
#include <type_traits>

#include "condense_common.h"

namespace hardkv {

namespace {

constexpr int UNR = 2;  // row groups (16 rows) per batch of loads

// score of one row from this lane's 8 elements: pairwise tree over the 128 products.
// bf16 pairs widened by byte permutes: (b1 b0 0 0) and (b3 b2 0 0)
HK_DEV void raw_to_f_perm(const Raw8<BF16> &r, float (&f)[8]) {
  const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(__builtin_amdgcn_perm(0u, w[i], 0x01000c0cu));
    f[2 * i + 1] = __uint_as_float(__builtin_amdgcn_perm(0u, w[i], 0x03020c0cu));
  }
}
HK_DEV void raw_to_f_perm(const Raw8<F32> &r, float (&f)[8]) { raw_to_f(r, f); }

// FUSED (only when every product is exact: 16-bit operands inside the safe magnitudes):
// a level-1 node fl(fl(q0 k0) + fl(q1 k1)) is then one fused multiply-add on fl(q1 k1).
template <bool FUSED>
HK_DEV float dot_lane(const float (&q)[8], const float (&k)[8]) {
  float a0, a1, a2, a3;
  if (FUSED) {
    a0 = __builtin_fmaf(q[0], k[0], q[1] * k[1]);
    a1 = __builtin_fmaf(q[2], k[2], q[3] * k[3]);
    a2 = __builtin_fmaf(q[4], k[4], q[5] * k[5]);
    a3 = __builtin_fmaf(q[6], k[6], q[7] * k[7]);
  } else {
    float p0 = q[0] * k[0], p1 = q[1] * k[1], p2 = q[2] * k[2], p3 = q[3] * k[3];
    float p4 = q[4] * k[4], p5 = q[5] * k[5], p6 = q[6] * k[6], p7 = q[7] * k[7];
    a0 = p0 + p1;
    a1 = p2 + p3;
    a2 = p4 + p5;
    a3 = p6 + p7;
  }
  float b0 = a0 + a1, b1 = a2 + a3;
  return b0 + b1;                    // level 3: node `sub` of 16
}

// The G trees of one row: levels 1-3 in each lane, then levels 4-7 across the 16 lanes of
// the row, one level for every query before the next (the DPP reads then never wait for
// the instruction just before them).
template <bool FUSED, int G>
HK_DEV void dot_trees(const float (&q)[G][8], const float (&k)[8], float (&c)[G]) {
#pragma unroll
  for (int g = 0; g < G; ++g) c[g] = dot_lane<FUSED>(q[g], k);
#pragma unroll
  for (int g = 0; g < G; ++g) c[g] = c[g] + dpp<DPP_XOR1>(c[g]);         // level 4: nodes (2i, 2i+1)
#pragma unroll
  for (int g = 0; g < G; ++g) c[g] = c[g] + dpp<DPP_XOR2>(c[g]);         // level 5: lanes 4i..4i+3
#pragma unroll
  for (int g = 0; g < G; ++g) c[g] = c[g] + dpp<DPP_HALF_MIRROR>(c[g]);  // level 6: lanes 8i..8i+7
#pragma unroll
  for (int g = 0; g < G; ++g) c[g] = c[g] + dpp<DPP_MIRROR>(c[g]);       // level 7: all 16 lanes
}

HK_DEV float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// (m, z, a) of a base-2 softmax piece: m its max logit, z = sum 2^(l - m), a = sum
// 2^(l - m) (l - m); two pieces of the same query merge exactly as below
HK_DEV void ent_merge(float &m, float &z, float &w, float m2, float z2, float w2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  const float d1 = m == -INFINITY ? 0.0f : m - M, d2 = m2 == -INFINITY ? 0.0f : m2 - M;
  const float s1 = m == -INFINITY ? 0.0f : exp2_fast(d1), s2 = m2 == -INFINITY ? 0.0f : exp2_fast(d2);
  w = s1 * (w + d1 * z) + s2 * (w2 + d2 * z2);
  z = s1 * z + s2 * z2;
  m = M;
}

// A piece (m, z, a) after one more logit x, with one exponential: of the old max and x,
// the lower one is scaled by 2^(lower - higher).  The same values as merging the
// single-logit piece (x, 1, 0) above, rounded in a different order; x = -inf adds
// nothing, as there.
HK_DEV void ent_add(float &m, float &z, float &w, float x) {
  const bool keep = x == -INFINITY;   // (every select below, not a branch)
  const bool first = m == -INFINITY;  // empty piece so far
  const bool up = x > m;              // x becomes the max
  const float d = first ? 0.0f : (up ? m - x : x - m);
  const float e = first ? 0.0f : exp2_fast(d);
  // up: old sums scaled by e, new term (1, 0); else: old sums kept, new term (e, e d)
  const float zn = (up ? e * z : z) + (up ? 1.0f : e);
  const float wn = up ? e * __builtin_fmaf(d, z, w) : __builtin_fmaf(e, d, w);
  z = keep ? z : zn;
  w = keep ? w : wn;
  m = up ? x : m;
}

// SHARED: the pool is the shared block pool (rows of a chunk's blocks anywhere in it, loaded
// through flat addresses from the block table), else the unit's own ring (one buffer resource).
// The score workgroup's (unit, chunk).  Workgroup i goes to XCD i mod 8; when the units
// come in groups of 8 (the KV heads of a sequence share its length), XCD x takes units
// x, x + 8, ..., each unit's chunks in order, so that every XCD gets the same share of
// long and short sequences.  Otherwise, contiguous ranges of the work (xcd_swizzle).
HK_DEV void score_work(int lin, int nch, int nbh, int &bh_rel, int &chunk) {
  if ((nbh & 7) == 0) {
    const int x = lin & 7, k = lin >> 3;
    const int j = k / nch;
    chunk = k - j * nch;
    bh_rel = x + 8 * j;
  } else {
    const int w = xcd_swizzle(lin, nch * nbh);
    bh_rel = w / nch;
    chunk = w - bh_rel * nch;
  }
}

template <typename T, int G, bool ENT, bool SHARED, bool LIVE>
__global__ __launch_bounds__(NTHREADS) void hardkv_score(Args a) {
  static_assert(!(ENT && LIVE), "destructive selection runs with the fixed temperature");
  constexpr int EB = Elem<T>::bytes;
  constexpr int CBL = LIVE ? SCORE_LIVE_BLOCKS : 8;  // most blocks of a chunk
  int bh_rel, chunk;
  score_work(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x, gridDim.y, bh_rel, chunk);
  const int bh = a.bh0 + bh_rel;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  // the wavefront index is uniform (readfirstlane tells the compiler so: its batch loop
  // then runs on scalar branches)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane & 15, grp = lane >> 4;
  const int P = a.P;

  __shared__ float s_sc[CBL * BK];  // the chunk's scores, stored at the end
  // LIVE (destructive selection): the chunk's rows in play, compacted -- the ring row and the
  // physical row of the e-th of them, and the count per block
  __shared__ uint32_t s_lrow[LIVE ? CBL * BK : 1];
  __shared__ uint32_t s_prow[LIVE && SHARED ? CBL * BK : 1];
  __shared__ int s_bcnt[LIVE ? CBL : 1];
  __shared__ float s_wmax[4];
  __shared__ float s_ent[ENT ? 4 : 1][G][3];
  // entropy calibration: lane `sub` < G keeps query sub's softmax piece over its rows
  float em = -INFINITY, ez = 0.0f, ew = 0.0f;
  constexpr float c2 = (float)(1.4426950408889634074 / 11.313708498984760390);  // log2(e) / sqrt(128)

  const int64_t t = a.seq_len[b];
  const int64_t c = a.pool_head[bh];
  const int64_t pend = pool_end(t, a.W, a.S);
  const int64_t row_lo = c + (int64_t)chunk * a.cb_score * BK;
  const int64_t row_hi = min(row_lo + (int64_t)a.cb_score * BK, pend);

  float wmax = -INFINITY;
  if (row_lo < row_hi) {
    float qf[G][8];
    const char *qb = (const char *)a.q + (((int64_t)b * a.Hq + (int64_t)h * G) * HD + sub * 8) * EB;
#pragma unroll
    for (int g = 0; g < G; ++g) load8(qb + (size_t)g * HD * EB, qf[g], T{});
    // exact products: 16-bit elements, no key outside the safe magnitudes in the pool,
    // and every query element zero or inside them (the same in every wavefront); decided
    // once the first keys are in flight, so that the wait for q does not delay them.
    // With eight queries the second tree would cost the kernel a wavefront per SIMD.
    constexpr bool CAN_FUSE = EB == 2 && G <= 4;
    bool exact_products = false;
    auto decide = [&]() {
      bool q_ok = true;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = fabsf(qf[g][i]);
          q_ok &= x == 0.0f || (x >= Q_SAFE_LO && x < Q_SAFE_HI);
        }
      exact_products =
          CAN_FUSE && a.kx_unknown == 0 &&
          __builtin_amdgcn_readfirstlane((int)(a.kx[bh] == 0u && ballot(!q_ok) == 0ull)) != 0;
    };
    const BufRes kb = make_buf((const char *)a.pool_k + (SHARED ? 0 : (size_t)bh * P * BK * HD * EB),
                               (uint64_t)P * BK * HD * EB);
    const uint32_t lane_b = (uint32_t)(sub * 8 * EB);  // the lane's 8 elements of a row
    float *srow = a.scores + (size_t)bh * P * BK;
    // row_lo is block aligned and the chunk spans fewer than P blocks, so one
    // subtraction wraps the ring index
    const int pb0 = (int)((row_lo / BK) % P);
    const int nrows = (int)(row_hi - row_lo);
    const int nblk_c = (nrows + BK - 1) / BK;  // blocks of the chunk (at most CBL)
    // shared pool: lane i < nblk_c holds the physical block of the chunk's block i, read out
    // by the wavefront for each batch (the batch's block is the same in every lane)
    int32_t phys_lane = 0;
    if constexpr (SHARED) {
      if (lane < nblk_c) {
        int pb = pb0 + lane;
        pb = pb >= P ? pb - P : pb;
        const int32_t ph = a.btab[(size_t)bh * P + pb];
        phys_lane = ph < 0 ? 0 : ph;
      }
    }
    // The rows scored: the chunk's rows, or (LIVE) only those in play -- the last selection's
    // kept rows and the positions that arrived after it.  A dropped row is neither read nor
    // scored; its score entry keeps what it held.  Wavefront w lists blocks w, w + 4, ...
    // (a chunk of LIVE spans more blocks, so that a pool with few rows in play costs few
    // workgroups).
    int nwork = nrows;
    if constexpr (LIVE) {
      const int64_t pend_last = pend_last_selection(a, bh);
      uint64_t lm[CBL / 4];
#pragma unroll
      for (int j = 0; j < CBL / 4; ++j) {
        const int bi = wave + 4 * j;
        bool live = false;
        if (bi < nblk_c) {
          int pb = pb0 + bi;
          pb = pb >= P ? pb - P : pb;
          const int rel = bi * BK + lane;
          live = rel < nrows && in_play(row_lo + rel, pend_last, a.mask[(size_t)bh * P + pb]);
        }
        lm[j] = ballot(live);
        if (lane == 0) s_bcnt[bi] = __popcll(lm[j]);
      }
      __syncthreads();
      // the blocks' first entries: an exclusive scan of the counts over lanes 0 .. CBL - 1
      const int cnt = lane < CBL ? s_bcnt[lane] : 0;
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < CBL; off <<= 1) {
        const int y = __shfl_up(incl, off);
        incl += lane >= off ? y : 0;
      }
      nwork = __builtin_amdgcn_readlane(incl, CBL - 1);
      const int excl = incl - cnt;
#pragma unroll
      for (int j = 0; j < CBL / 4; ++j) {
        const int bi = wave + 4 * j;
        const int first = __builtin_amdgcn_readlane(excl, bi);
        if ((lm[j] >> lane) & 1ull) {
          int pb = pb0 + bi;
          pb = pb >= P ? pb - P : pb;
          const int e = first + (int)popc_below(lm[j]);
          s_lrow[e] = (uint32_t)(pb * BK + lane);
          if constexpr (SHARED)
            s_prow[e] = (uint32_t)__builtin_amdgcn_readlane(phys_lane, bi) * BK + lane;
        }
      }
      __syncthreads();
    }
    const int ngroups = (nwork + 15) / 16;
    // Each wavefront takes row groups wave, wave + 4, ...; a batch is UNR of them
    // (UNR * 4 loads of 1 KB).  Two batches live in registers: the next batch's loads are
    // in flight while the current one is scored.
    auto issue = [&](Raw8<T> (&buf)[UNR][4], int g0) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int gi = g0 + 4 * u;
        int pb = pb0 + (gi >> 2);
        pb = pb >= P ? pb - P : pb;
#pragma unroll
        for (int l = 0; l < 4; ++l) {
          const int rel = gi * 16 + l * 4 + grp;
          if constexpr (LIVE) {
            // the e-th row in play (entries past them read zeros, or in the shared pool the
            // first block's first row, and are not kept)
            const bool ok = (gi < ngroups) & (rel < nwork);
            if constexpr (SHARED) {
              const uint32_t first = (uint32_t)__builtin_amdgcn_readlane(phys_lane, 0) * BK;
              const uint32_t prow = ok ? s_prow[ok ? rel : 0] : first;
              raw_load_nt((const char *)a.pool_k + (size_t)prow * (HD * EB) + lane_b, buf[u][l]);
            } else {
              const uint32_t off = ok ? s_lrow[ok ? rel : 0] * (uint32_t)(HD * EB) + lane_b : BUF_SKIP;
              buf_load_nt(kb, off, buf[u][l]);
            }
          } else if constexpr (SHARED) {
            // a row of the batch's block (the same in every lane) through the buffer
            // resource of the 1 GB pool segment that holds the block, so that every offset
            // stays inside a resource's range; rows past the chunk read zeros (offset
            // BUF_SKIP), with no branch
            constexpr uint32_t SEGB = (1u << 30) / (uint32_t)(BK * HD * EB);  // blocks per segment
            const int bi = min(gi >> 2, nblk_c - 1);
            const uint32_t phys = (uint32_t)__builtin_amdgcn_readlane(phys_lane, bi);
            const uint32_t seg = phys / SEGB, local = phys % SEGB;
            const uint64_t seg_bytes = (uint64_t)min((uint32_t)a.NB - seg * SEGB, SEGB) * BK * HD * EB;
            const BufRes sr = make_buf((const char *)a.pool_k + (size_t)seg * SEGB * BK * HD * EB, seg_bytes);
            const uint32_t row_b = (local * BK + (uint32_t)(rel & (BK - 1))) * (uint32_t)(HD * EB) + lane_b;
            const uint32_t off = ((gi < ngroups) & (rel < nrows)) ? row_b : BUF_SKIP;
            buf_load_nt(sr, off, buf[u][l]);
          } else {
            // rows past the chunk read zeros (offset BUF_SKIP), with no branch
            const uint32_t row_b = (uint32_t)(pb * BK + (rel & (BK - 1))) * (uint32_t)(HD * EB) + lane_b;
            const uint32_t off = ((gi < ngroups) & (rel < nrows)) ? row_b : BUF_SKIP;
            buf_load_nt(kb, off, buf[u][l]);
          }
        }
      }
    };
    // The group's max dot of a row, and the dot of query `sub` (lanes sub < G).  FUSED
    // (exact products): no infinities or NaNs can arise either, so the max may be the
    // hardware max (its choice between +0 and -0 vanishes in s + 0 below).
    auto group_dots = [&](const float (&kf)[8], float &dmine, auto fused) {
      constexpr bool FUSED = decltype(fused)::value;
      float c[G];
      dot_trees<FUSED, G>(qf, kf, c);
      float s = c[0];
      dmine = s;
#pragma unroll
      for (int g = 1; g < G; ++g) {
        const float d = c[g];
        if (ENT && g == sub) dmine = d;
        s = FUSED ? __builtin_fmaxf(s, d) : (d > s ? d : s);
      }
      return s;
    };
    auto score_with = [&](Raw8<T> (&buf)[UNR][4], int g0, auto fused) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int gi = g0 + 4 * u;  // rows past the chunk are zeros, scored but not kept
#pragma unroll
        for (int l = 0; l < 4; ++l) {
          // The plain tree's rows widen through byte permutes, the fused tree's through
          // shifts: the same values, but not code the compiler would hoist above the
          // choice of tree (all the batch's widened rows would then be live at once).
          float kf[8];
          if (CAN_FUSE && !decltype(fused)::value)
            raw_to_f_perm(buf[u][l], kf);
          else
            raw_to_f(buf[u][l], kf);
          float dmine;
          float s = group_dots(kf, dmine, fused);
          const int rel = gi * 16 + l * 4 + grp;
          if (ENT && sub < G && rel < nwork) ent_add(em, ez, ew, dmine * c2);
          s = s + 0.0f;  // a zero score is +0
          // s is needed in every lane here, so that the last tree level stays one DPP add
          // rather than a move plus an add sunk into the store's branch
          asm volatile("" : "+v"(s));
          if (sub == 0 && rel < nwork) s_sc[rel] = s;
        }
      }
    };
    // a uniform choice: a scalar branch per batch
    auto score = [&](Raw8<T> (&buf)[UNR][4], int g0) {
      if (exact_products)
        score_with(buf, g0, std::true_type{});
      else
        score_with(buf, g0, std::false_type{});
    };
    constexpr int STEP = 4 * UNR;
    // The wavefront's nb batches, two per trip with no exit inside the trip, and issues
    // that are unconditional (a batch past the chunk reads nothing): every path into the
    // loop head then has the same loads in flight, so the wait before scoring a batch
    // counts only that batch's loads.
    const int nb = wave < ngroups ? (ngroups - 1 - wave) / STEP + 1 : 0;
    Raw8<T> bufA[UNR][4], bufB[UNR][4];
    int g0 = wave;
    issue(bufA, g0);
    decide();
    for (int i = 0; i + 2 <= nb; i += 2) {
      issue(bufB, g0 + STEP);
      score(bufA, g0);
      issue(bufA, g0 + 2 * STEP);
      score(bufB, g0 + STEP);
      g0 += 2 * STEP;
    }
    if (nb & 1) score(bufA, g0);
    // the chunk's scores leave in one pass, with the chunk's maximum over the rows scored
    __syncthreads();
    for (int rel = tid; rel < nwork; rel += NTHREADS) {
      uint32_t row;
      if constexpr (LIVE) {
        row = s_lrow[rel];
      } else {
        int pb = pb0 + (rel >> 6);
        pb = pb >= P ? pb - P : pb;
        row = (uint32_t)(pb * BK + (rel & (BK - 1)));
      }
      const float s = s_sc[rel];
      srow[row] = s;
      wmax = s > wmax ? s : wmax;
    }
  }
  wmax = wave_max(wmax);
  if (lane == 0) s_wmax[wave] = wmax;
  if (ENT) {
    // the four row groups of the wavefront, then the four wavefronts
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float m2 = __shfl_xor(em, off), z2 = __shfl_xor(ez, off), w2 = __shfl_xor(ew, off);
      ent_merge(em, ez, ew, m2, z2, w2);
    }
    if (lane < G) {
      s_ent[wave][lane][0] = em;
      s_ent[wave][lane][1] = ez;
      s_ent[wave][lane][2] = ew;
    }
  }
  __syncthreads();
  if (tid == 0)
    a.cmax[(size_t)bh * a.nch_score + chunk] =
        fmaxf(fmaxf(s_wmax[0], s_wmax[1]), fmaxf(s_wmax[2], s_wmax[3]));
  if (ENT && tid < G) {
    float m = s_ent[0][tid][0], z = s_ent[0][tid][1], w = s_ent[0][tid][2];
#pragma unroll
    for (int wv = 1; wv < 4; ++wv) ent_merge(m, z, w, s_ent[wv][tid][0], s_ent[wv][tid][1], s_ent[wv][tid][2]);
    float *e = a.ent + (((size_t)bh * a.nch_score + chunk) * G + tid) * 3;
    e[0] = m;
    e[1] = z;
    e[2] = w;
  }
}

// ---------------------------------------------------------------------------------------
// selection
// ---------------------------------------------------------------------------------------

// w = max(1, floor(2^24 * 2^t)), t = (s - m) kappa; 2^t = 2^n * P(f), n = floor(t),
// f in [0, 1), P the degree-9 Taylor polynomial of 2^f with non-negative terms, so the
// result never decreases as s grows.
HK_DEV uint32_t calib_weight(float s, float m, float kap, const float *coeff) {
  float x = s - m;
  float t = x * kap;
  if (!(t >= -60.0f)) return 1u;
  float n = floorf(t);
  float f = t - n;
  float y = coeff[NCOEFF - 1];
#pragma unroll
  for (int i = NCOEFF - 2; i >= 0; --i) {
    float p = y * f;
    y = p + coeff[i];
  }
  float e = ldexpf(y, (int)n);
  float big = e * 16777216.0f;
  uint32_t w = (uint32_t)floorf(big);
  return w < 1u ? 1u : w;
}

// monotone radix key of a weight: float bits relative to 1.0 (w in [1, 2^24])
HK_DEV uint32_t wkey(uint32_t w) { return __float_as_uint((float)w) - 0x3F800000u; }
HK_DEV uint32_t key_to_w(uint32_t k) { return (uint32_t)__uint_as_float(k + 0x3F800000u); }

HK_DEV uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, off);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off);
    v += ((uint64_t)hi << 32) | lo;
  }
  return v;
}

constexpr int NW = SEL_THREADS / 64;  // wavefronts of the select workgroup
constexpr int UA = 4;                  // 16-byte loads in flight per lane in the pool passes

// A candidate of the cut bucket b1 packs its survivor block j and the low 16 bits of its
// key: (j << 16) | (key & 0xffff); its key is (b1 << 16) | (cand & 0xffff).
struct SelShared {
  unsigned long long hist[NB1];  // mass histogram of level 1
  unsigned long long h2[256], h3[256];  // levels 2 and 3 (cleared when the workgroup starts)
  union {
    uint32_t cand[CAND_CAP];     // the cut bucket's tokens
    float fold[NW][2][HD];       // after the selection: the wavefronts' sums of a condensing block
  };
  unsigned long long red[2][NW];
  unsigned long long wt[NW];     // level-1 cut: each wavefront's segment of 256 buckets
  float fred[NW];
  uint32_t ncand;
  unsigned long long carry;
  unsigned long long total;
  uint32_t w_th, r;
  uint32_t cand_base;  // split select: the workgroup's first slot in the head's candidate list
};
// Dynamic LDS: SelShared, then uint32_t blk[P], per survivor block gt | eq << 16.
constexpr size_t sel_lds_bytes(int P) { return sizeof(SelShared) + sizeof(uint32_t) * (size_t)P; }

HK_DEV void clear_levels(SelShared &sh) {
  for (int i = threadIdx.x; i < 256; i += SEL_THREADS) sh.h2[i] = sh.h3[i] = 0ull;
}

// the workgroup's sums of two values, with one barrier
HK_DEV void block_sum2_u64(uint64_t &x, uint64_t &y, SelShared &sh) {
  const int tid = threadIdx.x;
  x = wave_sum_u64(x);
  y = wave_sum_u64(y);
  if ((tid & 63) == 0) {
    sh.red[0][tid >> 6] = x;
    sh.red[1][tid >> 6] = y;
  }
  __syncthreads();
  uint64_t sx = 0, sy = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    sx += sh.red[0][w];
    sy += sh.red[1][w];
  }
  x = sx;
  y = sy;
}

HK_DEV uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = __shfl((uint32_t)v, src), hi = __shfl((uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

// inclusive prefix sums over the threads of the workgroup (thread order), or suffix sums
// (reverse order): a wavefront scan by lane exchanges, then a scan of the wavefront totals
HK_DEV uint64_t block_scan_u64(uint64_t mine, SelShared &sh, bool suffix) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pos = suffix ? 63 - lane : lane;  // position in the scan order inside the wave
  uint64_t v = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int src = suffix ? lane + off : lane - off;
    const uint64_t x = shfl_u64(v, src < 0 ? 0 : (src > 63 ? 63 : src));
    if (pos >= off) v += x;
  }
  if (pos == 63) sh.red[0][wave] = v;  // wave total
  __syncthreads();
  uint64_t before = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (suffix ? w > wave : w < wave) before += sh.red[0][w];
  __syncthreads();
  return before + v;
}

// The cut of a mass histogram: the largest bucket b with sum(h[b..]) >= target (1 <= target
// <= total), and *above = sum(h[b + 1 ..]).
// Over 256 buckets, by every wavefront on its own (no barrier): lane l sums
// buckets 4l .. 4l + 3, a suffix scan over the lanes finds the lane that holds the cut,
// and that lane walks its four buckets down.  The histogram must be complete and must
// not change until every wavefront has returned.
HK_DEV int find_cut256(const unsigned long long *h, uint64_t target, uint64_t *above, int nb = 256) {
  const int lane = threadIdx.x & 63;
  uint64_t v[4], mine = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[k] = 4 * lane + k < nb ? h[4 * lane + k] : 0ull;
    mine += v[k];
  }
  uint64_t incl = mine;  // sum(h[4 lane ..])
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t x = shfl_u64(incl, lane + off < 64 ? lane + off : 63);
    if (lane + off < 64) incl += x;
  }
  const uint64_t excl = incl - mine;  // sum(h[4 lane + 4 ..])
  const uint64_t hit = ballot(excl < target && incl >= target);
  const int src = hit ? __ffsll((long long)hit) - 1 : 0;
  int b = 4 * lane;
  uint64_t acc = excl;
#pragma unroll
  for (int k = 3; k >= 0; --k) {
    if (acc + v[k] >= target) {
      b = 4 * lane + k;
      break;
    }
    acc += v[k];
  }
  *above = shfl_u64(acc, src);
  return __shfl(b, src);
}

// The cut over the NB1 level-1 buckets, with one barrier: wavefront w totals buckets
// [256 w, 256 w + 256); then every wavefront finds the segment that holds the cut from the
// totals and the bucket inside it with find_cut256.  The histogram must be complete, and
// must not change (nor sh.wt) until every wavefront has returned.
HK_DEV int find_cut_l1(SelShared &sh, uint64_t target, uint64_t *above) {
  static_assert(NW * 256 >= NB1, "the wavefronts' segments cover the level-1 buckets");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t mine = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = 256 * wave + 4 * lane + k;
    mine += i < NB1 ? sh.hist[i] : 0ull;
  }
  mine = wave_sum_u64(mine);
  if (lane == 0) sh.wt[wave] = mine;
  __syncthreads();
  // suffix sums of the segment totals over lanes 0 .. NW - 1
  const uint64_t t = lane < NW ? sh.wt[lane] : 0ull;
  uint64_t incl = t;
#pragma unroll
  for (int off = 1; off < NW; off <<= 1) {
    const uint64_t x = shfl_u64(incl, lane + off < 64 ? lane + off : 63);
    if (lane + off < NW) incl += x;
  }
  const uint64_t excl = incl - t;
  const uint64_t hit = ballot(lane < NW && excl < target && incl >= target);
  const int seg = hit ? __ffsll((long long)hit) - 1 : 0;
  const uint64_t above_seg = shfl_u64(excl, seg);
  uint64_t above_in = 0;
  const int b = find_cut256(sh.hist + 256 * seg, target - above_seg, &above_in, NB1 - 256 * seg);
  *above = above_seg + above_in;
  return 256 * seg + b;
}

// the sum of 16-lane groups (lanes 16q .. 16q + 15), in every lane of the group
HK_DEV uint32_t sum16(uint32_t v) {
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// The head's pool as the select stage sees it.
struct SelGeo {
  int bh;
  int64_t t, c, pend, E, u0;
  int nblk;   // pool blocks, at most P
  int nx;     // condensing blocks (they come first)
  int nub;    // survivor blocks
  int pb_lo;  // ring block of the pool head
  float kap;  // calibration slope
  size_t rowbase;
  HK_DEV int ring(int i, int P) const {
    const int pb = pb_lo + i;
    return pb >= P ? pb - P : pb;
  }
};

HK_DEV SelGeo sel_geo(const Args &a, int bh) {
  SelGeo g;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  g.bh = bh;
  g.t = a.seq_len[b];
  g.c = a.pool_head[bh];
  g.pend = pool_end(g.t, a.W, a.S);
  const int64_t N = g.pend - g.c;
  g.E = plan_E(N, a.mode, a.S_cap);
  g.u0 = g.c + (int64_t)BK * g.E;
  g.nblk = (int)((g.pend + BK - 1) / BK - g.c / BK);
  g.nx = (int)g.E;
  g.nub = g.nblk - g.nx;
  g.pb_lo = (int)((g.c / BK) % a.P);
  // both slopes loaded, then a select of values: a select between the argument block and
  // a global address (which the compiler forms from a plain load under a branch) copies
  // the whole argument block to scratch
  const float kfix = a.kappa[h];
  const float kfit = __builtin_nontemporal_load(&a.head[bh].kappa);
  g.kap = a.calibration ? kfit : kfix;
  g.rowbase = (size_t)bh * a.P * BK;
  return g;
}

// m: max of the score workgroups' maxima (every thread gets it)
HK_DEV float sel_max(const Args &a, int bh, SelShared &sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float mx = -INFINITY;
  for (int i = tid; i < a.nch_score; i += SEL_THREADS) mx = fmaxf(mx, a.cmax[(size_t)bh * a.nch_score + i]);
  mx = wave_max(mx);
  if (lane == 0) sh.fred[wave] = mx;
  __syncthreads();
  float m = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) m = fmaxf(m, sh.fred[w]);
  return m;
}

// pass A over pool blocks [lo, hi): weights (written), pool and survivor mass, level-1
// histogram of the survivors' mass in sh.hist.  Wavefront `wave` takes blocks
// lo + 4 wave + 64 k .. + 3, one 16-byte load per lane each.
HK_DEV void sel_pass_a(const Args &a, const SelGeo &g, float m, int lo, int hi, SelShared &sh,
                       uint64_t &my_all, uint64_t &my_u, bool &bad) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, r4 = (lane & 15) * 4;  // a load: block q4 of 4, rows r4 .. r4 + 3
  const int P = a.P;
  // destructive selection: the rows in play are the last selection's kept rows (the mask
  // words as it left them) and the positions since it; a dropped row weighs 0
  const int64_t pend_last = a.destructive ? pend_last_selection(a, g.bh) : 0;
  for (int i0 = lo + wave * 4; i0 < hi; i0 += 4 * NW * UA) {
    float4 sv[UA];
    uint64_t mw[UA];
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int i = i0 + u * 4 * NW + q4;
      sv[u] = i < hi ? *reinterpret_cast<const float4 *>(a.scores + g.rowbase + (size_t)g.ring(i, P) * BK + r4)
                     : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      mw[u] = (a.destructive && i < hi) ? a.mask[(size_t)g.bh * P + g.ring(i, P)] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int i = i0 + u * 4 * NW + q4;
      if (i < hi) {
        const int64_t p = g.c + (int64_t)i * BK + r4;
        const float s4[4] = {sv[u].x, sv[u].y, sv[u].z, sv[u].w};
        uint32_t w4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bool valid = p + k < g.pend;
          bad |= valid && !isfinite(s4[k]);
          const bool live = !a.destructive || in_play(p + k, pend_last, mw[u]);
          w4[k] = (valid && live) ? calib_weight(s4[k], m, g.kap, a.coeff) : 0u;
          my_all += w4[k];
          if (valid && live && i >= g.nx) {
            my_u += w4[k];
            atomicAdd(&sh.hist[wkey(w4[k]) >> 16], (unsigned long long)w4[k]);
          }
        }
        uint32_t *wp = a.weights + g.rowbase + (size_t)g.ring(i, P) * BK + r4;
        if (p + 3 < g.pend) {
          *reinterpret_cast<uint4 *>(wp) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (p + k < g.pend) wp[k] = w4[k];
        }
      }
    }
  }
}

// pass B over survivor blocks [jlo, jhi): per block the weights above the cut bucket b1
// (into cnt[j], LDS, or the block's blkinfo.x in memory when SPLIT), and the bucket's
// tokens gathered into cand through the counter *ncand
template <bool SPLIT>
HK_DEV void sel_pass_b(const Args &a, int bh, const SelGeo &g, int b1, int jlo, int jhi, uint32_t *cnt,
                       uint32_t *cand, uint32_t *ncand) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, r4 = (lane & 15) * 4;
  const int P = a.P;
  for (int j0 = jlo + wave * 4; j0 < jhi; j0 += 4 * NW * UA) {
    uint4 wv[UA];
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int j = j0 + u * 4 * NW + q4;
      wv[u] = j < jhi ? *reinterpret_cast<const uint4 *>(a.weights + g.rowbase + (size_t)g.ring(g.nx + j, P) * BK + r4)
                      : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int jb = j0 + u * 4 * NW;  // wave-uniform
      if (jb >= jhi) break;
      const int j = jb + q4;
      const int64_t p = g.u0 + (int64_t)j * BK + r4;
      const uint32_t w4[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
      uint32_t n_above = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // (a row dropped by a destructive selection weighs 0 and has no key)
        const bool valid = j < jhi && p + k < g.pend && w4[k] != 0u;
        const uint32_t key = wkey(w4[k]);
        const int kb = (int)(key >> 16);
        n_above += (valid && kb > b1) ? 1u : 0u;
        const bool in = valid && kb == b1;
        const uint64_t inb = ballot(in);
        if (inb) {  // wave-uniform
          uint32_t base = 0;
          if (lane == 0) base = atomicAdd(ncand, (uint32_t)__popcll(inb));
          base = __shfl(base, 0);
          const uint32_t slot = base + popc_below(inb);
          if (in && slot < (uint32_t)CAND_CAP) cand[slot] = ((uint32_t)j << 16) | (key & 0xffffu);
        }
      }
      n_above = sum16(n_above);
      if ((lane & 15) == 0 && j < jhi) {
        if (SPLIT)
          reinterpret_cast<uint32_t *>(a.blkinfo + (size_t)bh * P + g.ring(g.nx + j, P))[0] = n_above;
        else
          cnt[j] = n_above;
      }
    }
  }
}

// From the cut bucket to the head's plan: the exact threshold w_th and the r ties kept
// (from the candidates in LDS, or, for a bucket too full for LDS, from the weights in
// memory), per-block counts, the scan over blocks, and the plan.  blk[j] holds the
// weights above the bucket of each survivor block, sh.cand / sh.ncand the bucket's tokens.
HK_DEV void sel_finish(const Args &a, int bh, const SelGeo &g, SelShared &sh, uint32_t *blk, uint64_t W_all,
                       uint64_t W_U, uint64_t T, uint64_t R1, int b1) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = a.P;
  HeadInfo *hd = a.head + bh;
  const int64_t t = g.t, c = g.c, pend = g.pend, E = g.E, u0 = g.u0;
  const int nx = g.nx, nub = g.nub;
  const size_t rowbase = g.rowbase;
  auto ring = [&](int i) { return g.ring(i, P); };
  uint32_t w_th = 0, r = 0;
  uint64_t n_gt = 0;
  if (W_U > 0) {
    uint64_t above2, above3;
    const uint32_t ncand = sh.ncand;
    const uint32_t kb1 = (uint32_t)b1 << 16;
    if (ncand <= 64u) {
      // one wavefront: the largest weight v of the bucket whose candidates of weight >= v
      // reach R1 is w_th; r ties at w_th make up what those above it leave to R1
      if (wave == 0) {
        const bool have = lane < (int)ncand;
        const uint32_t w = have ? key_to_w(kb1 | (sh.cand[lane] & 0xffffu)) : 0u;
        uint64_t gt = 0, ge = 0;
        for (uint32_t k = 0; k < ncand; ++k) {
          const uint32_t x = key_to_w(kb1 | (sh.cand[k] & 0xffffu));
          gt += x > w ? x : 0u;
          ge += x >= w ? x : 0u;
        }
        const uint64_t hit = ballot(have && gt < R1 && ge >= R1);
        const int src = hit ? __ffsll((long long)hit) - 1 : 0;
        const uint32_t wt = (uint32_t)__shfl((int)w, src);
        const uint64_t gts = shfl_u64(gt, src);
        if (lane == 0) {
          sh.w_th = wt;
          sh.r = wt ? (uint32_t)((R1 - gts + wt - 1) / wt) : 0u;
        }
      }
      __syncthreads();
      w_th = sh.w_th;
      r = sh.r;
    } else if (ncand <= (uint32_t)CAND_CAP) {
      // levels 2 and 3 over the candidates in LDS (their histograms start cleared)
      for (uint32_t i = tid; i < ncand; i += SEL_THREADS) {
        const uint32_t k = kb1 | (sh.cand[i] & 0xffffu);
        atomicAdd(&sh.h2[(k >> 8) & 255u], (unsigned long long)key_to_w(k));
      }
      __syncthreads();
      const int b2 = find_cut256(sh.h2, R1, &above2);
      const uint32_t pre = ((uint32_t)b1 << 8) | (uint32_t)b2;
      for (uint32_t i = tid; i < ncand; i += SEL_THREADS) {
        const uint32_t k = kb1 | (sh.cand[i] & 0xffffu);
        if ((k >> 8) == pre) atomicAdd(&sh.h3[k & 255u], (unsigned long long)key_to_w(k));
      }
      __syncthreads();
      const int b3 = find_cut256(sh.h3, R1 - above2, &above3);
      w_th = key_to_w((pre << 8) | (uint32_t)b3);
      r = (uint32_t)((R1 - above2 - above3 + w_th - 1) / w_th);
    }
    if (ncand <= (uint32_t)CAND_CAP) {
      // candidates above w_th and at w_th, per block
      for (uint32_t i = tid; i < ncand; i += SEL_THREADS) {
        const uint32_t cd = sh.cand[i];
        const uint32_t w = key_to_w(kb1 | (cd & 0xffffu));
        const uint32_t j = cd >> 16;
        if (w > w_th) atomicAdd(&blk[j], 1u);
        else if (w == w_th) atomicAdd(&blk[j], 1u << 16);
      }
    } else {
      // a bucket too full for LDS (for example many equal weights): levels 2 and 3 and
      // the per-block counts over the survivors' weights in memory
      for (int j = wave; j < nub; j += NW) {
        const int64_t p = u0 + (int64_t)j * BK + lane;
        if (p < pend) {
          const uint32_t w = a.weights[rowbase + (size_t)ring(nx + j) * BK + lane];
          const uint32_t k = wkey(w);
          if ((int)(k >> 16) == b1) atomicAdd(&sh.h2[(k >> 8) & 255u], (unsigned long long)w);
        }
      }
      __syncthreads();
      const int b2 = find_cut256(sh.h2, R1, &above2);
      const uint32_t pre = ((uint32_t)b1 << 8) | (uint32_t)b2;
      for (int j = wave; j < nub; j += NW) {
        const int64_t p = u0 + (int64_t)j * BK + lane;
        if (p < pend) {
          const uint32_t w = a.weights[rowbase + (size_t)ring(nx + j) * BK + lane];
          const uint32_t k = wkey(w);
          if ((k >> 8) == pre) atomicAdd(&sh.h3[k & 255u], (unsigned long long)w);
        }
      }
      __syncthreads();
      const int b3 = find_cut256(sh.h3, R1 - above2, &above3);
      w_th = key_to_w((pre << 8) | (uint32_t)b3);
      r = (uint32_t)((R1 - above2 - above3 + w_th - 1) / w_th);
      for (int j = wave; j < nub; j += NW) {
        const int64_t p = u0 + (int64_t)j * BK + lane;
        uint32_t w = 0;
        if (p < pend) w = a.weights[rowbase + (size_t)ring(nx + j) * BK + lane];
        const uint64_t gtm = ballot(p < pend && w > w_th);
        const uint64_t eqm = ballot(p < pend && w == w_th);
        if (lane == 0) blk[j] = (uint32_t)__popcll(gtm) | ((uint32_t)__popcll(eqm) << 16);
      }
    }
    __syncthreads();

    // scan over survivor blocks in position order: first view row GT_before +
    // min(EQ_before, r), and EQ_before for the tie ranks of the mask bits
    if (nub <= SEL_THREADS) {
      // one round: no carry between rounds
      const uint32_t v = (tid < nub) ? blk[tid] : 0u;
      const uint64_t mine = (uint64_t)(v & 0xffffu) | ((uint64_t)(v >> 16) << 32);
      const uint64_t incl = block_scan_u64(mine, sh, false);
      const uint64_t before = incl - mine;
      if (tid < nub) {
        const uint32_t gt_b = (uint32_t)before, eq_b = (uint32_t)(before >> 32);
        a.blkinfo[(size_t)bh * P + ring(nx + tid)] = make_uint2(gt_b + min(eq_b, r), eq_b);
      }
      if (tid == SEL_THREADS - 1) sh.total = incl;
      __syncthreads();
      n_gt = sh.total & 0xffffffffull;
    } else {
    if (tid == 0) sh.carry = 0ull;
    __syncthreads();
    for (int base = 0; base < nub; base += SEL_THREADS) {
      const int i = base + tid;
      const uint32_t v = (i < nub) ? blk[i] : 0u;
      const uint64_t mine = (uint64_t)(v & 0xffffu) | ((uint64_t)(v >> 16) << 32);
      const uint64_t incl = block_scan_u64(mine, sh, false);
      if (tid == SEL_THREADS - 1) sh.total = incl;  // round total
      const uint64_t before = sh.carry + incl - mine;
      __syncthreads();
      const uint64_t total = sh.total;
      if (i < nub) {
        const uint32_t gt_b = (uint32_t)before, eq_b = (uint32_t)(before >> 32);
        a.blkinfo[(size_t)bh * P + ring(nx + i)] = make_uint2(gt_b + min(eq_b, r), eq_b);
      }
      if (tid == 0) sh.carry += total;
      __syncthreads();
    }
    n_gt = sh.carry & 0xffffffffull;
    }
  }

  if (tid == 0) {
    const int64_t kstar = (int64_t)n_gt + r;
    a.budget[bh] = (int32_t)kstar;
    a.n_condense[bh] = (int32_t)E;
    a.w_all[bh] = W_all;
    a.w_u[bh] = W_U;
    a.thresh[bh] = T;
    hd->t_plan = t;
    hd->c_plan = c;
    hd->w_th = w_th;
    hd->r = r;
    hd->kstar = (int32_t)kstar;
    hd->E = (int32_t)E;
    hd->nu_plan = a.cond_cursor[bh];
    hd->w_all = W_all;
    // the regularize policy: rewrite every head, none, or those whose budget lies in
    // [L_lower, L_upper]
    const int rw = a.reg_policy == HARDKV_REG_REWRITE ? 1
                   : a.reg_policy == HARDKV_REG_SPARSE ? 0
                   : a.reg_policy == HARDKV_REG_MTI ? ((kstar >= a.mti_lower && kstar <= a.mti_upper) ? 1 : 0)
                   : (mti_rewrites(kstar, pend - u0, a.mti_horizon, a.mti_c_view, a.mti_c_write, a.mti_c_scan,
                                   a.mti_c_hold, a.mti_c_gather, a.mti_fixed) ? 1 : 0);
    hd->rw = rw;
    hd->voff = (int64_t)bh * a.V_cap;  // the maximum-length layout; the flatten kernel packs SUM
    if (a.regularized) a.regularized[bh] = rw;
    if (rw && !a.view_sum && kstar > a.V_cap) atomicOr(a.error_word, HARDKV_ERR_VIEW_OVERFLOW);
  }
}

// The condensation of the head's E oldest blocks by the select workgroup itself (FUSE:
// the fused step, when at most FUSE_COND_BLOCKS blocks can condense per step), after the
// plan is written (its cursor read comes first).  MERGE folds the blocks one after
// another with the whole workgroup: each wavefront takes
// 4 of the block's 64 rows (16 lanes a row, 8 head dims a lane) and sums w k and w v over
// them; the wavefronts' sums meet in LDS (in the candidate buffer, free once the plan is
// written) and 256 threads add them to the slot in wavefront order.  Blocks that land on
// the same slot (more than C of them) are added in age order.
template <typename T>
HK_DEV void select_condense(const Args &a, int bh, const SelGeo &g, int32_t nu, uint64_t W_all, SelShared &sh) {
  constexpr int EB = Elem<T>::bytes;
  constexpr size_t ROWB = (size_t)HD * EB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane & 15, grp = lane >> 4;
  const int P = a.P, C = a.C;
  __syncthreads();
  if (a.mode == HARDKV_COND_MERGE) {
    const float inv = W_all ? (float)(1.0 / (double)W_all) : 0.0f;
    for (int64_t e = 0; e < g.E; ++e) {
      const size_t pb = (size_t)((g.c / BK + e) % P);
      const size_t sg = (size_t)bh * C + (size_t)((nu + e) % C);
      const bool fresh = a.cond_n[sg] == 0;  // (read before this block's count is added)
      const int row = wave * 4 + grp;
      const uint32_t wl = a.weights[((size_t)bh * P + pb) * BK + row];
      const char *base = (const char *)a.pool_k + pool_row0(a, bh, (int)pb) * ROWB;
      const size_t roff = (size_t)row * ROWB + sub * 8 * EB;
      Raw8<T> kr, vr;
      raw_load_nt(base + roff, kr);
      raw_load_nt((const char *)a.pool_v + pool_row0(a, bh, (int)pb) * ROWB + roff, vr);
      float kf[8], vf[8], ak[8], av[8];
      raw_to_f(kr, kf);
      raw_to_f(vr, vf);
      const float wf = (float)wl;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        ak[k] = wf * kf[k];
        av[k] = wf * vf[k];
      }
#pragma unroll
      for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          ak[k] += __shfl_xor(ak[k], off);
          av[k] += __shfl_xor(av[k], off);
        }
      }
      const uint64_t wsum = wave_sum_u64(sub == 0 ? (uint64_t)wl : 0ull);
      const int nlive = __popcll(ballot(sub == 0 && wl != 0u));
      if (lane < 16) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          sh.fold[wave][0][sub * 8 + k] = ak[k];
          sh.fold[wave][1][sub * 8 + k] = av[k];
        }
      }
      if (lane == 0) {
        sh.red[0][wave] = wsum;
        sh.red[1][wave] = (unsigned long long)nlive;
      }
      __syncthreads();
      if (tid < 2 * HD) {
        const int half = tid / HD, d = tid - half * HD;
        float acc = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) acc += sh.fold[w][half][d];
        float *num = (half ? a.cond_vn : a.cond_kn) + sg * HD + d;
        *num = (fresh ? 0.0f : *num) + acc * inv;
      }
      if (tid == 0) {
        uint64_t ws = 0;
        int n = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          ws += sh.red[0][w];
          n += (int)sh.red[1][w];
        }
        a.cond_omega[sg] = (fresh ? 0.0f : a.cond_omega[sg]) + (W_all ? (float)((double)ws / (double)W_all) : 0.0f);
        a.cond_n[sg] += n;
      }
      __syncthreads();  // (the sums are read before the next block writes them)
    }
  }
  if (wave == 0) condense_advance(a, bh, g.c, g.E, nu);
}

// The whole select stage of one head in one workgroup (pools up to SEL_SPLIT_MIN slices);
// FUSE: and the condensation (T: the storage type of the rows it merges).
template <typename T, bool FUSE>
__global__ __launch_bounds__(SEL_THREADS) void hardkv_select(Args a) {
  const int bh = a.bh0 + blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int P = a.P;
  extern __shared__ unsigned char smem_raw[];
  SelShared &sh = *reinterpret_cast<SelShared *>(smem_raw);
  uint32_t *blk = reinterpret_cast<uint32_t *>(smem_raw + sizeof(SelShared));
  const SelGeo g = sel_geo(a, bh);
  const int32_t nu = FUSE ? a.cond_cursor[bh] : 0;

  for (int i = tid; i < NB1; i += SEL_THREADS) sh.hist[i] = 0ull;
  clear_levels(sh);
  if (tid == 0) sh.ncand = 0;
  // every mask word starts empty; the rewrite kernel writes the survivor blocks' words (a
  // destructive selection reads the last selection's words in pass A first)
  if (!a.destructive)
    for (int i = tid; i < P; i += SEL_THREADS) a.mask[(size_t)bh * P + i] = 0ull;
  const float m = sel_max(a, bh, sh);  // (its barrier also orders the clears above)

  uint64_t my_all = 0, my_u = 0;
  bool bad = false;
  sel_pass_a(a, g, m, 0, g.nblk, sh, my_all, my_u, bad);
  if (ballot(bad) && lane == 0) atomicOr(a.error_word, HARDKV_ERR_NONFINITE);
  uint64_t W_all = my_all, W_U = my_u;
  block_sum2_u64(W_all, W_U, sh);
  if (a.destructive)  // (after the barriers above: every thread's pass A has read its words)
    for (int i = tid; i < P; i += SEL_THREADS) a.mask[(size_t)bh * P + i] = 0ull;
  const uint64_t Tm = ((uint64_t)a.pq * W_U + 65535ull) >> 16;
  uint64_t R1 = 0;
  int b1 = 0;
  if (W_U > 0) {
    uint64_t above1;
    b1 = find_cut_l1(sh, Tm, &above1);
    R1 = Tm - above1;  // mass still needed from the cut bucket
    sel_pass_b<false>(a, bh, g, b1, 0, g.nub, blk, sh.cand, &sh.ncand);
    __syncthreads();
  }
  sel_finish(a, bh, g, sh, blk, W_all, W_U, Tm, R1, b1);
  if (FUSE) select_condense<T>(a, bh, g, nu, W_all, sh);
}

// Split select, for long pools: the head's blocks in slices of SEL_SLICE_BLOCKS, one
// workgroup each, for the two passes over every token; four kernels in stream order.
//
// hardkv_sel_weigh, grid (nsp, B*Hkv): pass A over the slice's pool blocks; the slice's
//   histogram and masses go to memory (phist, psum); the slice's share of the mask words
//   is cleared.
__global__ __launch_bounds__(SEL_THREADS) void hardkv_sel_weigh(Args a) {
  const int bh = a.bh0 + blockIdx.y, slice = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int P = a.P;
  extern __shared__ unsigned char smem_raw[];
  SelShared &sh = *reinterpret_cast<SelShared *>(smem_raw);
  const SelGeo g = sel_geo(a, bh);

  for (int i = tid; i < NB1; i += SEL_THREADS) sh.hist[i] = 0ull;
  const int zs = (P + a.nsp - 1) / a.nsp;
  if (!a.destructive)  // (a destructive selection's words are read by every slice: the cut clears them)
    for (int i = slice * zs + tid; i < min(P, (slice + 1) * zs); i += SEL_THREADS) a.mask[(size_t)bh * P + i] = 0ull;
  if (slice == 0 && tid == 0) a.selh[bh].ncand = 0u;
  const float m = sel_max(a, bh, sh);

  uint64_t my_all = 0, my_u = 0;
  bool bad = false;
  const int lo = slice * SEL_SLICE_BLOCKS, hi = min(g.nblk, lo + SEL_SLICE_BLOCKS);
  sel_pass_a(a, g, m, lo, hi, sh, my_all, my_u, bad);
  if (ballot(bad) && lane == 0) atomicOr(a.error_word, HARDKV_ERR_NONFINITE);
  uint64_t s_all = my_all, s_u = my_u;
  block_sum2_u64(s_all, s_u, sh);  // (its barrier also orders the histogram)
  unsigned long long *ph = a.phist + ((size_t)bh * a.nsp + slice) * NB1;
  for (int i = tid; i < NB1; i += SEL_THREADS) ph[i] = sh.hist[i];
  if (tid == 0) {
    a.psum[((size_t)bh * a.nsp + slice) * 2] = s_all;
    a.psum[((size_t)bh * a.nsp + slice) * 2 + 1] = s_u;
  }
}

// the head's masses from the slices' (every thread gets them)
HK_DEV void sel_masses(const Args &a, int bh, uint64_t &W_all, uint64_t &W_U) {
  W_all = 0;
  W_U = 0;
  const unsigned long long *ps = a.psum + (size_t)bh * a.nsp * 2;
  for (int k0 = 0; k0 < a.nsp; k0 += 8) {  // eight slices' loads in flight
    unsigned long long x[8][2];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool in = k0 + u < a.nsp;
      x[u][0] = in ? ps[(k0 + u) * 2] : 0ull;
      x[u][1] = in ? ps[(k0 + u) * 2 + 1] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      W_all += x[u][0];
      W_U += x[u][1];
    }
  }
}

// hardkv_sel_cut, grid (B*Hkv): the head's masses and histogram from the slices', the
//   cut bucket and the mass still needed from it, saved for the next two kernels.
__global__ __launch_bounds__(SEL_THREADS) void hardkv_sel_cut(Args a) {
  const int bh = a.bh0 + blockIdx.x;
  const int tid = threadIdx.x;
  extern __shared__ unsigned char smem_raw[];
  SelShared &sh = *reinterpret_cast<SelShared *>(smem_raw);
  if (a.destructive)  // every slice has read the last selection's words
    for (int i = tid; i < a.P; i += SEL_THREADS) a.mask[(size_t)bh * a.P + i] = 0ull;
  uint64_t W_all, W_U;
  sel_masses(a, bh, W_all, W_U);
  const uint64_t T = ((uint64_t)a.pq * W_U + 65535ull) >> 16;
  uint64_t above1 = 0;
  int b1 = 0;
  if (W_U > 0) {
    // the thread's buckets tid, tid + 1024, ... summed over the slices, four slices'
    // loads per bucket in flight
    constexpr int PER = (NB1 + SEL_THREADS - 1) / SEL_THREADS;
    const unsigned long long *ph = a.phist + (size_t)bh * a.nsp * NB1;
    unsigned long long acc[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) acc[q] = 0ull;
    for (int k0 = 0; k0 < a.nsp; k0 += 4) {
      unsigned long long x[4][PER];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          const int i = tid + q * SEL_THREADS;
          x[u][q] = (k0 + u < a.nsp && i < NB1) ? ph[(size_t)(k0 + u) * NB1 + i] : 0ull;
        }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < PER; ++q) acc[q] += x[u][q];
    }
#pragma unroll
    for (int q = 0; q < PER; ++q)
      if (tid + q * SEL_THREADS < NB1) sh.hist[tid + q * SEL_THREADS] = acc[q];
    __syncthreads();
    b1 = find_cut_l1(sh, T, &above1);
  }
  if (tid == 0) {
    SelHead *sx = a.selh + bh;
    sx->w_all = W_all;
    sx->w_u = W_U;
    sx->T = T;
    sx->R1 = T - above1;
    sx->b1 = b1;
  }
}

// hardkv_sel_count, grid (nsp, B*Hkv): pass B over the slice's survivor blocks: counts
//   into blkinfo.x; the cut bucket's tokens gathered in LDS, then appended to cand_g at
//   an offset reserved with one device-wide atomic per workgroup.
__global__ __launch_bounds__(SEL_THREADS) void hardkv_sel_count(Args a) {
  const int bh = a.bh0 + blockIdx.y, slice = blockIdx.x;
  const int tid = threadIdx.x;
  extern __shared__ unsigned char smem_raw[];
  SelShared &sh = *reinterpret_cast<SelShared *>(smem_raw);
  SelHead *sx = a.selh + bh;
  if (sx->w_u == 0) return;  // uniform: nothing to cut
  const int b1 = sx->b1;
  const SelGeo g = sel_geo(a, bh);
  const int lo = max(slice * SEL_SLICE_BLOCKS, g.nx) - g.nx;
  const int hi = min((slice + 1) * SEL_SLICE_BLOCKS, g.nblk) - g.nx;
  if (lo >= hi) return;  // uniform
  if (tid == 0) sh.ncand = 0;
  __syncthreads();
  sel_pass_b<true>(a, bh, g, b1, lo, hi, nullptr, sh.cand, &sh.ncand);
  __syncthreads();
  const uint32_t n = sh.ncand;  // may exceed CAND_CAP: the total then does too
  if (n == 0) return;           // uniform
  if (tid == 0) sh.cand_base = atomicAdd(&sx->ncand, n);
  __syncthreads();
  const uint32_t base = sh.cand_base;
  uint32_t *cg = a.cand_g + (size_t)bh * CAND_CAP;
  for (uint32_t i = tid; i < min(n, (uint32_t)CAND_CAP); i += SEL_THREADS)
    if (base + i < (uint32_t)CAND_CAP) cg[base + i] = sh.cand[i];
}

// hardkv_sel_finish, grid (B*Hkv): the per-block counts and the candidates back into LDS,
//   then the rest of the select stage as in the one-workgroup kernel (FUSE: with the
//   condensation).
template <typename T, bool FUSE>
__global__ __launch_bounds__(SEL_THREADS) void hardkv_sel_finish(Args a) {
  const int bh = a.bh0 + blockIdx.x;
  const int tid = threadIdx.x;
  const int P = a.P;
  extern __shared__ unsigned char smem_raw[];
  SelShared &sh = *reinterpret_cast<SelShared *>(smem_raw);
  uint32_t *blk = reinterpret_cast<uint32_t *>(smem_raw + sizeof(SelShared));
  const SelGeo g = sel_geo(a, bh);
  const int32_t nu = FUSE ? a.cond_cursor[bh] : 0;
  const SelHead *sx = a.selh + bh;
  const uint64_t W_all = sx->w_all, W_U = sx->w_u, Tm = sx->T;
  uint64_t R1 = 0;
  int b1 = 0;
  clear_levels(sh);  // (ordered before sel_finish by the barrier below, or unused)
  if (W_U > 0) {
    R1 = sx->R1;
    b1 = sx->b1;
    const uint32_t nc = sx->ncand;
    if (tid == 0) sh.ncand = nc;
    if (nc <= (uint32_t)CAND_CAP)
      for (uint32_t i = tid; i < nc; i += SEL_THREADS) sh.cand[i] = a.cand_g[(size_t)bh * CAND_CAP + i];
    for (int j = tid; j < g.nub; j += SEL_THREADS)
      blk[j] = reinterpret_cast<const uint32_t *>(a.blkinfo + (size_t)bh * P + g.ring(g.nx + j, P))[0];
    __syncthreads();
  }
  sel_finish(a, bh, g, sh, blk, W_all, W_U, Tm, R1, b1);
  if (FUSE) select_condense<T>(a, bh, g, nu, W_all, sh);
}

// Flatten Index to the sum: one workgroup scans n_u = k* (rewritten heads) or 0 over
// the units in order; head u's view starts at row voff_u = sum of n over units before u.
__global__ __launch_bounds__(SEL_THREADS) void hardkv_flatten(Args a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int BH = a.B * a.Hkv;
  __shared__ int64_t s_wave[NW];
  __shared__ int64_t s_carry;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < BH; base += SEL_THREADS) {
    const int u = base + tid;
    int64_t n = 0;
    if (u < BH) n = a.head[u].rw ? (int64_t)a.head[u].kstar : 0;
    int64_t v = n;  // inclusive scan inside the wavefront
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int src = lane - off < 0 ? 0 : lane - off;
      const uint32_t lo = __shfl((uint32_t)v, src), hi = __shfl((uint32_t)((uint64_t)v >> 32), src);
      const int64_t x = (int64_t)(((uint64_t)hi << 32) | lo);
      if (lane >= off) v += x;
    }
    if (lane == 63) s_wave[wave] = v;
    __syncthreads();
    int64_t before = s_carry, total = s_carry;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      before += w < wave ? s_wave[w] : 0;
      total += s_wave[w];
    }
    if (u < BH) {
      const int64_t off = before + v - n;
      a.head[u].voff = off;
      a.view_off[u] = (int32_t)min(off, (int64_t)INT32_MAX);
    }
    __syncthreads();
    if (tid == 0) s_carry = total;
    __syncthreads();
  }
  if (tid == 0) {
    a.view_off[BH] = (int32_t)min(s_carry, (int64_t)INT32_MAX);
    if (s_carry > a.view_rows) atomicOr(a.error_word, HARDKV_ERR_VIEW_OVERFLOW);
  }
}

// ---------------------------------------------------------------------------------------
// calibration temperature fitted by entropy
// ---------------------------------------------------------------------------------------
constexpr int FIT_THREADS = 512;  // 2 waves per SIMD: the 3 x 17 per-candidate values stay in registers
constexpr int FIT_NW = FIT_THREADS / 64;
constexpr int FIT_UNR = 8;          // score loads in flight per thread
constexpr float FIT_FAR = 1.0e30f;  // distance below the max of a padding row (times any slope: finite)

HK_DEV double shfl_xor_d(double v, int off) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = __shfl_xor((uint32_t)u, off), hi = __shfl_xor((uint32_t)(u >> 32), off);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Sums over the wavefront's 64 lanes of each of the NV values v[0..NV), in six exchange
// steps that each halve the values a lane holds: at the step of offset o, a lane with bit
// o clear keeps the lower half of its values and one with it set the upper half (the
// upper half one shorter, padded with zero, when the count is odd); each adds what its
// partner lane ^ o held of the half it keeps.  Partners have made the same choices at the
// earlier steps, so they hold the same values.  37 exchanges for NV = 34, against 6 NV
// for a butterfly per value.  Returns the index whose sum v[0] now holds, or -1 for a
// lane left with padding.
template <int NV>
HK_DEV int wave_sum_halving(double (&v)[NV]) {
  static_assert(NV >= 1 && NV <= 64, "one value per lane at the end");
  const int lane = threadIdx.x & 63;
  int lo = 0, cnt = NV;
  int n = NV;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const int h = (n + 1) / 2;
    const bool up = (lane & off) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const double x = v[i], y = i + h < n ? v[i + h] : 0.0;
      v[i] = (up ? y : x) + shfl_xor_d(up ? x : y, off);
    }
    if (up) {
      lo += h;
      cnt = max(0, cnt - h);
    } else {
      cnt = min(cnt, h);
    }
    n = h;
  }
  return cnt > 0 ? lo : -1;
}

// The target entropy (nats) of head bh: the mean over the group's queries of the entropy
// of their raw attention over the pool, merged from the per-chunk softmax pieces the
// score kernel left; and the head's max score.  Every thread gets both.
HK_DEV void fit_target(const Args &a, int bh, double &H, float &m) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.G;
  __shared__ float s_piece[FIT_NW][8][3];
  __shared__ double s_hq[8];
  __shared__ float s_mx[FIT_NW];
  __shared__ double s_H;
  __shared__ float s_m;
  {
    // each thread merges, per query, the pieces of chunks tid, tid + FIT_THREADS, ...;
    // then the lanes of a wavefront, then the wavefronts
    float pm[8], pz[8], pw[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      pm[g] = -INFINITY;
      pz[g] = pw[g] = 0.0f;
    }
    for (int ch = tid; ch < a.nch_score; ch += FIT_THREADS) {
      const float *e = a.ent + ((size_t)bh * a.nch_score + ch) * G * 3;
#pragma unroll
      for (int g = 0; g < 8; ++g)
        if (g < G) ent_merge(pm[g], pz[g], pw[g], e[g * 3], e[g * 3 + 1], e[g * 3 + 2]);
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (g >= G) break;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(pm[g], off), z2 = __shfl_xor(pz[g], off), w2 = __shfl_xor(pw[g], off);
        ent_merge(pm[g], pz[g], pw[g], m2, z2, w2);
      }
      if (lane == 0) {
        s_piece[wave][g][0] = pm[g];
        s_piece[wave][g][1] = pz[g];
        s_piece[wave][g][2] = pw[g];
      }
    }
  }
  float mx = -INFINITY;
  for (int i = tid; i < a.nch_score; i += FIT_THREADS) mx = fmaxf(mx, a.cmax[(size_t)bh * a.nch_score + i]);
  mx = wave_max(mx);
  if (lane == 0) s_mx[wave] = mx;
  __syncthreads();
  if (tid < G) {
    float m1 = s_piece[0][tid][0], z = s_piece[0][tid][1], w = s_piece[0][tid][2];
    for (int wv = 1; wv < FIT_NW; ++wv)
      ent_merge(m1, z, w, s_piece[wv][tid][0], s_piece[wv][tid][1], s_piece[wv][tid][2]);
    const double hbits = z > 0.0f ? log2((double)z) - (double)w / (double)z : 0.0;
    s_hq[tid] = hbits * 0.69314718055994530942;  // nats
  }
  __syncthreads();
  if (tid == 0) {
    double h = 0.0;
    for (int g = 0; g < G; ++g) h += s_hq[g];
    s_H = h / (double)G;
    float mm = -INFINITY;
    for (int w = 0; w < FIT_NW; ++w) mm = fmaxf(mm, s_mx[w]);
    s_m = mm;
  }
  __syncthreads();
  H = s_H;
  m = s_m;
}

// The candidates' slopes of a round over [lo, hi]: log2(e) / (sqrt(D) tau_k) with
// log2 tau_k = lo + k (hi - lo) / 16.
HK_DEV float fit_slope(double lo, double hi, int k) {
  return (float)(1.0 / sqrt((double)HD) * 1.4426950408889634074 / exp2(lo + k * ((hi - lo) / 16.0)));
}

// Per candidate k (threads k < FIT_POINTS get them): Z = sum 2^x2 and A = sum 2^x2 x2 over
// pool rows [r0, r1) (offsets from the pool head c), x2 = (s - m) slope_k the logit in
// bits.  Each thread sums rows r0 + tid, r0 + tid + FIT_THREADS, ... in that order in
// fp32, FIT_UNR loads in flight; a row past r1 scores FIT_FAR below the max, whose terms
// are exactly 0 (2^x2 is 0 and 0 * x2 is -0).  The workgroup sums in fp64: lanes by
// halving exchanges, then wavefronts in order.
HK_DEV void fit_sums(const Args &a, int bh, int64_t c, int64_t r0, int64_t r1, float m, double lo, double hi,
                     double &Z, double &A) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = a.P;
  const size_t rowbase = (size_t)bh * P * BK;
  __shared__ float s_ck[FIT_POINTS];
  __shared__ double s_acc[FIT_NW][2 * FIT_POINTS];
  if (tid < FIT_POINTS) s_ck[tid] = fit_slope(lo, hi, tid);
  __syncthreads();
  float ck[FIT_POINTS], cz[FIT_POINTS], ca[FIT_POINTS];
#pragma unroll
  for (int k = 0; k < FIT_POINTS; ++k) {
    cz[k] = ca[k] = 0.0f;
    ck[k] = s_ck[k];
  }
  for (int64_t i0 = r0 + tid; i0 < r1; i0 += (int64_t)FIT_UNR * FIT_THREADS) {
    float x0[FIT_UNR];
#pragma unroll
    for (int u = 0; u < FIT_UNR; ++u) {
      const int64_t i = i0 + (int64_t)u * FIT_THREADS;
      const int64_t p = c + (i < r1 ? i : r0);
      const float sc = a.scores[rowbase + (size_t)((p / BK) % P) * BK + (size_t)(p % BK)];
      x0[u] = i < r1 ? sc - m : -FIT_FAR;
    }
#pragma unroll
    for (int u = 0; u < FIT_UNR; ++u)
#pragma unroll
      for (int k = 0; k < FIT_POINTS; ++k) {
        const float x2 = x0[u] * ck[k];
        const float e = exp2_fast(x2);
        cz[k] += e;
        ca[k] = __builtin_fmaf(e, x2, ca[k]);
      }
  }
  double v[2 * FIT_POINTS];
#pragma unroll
  for (int k = 0; k < FIT_POINTS; ++k) {
    v[k] = (double)cz[k];
    v[FIT_POINTS + k] = (double)ca[k];
  }
  const int idx = wave_sum_halving(v);
  if (idx >= 0) s_acc[wave][idx] = v[0];
  __syncthreads();
  Z = A = 0.0;
  if (tid < FIT_POINTS) {
    for (int w = 0; w < FIT_NW; ++w) {
      Z += s_acc[w][tid];
      A += s_acc[w][FIT_POINTS + tid];
    }
  }
  __syncthreads();  // (s_ck and s_acc are reused by the next call)
}

// The next bracket from a round's sums (Z, A of candidate k in thread k): the first
// candidate whose calibrated entropy ln Z - ln 2 A / Z reaches H bounds it from above
// (the entropy grows with tau).  Every thread gets it.
HK_DEV void fit_next(double Z, double A, double H, double &lo, double &hi) {
  const int tid = threadIdx.x;
  __shared__ int s_reach[FIT_POINTS];
  __shared__ double s_lo, s_hi;
  if (tid < FIT_POINTS) s_reach[tid] = log(Z) - 0.69314718055994530942 * A / Z >= H;
  __syncthreads();
  if (tid == 0) {
    const double step = (hi - lo) / 16.0;
    int kk = 0;
    while (kk < FIT_POINTS && !s_reach[kk]) ++kk;
    double nlo = lo, nhi = hi;
    if (kk == 0) {
      nhi = lo;
    } else if (kk >= FIT_POINTS) {
      nlo = hi;
    } else {
      nlo = lo + (kk - 1) * step;
      nhi = lo + kk * step;
    }
    s_lo = nlo;
    s_hi = nhi;
  }
  __syncthreads();
  lo = s_lo;
  hi = s_hi;
  __syncthreads();
}

// tau = 2^(midpoint of the last bracket) (1 for an empty pool), into the head's plan
HK_DEV void fit_store(const Args &a, int bh, int64_t N, double lo, double hi) {
  if (threadIdx.x == 0) {
    const float tau = N > 0 ? (float)exp2(0.5 * (lo + hi)) : 1.0f;
    HeadInfo *hd = a.head + bh;
    hd->tau = tau;
    hd->kappa = (float)(1.4426950408889634074 / (sqrt((double)HD) * (double)tau));
    if (a.tau_fit) a.tau_fit[bh] = tau;
  }
}

HK_DEV int64_t fit_pool(const Args &a, int bh, int64_t &c) {
  const int b = bh / a.Hkv;
  c = a.pool_head[bh];
  return pool_end(a.seq_len[b], a.W, a.S) - c;
}

// hardkv_fit, grid (B*Hkv), 512 threads: one workgroup per head.  The target is the mean
// over the group's queries of the entropy (nats) of their raw attention over the pool;
// then five rounds of a 17-point grid on
// log2 tau in [-12, 12] find the bracket where the entropy of the calibrated
// softmax(s / (sqrt(D) tau)) over the pool reaches the target (it grows with tau); tau
// is the midpoint of the last bracket.
__global__ __launch_bounds__(FIT_THREADS) void hardkv_fit(Args a) {
  const int bh = a.bh0 + blockIdx.x;
  int64_t c;
  const int64_t N = fit_pool(a, bh, c);
  double H;
  float m;
  fit_target(a, bh, H, m);
  double lo = -12.0, hi = 12.0;
  for (int round = 0; round < FIT_ROUNDS && N > 0; ++round) {
    double Z, A;
    fit_sums(a, bh, c, 0, N, m, lo, hi, Z, A);
    fit_next(Z, A, H, lo, hi);
  }
  fit_store(a, bh, N, lo, hi);
}

// The same fit for long pools of few heads, the rows of each round spread over slices of
// FIT_SPLIT_ROWS rows (a.nfs per head), in FIT_ROUNDS + 2 kernels:
// hardkv_fit_prep, grid (B*Hkv): the target and the max into the head's FitHead.
__global__ __launch_bounds__(FIT_THREADS) void hardkv_fit_prep(Args a) {
  const int bh = a.bh0 + blockIdx.x;
  double H;
  float m;
  fit_target(a, bh, H, m);
  if (threadIdx.x == 0) {
    a.fith[bh].H = H;
    a.fith[bh].m = m;
  }
}

// Round r's sums over the head's slices, added in slice order (candidate k's in thread k
// < FIT_POINTS).  Every thread first copies some of the slices' sums into LDS, so that
// the loads are in flight together rather than one slice after another.
HK_DEV void fit_slice_sums(const Args &a, int bh, int r, double &Z, double &A) {
  constexpr int PER = 2 * FIT_POINTS;
  __shared__ double s_sl[FIT_MAX_SLICES * PER];
  const int tid = threadIdx.x;
  const double *ps = a.fitp + ((size_t)r * a.B * a.Hkv + bh) * a.nfs * PER;
  for (int i = tid; i < a.nfs * PER; i += FIT_THREADS) s_sl[i] = ps[i];
  __syncthreads();
  Z = A = 0.0;
  if (tid < FIT_POINTS)
    for (int sl = 0; sl < a.nfs; ++sl) {
      Z += s_sl[sl * PER + tid];
      A += s_sl[sl * PER + FIT_POINTS + tid];
    }
}

// hardkv_fit_round, grid (nfs, B*Hkv): round r's bracket from round r - 1's (its slices'
// sums, summed in slice order, so that every workgroup derives the same bracket; slice 0
// records it for round r + 1), then the slice's sums for round r's candidates.
__global__ __launch_bounds__(FIT_THREADS) void hardkv_fit_round(Args a, int r) {
  const int bh = a.bh0 + blockIdx.y, slice = blockIdx.x;
  const int tid = threadIdx.x;
  int64_t c;
  const int64_t N = fit_pool(a, bh, c);
  if (N <= 0) return;  // uniform
  FitHead *fh = a.fith + bh;
  const double H = fh->H;
  const float m = fh->m;
  double lo = -12.0, hi = 12.0;
  if (r > 0) {
    lo = fh->lo[r - 1];
    hi = fh->hi[r - 1];
    double Z, A;
    fit_slice_sums(a, bh, r - 1, Z, A);
    fit_next(Z, A, H, lo, hi);
  }
  if (slice == 0 && tid == 0) {
    fh->lo[r] = lo;
    fh->hi[r] = hi;
  }
  const int64_t r0 = (int64_t)slice * FIT_SPLIT_ROWS, r1 = min(N, r0 + (int64_t)FIT_SPLIT_ROWS);
  double Z, A;
  fit_sums(a, bh, c, r0, max(r0, r1), m, lo, hi, Z, A);
  if (tid < FIT_POINTS) {
    double *ps = a.fitp + (((size_t)r * a.B * a.Hkv + bh) * a.nfs + slice) * 2 * FIT_POINTS;
    ps[tid] = Z;
    ps[FIT_POINTS + tid] = A;
  }
}

// hardkv_fit_final, grid (B*Hkv): the last round's bracket and tau.
__global__ __launch_bounds__(FIT_THREADS) void hardkv_fit_final(Args a) {
  const int bh = a.bh0 + blockIdx.x;
  const int tid = threadIdx.x;
  int64_t c;
  const int64_t N = fit_pool(a, bh, c);
  double lo = -12.0, hi = 12.0;
  if (N > 0) {
    const FitHead *fh = a.fith + bh;
    constexpr int r = FIT_ROUNDS - 1;
    lo = fh->lo[r];
    hi = fh->hi[r];
    double Z, A;
    fit_slice_sums(a, bh, r, Z, A);
    fit_next(Z, A, fh->H, lo, hi);
  }
  fit_store(a, bh, N, lo, hi);
}

template <typename T, bool ENT, bool SHARED, bool LIVE = false>
hipError_t launch_score_ge(const Args &a, hipStream_t s) {
  dim3 grid(a.nch_score, a.nbh);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((hardkv_score<T, 1, ENT, SHARED, LIVE>), grid, dim3(NTHREADS), 0, s, a); break;
    case 2: hipLaunchKernelGGL((hardkv_score<T, 2, ENT, SHARED, LIVE>), grid, dim3(NTHREADS), 0, s, a); break;
    case 4: hipLaunchKernelGGL((hardkv_score<T, 4, ENT, SHARED, LIVE>), grid, dim3(NTHREADS), 0, s, a); break;
    case 8: hipLaunchKernelGGL((hardkv_score<T, 8, ENT, SHARED, LIVE>), grid, dim3(NTHREADS), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_score_g(const Args &a, hipStream_t s) {
  if (a.destructive)  // (the fixed temperature: no entropy pieces)
    return a.pool_shared ? launch_score_ge<T, false, true, true>(a, s) : launch_score_ge<T, false, false, true>(a, s);
  if (a.pool_shared)
    return a.calibration ? launch_score_ge<T, true, true>(a, s) : launch_score_ge<T, false, true>(a, s);
  return a.calibration ? launch_score_ge<T, true, false>(a, s) : launch_score_ge<T, false, false>(a, s);
}

}  // namespace

hipError_t launch_score(const Args &a, hipStream_t s, bool bf16) {
  return bf16 ? launch_score_g<BF16>(a, s) : launch_score_g<F32>(a, s);
}

hipError_t launch_fit(const Args &a, hipStream_t s) {
  if (a.nfs <= 1) {
    hipLaunchKernelGGL(hardkv_fit, dim3(a.nbh), dim3(FIT_THREADS), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(hardkv_fit_prep, dim3(a.nbh), dim3(FIT_THREADS), 0, s, a);
  for (int r = 0; r < FIT_ROUNDS; ++r)
    hipLaunchKernelGGL(hardkv_fit_round, dim3(a.nfs, a.nbh), dim3(FIT_THREADS), 0, s, a, r);
  hipLaunchKernelGGL(hardkv_fit_final, dim3(a.nbh), dim3(FIT_THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_flatten(const Args &a, hipStream_t s) {
  hipLaunchKernelGGL(hardkv_flatten, dim3(1), dim3(SEL_THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select(const Args &a, hipStream_t s, bool bf16) {
  // the dynamic LDS limit is an attribute of each function: raised once per process
  static std::once_flag once;
  static hipError_t configured = hipSuccess;
  std::call_once(once, [] {
    const void *fs[] = {(const void *)hardkv_select<BF16, false>, (const void *)hardkv_select<BF16, true>,
                        (const void *)hardkv_select<F32, true>, (const void *)hardkv_sel_weigh,
                        (const void *)hardkv_sel_cut, (const void *)hardkv_sel_count,
                        (const void *)hardkv_sel_finish<BF16, false>, (const void *)hardkv_sel_finish<BF16, true>,
                        (const void *)hardkv_sel_finish<F32, true>};
    for (const void *f : fs) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)sel_lds_bytes(MAX_POOL_BLOCKS));
      if (e != hipSuccess && configured == hipSuccess) configured = e;
    }
  });
  if (configured != hipSuccess) return configured;
  // (the storage type matters only to the condensation; without it one instance serves)
  auto sel = !a.fuse_cond ? hardkv_select<BF16, false> : bf16 ? hardkv_select<BF16, true> : hardkv_select<F32, true>;
  auto fin = !a.fuse_cond ? hardkv_sel_finish<BF16, false>
             : bf16       ? hardkv_sel_finish<BF16, true>
                          : hardkv_sel_finish<F32, true>;
  if (a.nsp <= 1) {
    hipLaunchKernelGGL(sel, dim3(a.nbh), dim3(SEL_THREADS), sel_lds_bytes(a.P), s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(hardkv_sel_weigh, dim3(a.nsp, a.nbh), dim3(SEL_THREADS), sizeof(SelShared), s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(hardkv_sel_cut, dim3(a.nbh), dim3(SEL_THREADS), sizeof(SelShared), s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(hardkv_sel_count, dim3(a.nsp, a.nbh), dim3(SEL_THREADS), sizeof(SelShared), s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fin, dim3(a.nbh), dim3(SEL_THREADS), sel_lds_bytes(a.P), s, a);
  return hipGetLastError();
}

}  // namespace hardkv
