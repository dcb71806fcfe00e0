// k_rewrite.hip -- stage 3 of the decode step: Index Regularization by Rewrite Cache.
//
// HARD-KV explainer, technical summary 2.C: the tokens the top-p mask keeps are moved
// into contiguous ranges, each head owning a fixed-capacity view (the max-length form
// of Flatten Index), so that attention reads static, contiguous, fixed-stride blocks.
//
// Grid (chunks [+ attention segments], B*Hkv), 256 threads.  A chunk is four survivor
// blocks, one per wavefront (sixteen, four per wavefront, for a head that keeps at most a
// quarter of its survivors).  From the block's weights and the head's cut (w_th, r,
// and the block's ties-before count from the select stage) each lane decides whether its
// row is kept: w > w_th, or w == w_th and its tie rank (ties before the block plus the
// mbcnt of equal weights below it) is under r.  The ballot of those bits is the block's
// mask word.  A kept row's view row is the block's first view row plus the row's rank
// inside the word, so the order of positions is preserved.  Kept rows are copied as
// 16-byte pieces, 16 lanes per row, 16 rows per batch; with buffer accesses whose
// out-of-range offsets the hardware drops, no branch surrounds a load or store.  A
// wavefront with more than two batches of 16-bit rows pipelines keys and values half a
// batch apart, so that its stores drain while the next batch's loads are in flight.
//
// In the fused step the kernel also runs the attention of the group's queries over the
// rows it copies (one split-K partial per workgroup, so the view is never read back),
// and extra workgroups attend the condensed slots and the dense window.
#include "attn_common.h"

namespace hardkv {

namespace {

// Lists of at most this many kept rows per wavefront are copied batch by batch; longer
// ones through the pipeline below (which pays a prologue of its own).
constexpr int PIPE_MIN_ROWS = 32;

// STORE: whether the launch can write views at all (not under SPARSE, nor for the
// attention-only gathers): without it the kernel keeps no registers for stores.
// SHARED: the shared block pool (kept rows anywhere in it, loaded through flat addresses of
// their physical rows), else the unit's own ring (one buffer resource).
template <typename T, int G, bool MASK, bool COPY, bool ATTN, bool STORE, bool SHARED>
__global__ __launch_bounds__(NTHREADS) void hardkv_rewrite(Args a) {
  constexpr int EB = Elem<T>::bytes;
  constexpr size_t ROWB = (size_t)HD * EB;
  const int bh = a.bh0 + blockIdx.y, chunk = blockIdx.x;
  __shared__ uint32_t s_src[4][4 * BK];  // per wavefront: kept rows (pool ring row of the head)
  __shared__ uint32_t s_dst[4][4 * BK];  // and their view rows
  __shared__ float s_part[ATTN ? 4 : 1][G][2 + HD];
  if (ATTN && chunk >= a.nch_reg) {  // condensed / dense attention segments (fused step)
    attend_segment<T, G>(a, bh, a.nv_att + (chunk - a.nch_reg), s_part);
    return;
  }
  // partial slot of this chunk's gathered rows
  const int pslot = a.gather_mode == GATHER_STEP ? chunk : a.xp_base + chunk;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane & 15, grp = lane >> 4;
  const int P = a.P, V = a.V_cap;

  const HeadInfo *hd = a.head + bh;
  // store the gathered rows into the view only when the head is rewritten this step; in
  // the standalone attention of a mixed policy, rewritten heads are attended from their
  // views by the tier kernel instead
  const bool store = STORE && COPY && (a.gather_mode == GATHER_STEP || a.gather_mode == GATHER_REWRITE) && hd->rw;
  const bool skip = a.gather_mode == GATHER_ATTEND_NRW && hd->rw;
  const int64_t t = hd->t_plan, c = hd->c_plan;
  const uint32_t w_th = hd->w_th, r = hd->r;
  const int nx = hd->E;
  const int64_t pend = pool_end(t, a.W, a.S);
  const int nblk = (int)((pend + BK - 1) / BK - c / BK);
  const int pb_lo = (int)((c / BK) % P);
  // Chunks cover the survivor blocks [nx, nblk) (pool-relative block indices; the select
  // kernel has cleared every mask word).  Blocks per wavefront: one when the head keeps
  // more than a quarter of its survivors, else four (a chunk then spans 4 * cb_reg blocks
  // and the chunks past the survivors are empty), so that sparse selections fill the
  // 16-row copy batches of fewer workgroups.
  const int nub = max(0, nblk - nx);
  const int bpw = ((int64_t)hd->kstar * 4 <= (int64_t)nub * BK) ? 4 : 1;
  const int i0 = nx + chunk * a.cb_reg * bpw, i1 = min(i0 + a.cb_reg * bpw, nblk);
  auto ring = [&](int i) { return pb_lo + i >= P ? pb_lo + i - P : pb_lo + i; };

  // A chunk that keeps no row (past the survivors, or no kept token: the first view rows
  // of its first block and of the block after it are equal) leaves an empty partial.
  {
    bool empty = i0 >= i1 || skip || (!ATTN && !MASK && !store);
    if (!empty) {
      const uint32_t x0 = a.blkinfo[(size_t)bh * P + ring(i0)].x;
      const uint32_t x1 = i1 < nblk ? a.blkinfo[(size_t)bh * P + ring(i1)].x : (uint32_t)hd->kstar;
      empty = x1 == x0;
    }
    if (empty) {
      if (ATTN && tid < G) {
        float *o = a.part + ((size_t)bh * a.npart + pslot) * G * (2 + HD) + (size_t)tid * (2 + HD);
        o[0] = -INFINITY;
        o[1] = 0.0f;
      }
      return;
    }
  }

  AttnState<G> st;
  float qs[G][8];
  if (ATTN) {
    st.init();
    load_q_scaled<T, G>(a, b, h, sub, qs);
  }
  const size_t rowbase = (size_t)bh * P * BK;
  const uint64_t poolb = (uint64_t)P * BK * ROWB;
  const BufRes pk = make_buf((const char *)a.pool_k + (SHARED ? 0 : rowbase * ROWB), poolb);
  const BufRes pv = make_buf((const char *)a.pool_v + (SHARED ? 0 : rowbase * ROWB), poolb);
  // the head's view rows start at voff (bh * V_cap, or its packed offset); vcap rows fit,
  // and the view buffers end there, so a row past them is not written
  const int64_t voff = hd->voff;
  const uint32_t vcap = a.view_sum ? (uint32_t)max((int64_t)0, min(a.view_rows - voff, (int64_t)UINT32_MAX))
                                   : (uint32_t)V;
  const BufRes vk = make_buf((const char *)a.view_k + (size_t)voff * ROWB, (uint64_t)vcap * ROWB);
  const BufRes vv = make_buf((const char *)a.view_v + (size_t)voff * ROWB, (uint64_t)vcap * ROWB);
  const uint32_t lane_b = (uint32_t)(sub * 8 * EB);  // the lane's 8 elements of a row
  int32_t *vpos = a.view_pos + voff;

  // the wavefront's blocks: weights and block info of all of them in flight at once
  const int iw = i0 + wave * bpw;
  uint32_t wv[4];
  uint2 bi[4];
  int32_t ph[4];  // physical blocks (shared pool)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = iw + j;
    const bool live = j < bpw && i < i1;
    const int64_t p = c + (int64_t)i * BK + lane;
    wv[j] = (live && p < pend) ? a.weights[rowbase + (size_t)ring(i) * BK + lane] : 0u;
    bi[j] = live ? a.blkinfo[(size_t)bh * P + ring(i)] : make_uint2(0u, 0u);
    ph[j] = (SHARED && live) ? a.btab[(size_t)bh * P + ring(i)] : 0;
  }
  // mask words, and the list of kept rows in position order
  int ns = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = iw + j;
    if (j >= bpw || i >= i1) break;  // wave-uniform
    const int pb = ring(i);
    const int64_t p = c + (int64_t)i * BK + lane;
    const bool valid = p < pend;
    const uint32_t w = wv[j];
    const uint64_t eqm = ballot(valid && w == w_th);
    const bool sel = valid && (w > w_th || (w == w_th && bi[j].y + popc_below(eqm) < r));
    const uint64_t mw = ballot(sel);
    if (MASK && lane == 0) a.mask[(size_t)bh * P + pb] = mw;
    if (!COPY || mw == 0) continue;  // wave-uniform
    const uint32_t vo = bi[j].x, idx = popc_below(mw);
    if (sel) {
      s_src[wave][ns + idx] = SHARED ? (uint32_t)(max(ph[j], 0) * BK + lane) : (uint32_t)(pb * BK + lane);
      s_dst[wave][ns + idx] = vo + idx;
      if (store && vo + idx < vcap) vpos[vo + idx] = (int32_t)p;
    }
    ns += __popcll(mw);
  }
  // a launch that only rewrites (no attention) copies nothing for a head it does not rewrite
  if (COPY && (ATTN || store)) {
    wave_sync();
    // Kept rows move 16 at a time (4 per 16-lane group) and are attended while in
    // registers.  Keys and values are pipelined half a batch apart: the next batch's key
    // loads go out as soon as this batch's keys are stored, before its values are waited
    // for, so a wait for loads never waits for the stores just issued (the counter of
    // loads and stores completes in order).  Rows past the list read zeros and write
    // nothing (offset BUF_SKIP), and so does every store when the view is not written;
    // rows past the view's capacity are attended but fall outside the view buffers.
    // source offsets: bytes into the unit's ring (BUF_SKIP for rows past the list), or, in
    // the shared pool, physical rows, whose 64-bit address is formed at the load (rows past
    // the list read a listed row, which nothing uses)
    using SOff = uint32_t;
    SOff so[4];
    uint32_t dof[4];
    bool ac[4];
    auto offsets = [&](int it, SOff (&o_s)[4], uint32_t (&o_d)[4], bool (&o_a)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = it + j * 4 + grp;
        const int kk = k < ns ? k : 0;
        o_a[j] = k < ns;
        // read in every lane (kk is in the list), so that no branch surrounds the
        // memory accesses that follow
        uint32_t sv = s_src[wave][kk], dv = s_dst[wave][kk];
        asm volatile("" : "+v"(sv), "+v"(dv));
        if constexpr (SHARED)
          o_s[j] = sv;
        else
          o_s[j] = o_a[j] ? sv * (uint32_t)ROWB + lane_b : BUF_SKIP;
        o_d[j] = (o_a[j] && store) ? dv * (uint32_t)ROWB + lane_b : BUF_SKIP;
      }
    };
    auto ldk = [&](SOff o, Raw8<T> &r) {
      if constexpr (SHARED) {
        size_t off = (size_t)o * ROWB + lane_b;
        asm volatile("" : "+v"(off));  // formed here, not held from earlier
        raw_load_nt((const char *)a.pool_k + off, r);
      } else {
        buf_load_nt(pk, o, r);
      }
    };
    auto ldv = [&](SOff o, Raw8<T> &r) {
      if constexpr (SHARED) {
        size_t off = (size_t)o * ROWB + lane_b;
        asm volatile("" : "+v"(off));
        raw_load_nt((const char *)a.pool_v + off, r);
      } else {
        buf_load_nt(pv, o, r);
      }
    };
    Raw8<T> kr[4], vr[4];
    // The pipeline holds the next batch's keys beside this batch's probabilities: with
    // fp32 rows or 8 queries per group that costs a wave per SIMD, so only 16-bit rows
    // with up to 4 queries take it.
    constexpr bool PIPE = STORE && Elem<T>::bytes == 2 && G <= 4;
    if (!PIPE || ns <= PIPE_MIN_ROWS) {
      // a short list: batch by batch, each store waiting only for its own load
      for (int it = 0; it < ns; it += 16) {
        offsets(it, so, dof, ac);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ldk(so[j], kr[j]);
          ldv(so[j], vr[j]);
        }
        if constexpr (STORE) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            buf_store_nt(vk, dof[j], kr[j]);
            buf_store_nt(vv, dof[j], vr[j]);
          }
        }
        if (ATTN) attn_rows<T, G, 4>(st, qs, kr, vr, ac);
      }
    } else if constexpr (PIPE) {
      // (scheduling barriers keep the phases in this order: the waits depend on the order
      // in which the loads and stores were issued)
      offsets(0, so, dof, ac);
#pragma unroll
      for (int j = 0; j < 4; ++j) ldk(so[j], kr[j]);
      __builtin_amdgcn_sched_barrier(0);
      {
        // stores that write nothing, so that the first batch's loads are followed by as
        // many accesses as every later batch's: the waits in the loop count the same way
        const Raw8<T> zero{};
#pragma unroll
        for (int j = 0; j < 4; ++j) buf_store_nt(vv, BUF_SKIP + 64u * j, zero);  // distinct, not merged
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) ldv(so[j], vr[j]);
      __builtin_amdgcn_sched_barrier(0);
      // every batch but the last loads its successor; the last only stores and attends
      int it = 0;
      for (; it + 16 < ns; it += 16) {
        float p[G][4];
        if (ATTN) attn_keys<T, G, 4>(st, qs, kr, ac, p);
#pragma unroll
        for (int j = 0; j < 4; ++j) buf_store_nt(vk, dof[j], kr[j]);
        __builtin_amdgcn_sched_barrier(0);
        {
          SOff so2[4];
          uint32_t dof2[4];
          bool ac2[4];
          offsets(it + 16, so2, dof2, ac2);
#pragma unroll
          for (int j = 0; j < 4; ++j) ldk(so2[j], kr[j]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (ATTN) attn_values<T, G, 4>(st, p, vr);
#pragma unroll
        for (int j = 0; j < 4; ++j) buf_store_nt(vv, dof[j], vr[j]);
        __builtin_amdgcn_sched_barrier(0);
        offsets(it + 16, so, dof, ac);  // read again rather than held through the values
#pragma unroll
        for (int j = 0; j < 4; ++j) ldv(so[j], vr[j]);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) buf_store_nt(vk, dof[j], kr[j]);
#pragma unroll
      for (int j = 0; j < 4; ++j) buf_store_nt(vv, dof[j], vr[j]);
      if (ATTN) attn_rows<T, G, 4>(st, qs, kr, vr, ac);
    }
  }
  if (ATTN) attn_write_partial<G>(st, a.part + ((size_t)bh * a.npart + pslot) * G * (2 + HD), s_part);
}

template <typename T, bool MASK, bool COPY, bool ATTN, bool STORE, bool SHARED>
hipError_t launch_gs(const Args &a, hipStream_t s) {
  dim3 grid(a.nch_reg + (ATTN && a.gather_mode == GATHER_STEP ? a.nc_att + a.nd_att + a.ns_att : 0), a.nbh);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((hardkv_rewrite<T, 1, MASK, COPY, ATTN, STORE, SHARED>), grid, dim3(NTHREADS), 0, s, a); break;
    case 2: hipLaunchKernelGGL((hardkv_rewrite<T, 2, MASK, COPY, ATTN, STORE, SHARED>), grid, dim3(NTHREADS), 0, s, a); break;
    case 4: hipLaunchKernelGGL((hardkv_rewrite<T, 4, MASK, COPY, ATTN, STORE, SHARED>), grid, dim3(NTHREADS), 0, s, a); break;
    case 8: hipLaunchKernelGGL((hardkv_rewrite<T, 8, MASK, COPY, ATTN, STORE, SHARED>), grid, dim3(NTHREADS), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, bool MASK, bool COPY, bool ATTN, bool STORE>
hipError_t launch_g(const Args &a, hipStream_t s) {
  return a.pool_shared ? launch_gs<T, MASK, COPY, ATTN, STORE, true>(a, s)
                       : launch_gs<T, MASK, COPY, ATTN, STORE, false>(a, s);
}

template <typename T>
hipError_t launch_t(const Args &a, hipStream_t s, bool mask, bool copy, bool attend) {
  // the fused step writes views unless every head only gathers (SPARSE); the attention
  // gathers never write them
  if (mask && copy && attend)
    return a.reg_launch == HARDKV_REG_SPARSE ? launch_g<T, true, true, true, false>(a, s)
                                             : launch_g<T, true, true, true, true>(a, s);
  if (mask && !copy && !attend) return launch_g<T, true, false, false, false>(a, s);
  if (mask && copy && !attend) return launch_g<T, true, true, false, true>(a, s);
  if (!mask && copy && !attend) return launch_g<T, false, true, false, true>(a, s);
  if (!mask && copy && attend) return launch_g<T, false, true, true, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_rewrite(const Args &a, hipStream_t s, bool bf16, bool mask, bool copy, bool attend) {
  return bf16 ? launch_t<BF16>(a, s, mask, copy, attend) : launch_t<F32>(a, s, mask, copy, attend);
}

}  // namespace hardkv
