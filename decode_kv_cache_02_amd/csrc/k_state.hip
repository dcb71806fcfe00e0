// k_state.hip -- placing a context into the cascade cache, and stage 1 of the decode
// step: linear append to the dense tier.
//
// HARD-KV explainer, technical summary 2.A: the dense tier buffers the most recent
// tokens in contiguous memory; tokens that age out of the dense window move to the
// sparse tier.  The dense tier is a ring of W slots (position p in slot p mod W), the
// sparse tier a ring of P blocks of 64 rows (position p in block (p / 64) mod P).  With
// a sink prefix of S tokens, positions below S go to the sink rows (row p) instead and
// the dense window holds [max(S, t - W), t).
#include "hardkv_internal.h"

namespace hardkv {

namespace {

// grid (ceil(B*Hkv / 256)): clears each head's flag of keys outside the range where the
// score's products are exact; the placement below and every append set it again.
__global__ __launch_bounds__(NTHREADS) void hardkv_prefill_clear(Args a) {
  const int i = blockIdx.x * NTHREADS + threadIdx.x;
  if (i < a.B * a.Hkv) a.kx[i] = 0u;
}

// grid 1 (the shared pool only): every unit gets, in unit order, the physical blocks its pool
// [S, max(S, L_b - W)) holds, ring block S / 64 + i -> physical block base_u + i; the table's
// other entries are -1 and the blocks left over form the free list.  A unit whose blocks do
// not fit gets none past the end (its rows are not placed) and the overflow bit is set.
__global__ __launch_bounds__(NTHREADS) void hardkv_prefill_alloc(Args a) {
  __shared__ int64_t s_need[NTHREADS];
  __shared__ int64_t s_carry;
  const int tid = threadIdx.x, BH = a.B * a.Hkv, P = a.P;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int u0 = 0; u0 < BH; u0 += NTHREADS) {
    const int u = u0 + tid;
    int64_t need = 0;
    if (u < BH) {
      const int64_t L = a.ctx_len[u / a.Hkv];
      const int64_t pend = pool_end(L, a.W, a.S);
      need = pend > a.S ? (pend + BK - 1) / BK - a.S / BK : 0;
    }
    s_need[tid] = need;
    __syncthreads();
    // exclusive scan of the chunk (a plain serial pass by one thread: setup, not the step)
    if (tid == 0) {
      int64_t run = s_carry;
      for (int k = 0; k < NTHREADS; ++k) {
        const int64_t n = s_need[k];
        s_need[k] = run;
        run += n;
      }
      s_carry = run;
    }
    __syncthreads();
    for (int k = 0; k < NTHREADS && u0 + k < BH; ++k) {
      const int uk = u0 + k;
      const int64_t base = s_need[k];
      const int64_t L = a.ctx_len[uk / a.Hkv];
      const int64_t pend = pool_end(L, a.W, a.S);
      const int64_t n = pend > a.S ? (pend + BK - 1) / BK - a.S / BK : 0;
      for (int i = tid; i < P; i += NTHREADS) a.btab[(size_t)uk * P + i] = -1;
      __syncthreads();
      for (int64_t i = tid; i < n; i += NTHREADS) {
        const int64_t phys = base + i;
        a.btab[(size_t)uk * P + (size_t)((a.S / BK + i) % P)] = phys < a.NB ? (int32_t)phys : -1;
      }
      __syncthreads();
    }
  }
  const int64_t used = s_carry;
  if (used > a.NB && tid == 0) atomicOr(a.error_word, HARDKV_ERR_POOL_OVERFLOW);
  const int64_t nfree = used < a.NB ? a.NB - used : 0;
  for (int64_t k = tid; k < nfree; k += NTHREADS) a.free_list[k] = (int32_t)(used + k);
  if (tid == 0) *a.free_top = (int32_t)nfree;
}

// grid (ceil(max_len / 64) + 1, B*Hkv): blocks of 64 context positions, then one
// workgroup per head that resets the head's counters and condensed tier.
template <typename T>
__global__ __launch_bounds__(NTHREADS) void hardkv_prefill(Args a) {
  constexpr int EB = Elem<T>::bytes;
  constexpr int CPR = HD * EB / 16;  // 16-byte pieces per row
  const int bh = blockIdx.y, x = blockIdx.x;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int tid = threadIdx.x;
  const int64_t L = a.ctx_len[b];
  const int W = a.W, P = a.P;
  const size_t ROWB = (size_t)HD * EB;

  const int64_t dense_lo = dense_lo_of(L, W, a.S);
  if (x == (int)gridDim.x - 1) {
    if (tid == 0) {
      a.pool_head[bh] = a.S;
      a.cond_cursor[bh] = 0;
      if (h == 0) a.seq_len[b] = L;
      // no selection yet: an empty plan whose pool ends at the pool head, so that a step
      // without selection attends the whole pool as positions since the last selection
      HeadInfo z = {};
      z.c_plan = a.S;
      a.head[bh] = z;
    }
    for (int k = tid; k < a.C * HD; k += NTHREADS) {
      a.cond_kn[(size_t)bh * a.C * HD + k] = 0.0f;
      a.cond_vn[(size_t)bh * a.C * HD + k] = 0.0f;
    }
    for (int k = tid; k < a.C; k += NTHREADS) {
      a.cond_omega[(size_t)bh * a.C + k] = 0.0f;
      a.cond_n[(size_t)bh * a.C + k] = 0;
    }
    // dense slots that hold no position of [dense_lo, L), and sink rows past L
    for (int64_t k = tid; k < (int64_t)W * CPR; k += NTHREADS) {
      const int64_t slot = k / CPR, piece = k % CPR;
      if (((slot - dense_lo % W) + W) % W >= L - dense_lo) {
        const size_t off = ((size_t)bh * W + slot) * ROWB + piece * 16;
        *reinterpret_cast<uint4 *>((char *)a.dense_k + off) = uint4{0, 0, 0, 0};
        *reinterpret_cast<uint4 *>((char *)a.dense_v + off) = uint4{0, 0, 0, 0};
      }
    }
    for (int64_t k = tid; k < (int64_t)a.S * CPR; k += NTHREADS) {
      const int64_t row = k / CPR, piece = k % CPR;
      if (row >= L) {
        const size_t off = ((size_t)bh * a.S + row) * ROWB + piece * 16;
        *reinterpret_cast<uint4 *>((char *)a.sink_k + off) = uint4{0, 0, 0, 0};
        *reinterpret_cast<uint4 *>((char *)a.sink_v + off) = uint4{0, 0, 0, 0};
      }
    }
    return;
  }
  for (int k = tid; k < BK * CPR; k += NTHREADS) {
    const int64_t p = (int64_t)x * BK + k / CPR;
    const int piece = k % CPR;
    if (p >= L) continue;
    const size_t src = ((size_t)bh * a.max_len + p) * ROWB + piece * 16;
    size_t dst;
    void *dk, *dv;
    if (p < a.S) {
      dst = ((size_t)bh * a.S + (size_t)p) * ROWB + piece * 16;
      dk = a.sink_k;
      dv = a.sink_v;
    } else if (p >= dense_lo) {
      dst = ((size_t)bh * W + (size_t)(p % W)) * ROWB + piece * 16;
      dk = a.dense_k;
      dv = a.dense_v;
    } else {
      const int pb = (int)((p / BK) % P);
      if (a.pool_shared && a.btab[(size_t)bh * P + pb] < 0) continue;  // no block (pool overflow)
      dst = (pool_row0(a, bh, pb) + (size_t)(p % BK)) * ROWB + piece * 16;
      dk = a.pool_k;
      dv = a.pool_v;
    }
    const uint4 kp = *reinterpret_cast<const uint4 *>((const char *)a.k_ctx + src);
    *reinterpret_cast<uint4 *>((char *)dk + dst) = kp;
    *reinterpret_cast<uint4 *>((char *)dv + dst) = *reinterpret_cast<const uint4 *>((const char *)a.v_ctx + src);
    if (EB == 2 && dk == a.pool_k && key_piece_unsafe(kp)) atomicOr(&a.kx[bh], 1u);
  }
}

// grid B: one workgroup per sequence moves, for each KV head, position t - W from the
// dense ring to the pool tail (when it is past the sink prefix), writes the new token
// into its dense slot (the same slot) or, below S, into its sink row, and then advances t.
template <typename T>
__global__ __launch_bounds__(NTHREADS) void hardkv_append(Args a) {
  constexpr int EB = Elem<T>::bytes;
  constexpr int CPR = HD * EB / 16;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int W = a.W, P = a.P, H = a.Hkv;
  const size_t ROWB = (size_t)HD * EB;
  const int64_t t = a.seq_len[b];
  const int64_t p = t - W;          // leaves the window when it is past the sinks
  const bool moves = p >= a.S;      // (and then t >= W)
  const bool sink = t < a.S;        // the new token is a sink position
  const int pb = (int)((p / BK) % P);
  if (a.pool_shared && moves && p % BK == 0) {
    // the position starts a new block: each head takes one from the free list (unless its
    // ring is full: the block then stays mapped and is overwritten, as in the ring layout)
    if (tid < H && p + 1 - a.pool_head[(size_t)b * H + tid] <= (int64_t)P * BK) {
      const size_t bh = (size_t)b * H + tid;
      const int32_t idx = atomicSub(a.free_top, 1) - 1;
      int32_t phys = -1;
      if (idx >= 0 && idx < a.NB) {
        phys = a.free_list[idx];
      } else {
        atomicAdd(a.free_top, 1);
        atomicOr(a.error_word, HARDKV_ERR_POOL_OVERFLOW);
      }
      a.btab[bh * P + pb] = phys;
    }
    __syncthreads();
  }
  for (int k = tid; k < H * 2 * CPR; k += NTHREADS) {
    const int h = k / (2 * CPR), rem = k % (2 * CPR);
    const int which = rem / CPR, piece = rem % CPR;
    const size_t bh = (size_t)b * H + h;
    const char *src = (const char *)(which ? a.v_new : a.k_new) + bh * ROWB + piece * 16;
    if (sink) {
      char *srow = (char *)(which ? a.sink_v : a.sink_k) + (bh * a.S + (size_t)t) * ROWB + piece * 16;
      *reinterpret_cast<uint4 *>(srow) = *reinterpret_cast<const uint4 *>(src);
      continue;
    }
    char *dense = (char *)(which ? a.dense_v : a.dense_k) + (bh * W + (size_t)(t % W)) * ROWB + piece * 16;
    if (moves && !(a.pool_shared && a.btab[bh * P + pb] < 0)) {
      char *pool = (char *)(which ? a.pool_v : a.pool_k) + (pool_row0(a, (int)bh, pb) + (size_t)(p % BK)) * ROWB +
                   piece * 16;
      const uint4 x = *reinterpret_cast<const uint4 *>(dense);
      *reinterpret_cast<uint4 *>(pool) = x;
      if (EB == 2 && !which && key_piece_unsafe(x)) atomicOr(&a.kx[bh], 1u);
    }
    *reinterpret_cast<uint4 *>(dense) = *reinterpret_cast<const uint4 *>(src);
  }
  if (tid < H && moves) {
    const int64_t c = a.pool_head[(size_t)b * H + tid];
    if (p + 1 - c > (int64_t)P * BK) atomicOr(a.error_word, HARDKV_ERR_POOL_OVERFLOW);
  }
  __syncthreads();
  if (tid == 0) a.seq_len[b] = t + 1;
}

// grid (ceil(B*Hkv / 256)): the snapshot of t for a selection made ahead, and the key
// flags of the state it forks from (kept through that state's appends so far).
__global__ __launch_bounds__(NTHREADS) void hardkv_fork(Args a) {
  const int i = blockIdx.x * NTHREADS + threadIdx.x;
  if (i < a.B) a.tsnap[i] = a.seq_len[i];
  if (i < a.B * a.Hkv) a.kx[i] = a.kx_src[i];
}

}  // namespace

hipError_t launch_fork(const Args &a, hipStream_t s) {
  hipLaunchKernelGGL(hardkv_fork, dim3((a.B * a.Hkv + NTHREADS - 1) / NTHREADS), dim3(NTHREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill(const Args &a, hipStream_t s, bool bf16) {
  hipLaunchKernelGGL(hardkv_prefill_clear, dim3((a.B * a.Hkv + NTHREADS - 1) / NTHREADS), dim3(NTHREADS), 0, s, a);
  if (a.pool_shared) hipLaunchKernelGGL(hardkv_prefill_alloc, dim3(1), dim3(NTHREADS), 0, s, a);
  dim3 grid((unsigned)((a.max_len + BK - 1) / BK) + 1, a.B * a.Hkv);
  if (bf16)
    hipLaunchKernelGGL((hardkv_prefill<BF16>), grid, dim3(NTHREADS), 0, s, a);
  else
    hipLaunchKernelGGL((hardkv_prefill<F32>), grid, dim3(NTHREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append(const Args &a, hipStream_t s, bool bf16) {
  dim3 grid(a.B);
  if (bf16)
    hipLaunchKernelGGL((hardkv_append<BF16>), grid, dim3(NTHREADS), 0, s, a);
  else
    hipLaunchKernelGGL((hardkv_append<F32>), grid, dim3(NTHREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace hardkv
