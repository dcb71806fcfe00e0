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
#include "condense_common.h"

namespace hardkv {

namespace {

template <typename T>
__global__ __launch_bounds__(NTHREADS) void hardkv_condense(Args a) {
  const int bh = a.bh0 + blockIdx.y;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);  // slot offset from the cursor
  const HeadInfo *hd = a.head + bh;
  const int64_t c = hd->c_plan;
  const int64_t E = hd->E;
  const int32_t nu = hd->nu_plan;
  if (a.mode == HARDKV_COND_MERGE && i < E && i < a.C)  // chain heads: blocks 0 .. min(E, C) - 1
    condense_chain<T, Elem<T>::bytes == 2 ? 8 : 4>(a, bh, i, c, E, nu, hd->w_all);
  if (i == 0) condense_advance(a, bh, c, E, nu);  // (the whole wavefront of slot 0)
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
