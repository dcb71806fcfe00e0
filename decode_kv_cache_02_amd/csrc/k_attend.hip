// k_attend.hip -- decode attention over the three tiers, and the split-K combine.
//
// HARD-KV explainer, technical summary 2.A: the dense tier keeps the most recent tokens,
// the sparse tier the kept tokens (here rewritten into the head's view), and the
// condensed tier constant-size merged slots; each query attends to all three.
//
// hardkv_attend_tiers, grid (segments, B*Hkv), 256 threads: the standalone attention;
//   each workgroup attends one range of view rows, condensed slots or dense positions
//   and writes one partial (the fused step gets the same partials from the rewrite
//   kernel instead).
// hardkv_combine, grid (G, B*Hkv), 256 threads: one workgroup per query; it scales every
//   partial's (m, l) against the common max, lists the partials that carry weight in
//   partial order, then sums their accumulators in two streams of 128 head dims, eight
//   partials in flight per thread.
#include "attn_common.h"

namespace hardkv {

namespace {

template <typename T, int G>
__global__ __launch_bounds__(NTHREADS) void hardkv_attend_tiers(Args a) {
  __shared__ float s_part[4][G][2 + HD];
  attend_segment<T, G>(a, a.bh0 + blockIdx.y, blockIdx.x, s_part);
}

constexpr int MAX_COMBINE = 2048;  // partials per round of the combine

constexpr int COMB_UNR = 8;  // loads in flight per thread
// heads with at least this many partials are combined by 512 threads (four streams of 128
// head dims), fewer by 256 (two streams), which start and finish sooner
constexpr int COMB_WIDE_MIN = 256;

template <int G, int COMB_THREADS>
__global__ __launch_bounds__(COMB_THREADS) void hardkv_combine(Args a) {
  constexpr int COMB_WAVES = COMB_THREADS / 64;
  constexpr int COMB_STREAMS = COMB_THREADS / HD;  // partials summed in this many streams of 128 dims
  const int g = blockIdx.x, bh = a.bh0 + blockIdx.y;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float s_f[MAX_COMBINE];
  __shared__ int s_slot[MAX_COMBINE];
  __shared__ float s_red[COMB_WAVES];
  __shared__ int s_cnt[COMB_WAVES];
  __shared__ float s_acc[COMB_STREAMS][HD];
  const float *base = a.part + (size_t)bh * a.npart * G * (2 + HD) + (size_t)g * (2 + HD);
  const size_t stride = (size_t)G * (2 + HD);  // from one partial slot to the next
  const int ncd = a.nc_att + a.nd_att + a.ns_att + a.ntp;
  const int ns = a.nvp + ncd + a.nxp;
  // partials: view or rewrite chunks at [0, nvp), condensed, dense, sink and (without a
  // selection this step) pool-tail segments at part_cd_base, gathered-row chunks of the
  // standalone attention at xp_base
  auto slot = [&](int i) {
    return i < a.nvp ? i : (i < a.nvp + ncd ? a.part_cd_base + (i - a.nvp) : a.xp_base + (i - a.nvp - ncd));
  };

  // the common maximum of the partials that saw any row
  float M = -INFINITY;
  for (int i = tid; i < ns; i += COMB_THREADS) {
    const float *ps = base + (size_t)slot(i) * stride;
    if (ps[1] > 0.0f) M = fmaxf(M, ps[0]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) s_red[wave] = M;
  __syncthreads();
  M = s_red[0];
#pragma unroll
  for (int w = 1; w < COMB_WAVES; ++w) M = fmaxf(M, s_red[w]);
  __syncthreads();

  // per round: the scale factors 2^(m - M) of the partials that carry weight, listed in
  // partial order, and the scaled sum of l; then the scaled sum of their accumulators in
  // COMB_STREAMS streams of 128 head dims, COMB_UNR partials in flight per stream
  const int d = tid & (HD - 1), strm = tid >> 7;
  float L = 0.0f, A = 0.0f;
  for (int r0 = 0; r0 < ns; r0 += MAX_COMBINE) {
    const int r1 = min(ns, r0 + MAX_COMBINE);
    float Lp = 0.0f;
    int nnz = 0;
    for (int ib = r0; ib < r1; ib += COMB_THREADS) {
      const int i = ib + tid;
      float f = 0.0f;
      if (i < r1) {
        const float *ps = base + (size_t)slot(i) * stride;
        f = ps[1] > 0.0f ? exp2_fast(ps[0] - M) : 0.0f;
        Lp += ps[1] * f;
      }
      const uint64_t bal = ballot(f > 0.0f);
      if (lane == 0) s_cnt[wave] = __popcll(bal);
      __syncthreads();
      int before = nnz, all = 0;
#pragma unroll
      for (int w = 0; w < COMB_WAVES; ++w) {
        before += w < wave ? s_cnt[w] : 0;
        all += s_cnt[w];
      }
      if (f > 0.0f) {
        const int pos = before + (int)popc_below(bal);
        s_slot[pos] = slot(i);
        s_f[pos] = f;
      }
      nnz += all;
      __syncthreads();
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) Lp += __shfl_xor(Lp, off);
    if (lane == 0) s_red[wave] = Lp;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < COMB_WAVES; ++w) L += s_red[w];
    int k = strm;
    for (; k + (COMB_UNR - 1) * COMB_STREAMS < nnz; k += COMB_UNR * COMB_STREAMS) {
      float x[COMB_UNR];
#pragma unroll
      for (int u = 0; u < COMB_UNR; ++u) x[u] = base[(size_t)s_slot[k + COMB_STREAMS * u] * stride + 2 + d];
#pragma unroll
      for (int u = 0; u < COMB_UNR; ++u) A = __builtin_fmaf(x[u], s_f[k + COMB_STREAMS * u], A);
    }
    for (; k < nnz; k += COMB_STREAMS) A = __builtin_fmaf(base[(size_t)s_slot[k] * stride + 2 + d], s_f[k], A);
    __syncthreads();
  }
  s_acc[strm][d] = A;
  __syncthreads();
  if (strm == 0) {
    float sum = s_acc[0][d];
#pragma unroll
    for (int q = 1; q < COMB_STREAMS; ++q) sum += s_acc[q][d];
    a.out[((size_t)b * a.Hq + (size_t)h * G + g) * HD + d] = sum / L;
  }
}

template <typename T>
hipError_t launch_tiers(const Args &a, hipStream_t s) {
  dim3 grid(a.nv_att + a.nc_att + a.nd_att + a.ns_att + a.ntp, a.nbh);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((hardkv_attend_tiers<T, 1>), grid, dim3(NTHREADS), 0, s, a); break;
    case 2: hipLaunchKernelGGL((hardkv_attend_tiers<T, 2>), grid, dim3(NTHREADS), 0, s, a); break;
    case 4: hipLaunchKernelGGL((hardkv_attend_tiers<T, 4>), grid, dim3(NTHREADS), 0, s, a); break;
    case 8: hipLaunchKernelGGL((hardkv_attend_tiers<T, 8>), grid, dim3(NTHREADS), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend(const Args &a, hipStream_t s, bool bf16) {
  return bf16 ? launch_tiers<BF16>(a, s) : launch_tiers<F32>(a, s);
}

template <int CT>
hipError_t launch_combine_t(const Args &a, hipStream_t s) {
  dim3 grid(a.G, a.nbh);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((hardkv_combine<1, CT>), grid, dim3(CT), 0, s, a); break;
    case 2: hipLaunchKernelGGL((hardkv_combine<2, CT>), grid, dim3(CT), 0, s, a); break;
    case 4: hipLaunchKernelGGL((hardkv_combine<4, CT>), grid, dim3(CT), 0, s, a); break;
    case 8: hipLaunchKernelGGL((hardkv_combine<8, CT>), grid, dim3(CT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const Args &a, hipStream_t s) {
  const int ns = a.nvp + a.nc_att + a.nd_att + a.ns_att + a.ntp + a.nxp;  // partials per head
  return ns >= COMB_WIDE_MIN ? launch_combine_t<512>(a, s) : launch_combine_t<256>(a, s);
}

}  // namespace hardkv
