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
// hardkv_combine, grid (B*Hkv), 256 threads: one wavefront per query of the group; the
//   lanes first scale every partial's (m, l) against the common max, then sum the
//   partials' accumulators two head dims per lane, eight partials in flight.
#include "attn_common.h"

namespace hardkv {

namespace {

template <typename T, int G>
__global__ __launch_bounds__(NTHREADS) void hardkv_attend_tiers(Args a) {
  __shared__ float s_part[4][G][2 + HD];
  attend_segment<T, G>(a, blockIdx.y, blockIdx.x, s_part);
}

constexpr int MAX_COMBINE = 2048;  // partials per round of the combine

template <int G>
__global__ __launch_bounds__(NTHREADS) void hardkv_combine(Args a) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float s_f[4][MAX_COMBINE];
  const float *base = a.part + (size_t)bh * a.npart * G * (2 + HD);
  const int ns = a.nvp + a.nc_att + a.nd_att;
  auto slot = [&](int i) { return i < a.nvp ? i : a.part_cd_base + (i - a.nvp); };
  for (int g = wave; g < G; g += 4) {
    float M = -INFINITY;
    for (int i = lane; i < ns; i += 64) {
      const float *ps = base + ((size_t)slot(i) * G + g) * (2 + HD);
      if (ps[1] > 0.0f) M = fmaxf(M, ps[0]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float L = 0.0f, A0 = 0.0f, A1 = 0.0f;
    for (int r0 = 0; r0 < ns; r0 += MAX_COMBINE) {
      const int r1 = min(ns, r0 + MAX_COMBINE);
      float Lp = 0.0f;
      for (int i = r0 + lane; i < r1; i += 64) {
        const float *ps = base + ((size_t)slot(i) * G + g) * (2 + HD);
        const float f = ps[1] > 0.0f ? exp2_fast(ps[0] - M) : 0.0f;
        s_f[wave][i - r0] = f;
        Lp += ps[1] * f;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) Lp += __shfl_xor(Lp, off);
      L += Lp;
      wave_sync();
      int i = r0;
      for (; i + 8 <= r1; i += 8) {
        float x0[8], x1[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float *ps = base + ((size_t)slot(i + u) * G + g) * (2 + HD) + 2;
          x0[u] = ps[lane];
          x1[u] = ps[lane + 64];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float f = s_f[wave][i + u - r0];
          A0 = __builtin_fmaf(x0[u], f, A0);
          A1 = __builtin_fmaf(x1[u], f, A1);
        }
      }
      for (; i < r1; ++i) {
        const float *ps = base + ((size_t)slot(i) * G + g) * (2 + HD) + 2;
        const float f = s_f[wave][i - r0];
        A0 = __builtin_fmaf(ps[lane], f, A0);
        A1 = __builtin_fmaf(ps[lane + 64], f, A1);
      }
      wave_sync();
    }
    float *o = a.out + ((size_t)b * a.Hq + (size_t)h * G + g) * HD;
    o[lane] = A0 / L;
    o[lane + 64] = A1 / L;
  }
}

template <typename T>
hipError_t launch_tiers(const Args &a, hipStream_t s) {
  dim3 grid(a.nv_att + a.nc_att + a.nd_att, a.B * a.Hkv);
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

hipError_t launch_combine(const Args &a, hipStream_t s) {
  dim3 grid(a.B * a.Hkv);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((hardkv_combine<1>), grid, dim3(NTHREADS), 0, s, a); break;
    case 2: hipLaunchKernelGGL((hardkv_combine<2>), grid, dim3(NTHREADS), 0, s, a); break;
    case 4: hipLaunchKernelGGL((hardkv_combine<4>), grid, dim3(NTHREADS), 0, s, a); break;
    case 8: hipLaunchKernelGGL((hardkv_combine<8>), grid, dim3(NTHREADS), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hardkv
