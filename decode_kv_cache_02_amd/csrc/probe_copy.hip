// Copy references for the rewrite (a measurement aid, not part of the step): the kept rows
// of a pool, K and V rows of 128 bf16 elements (256 bytes), gathered through a list of row
// indices and written to contiguous rows, in the two access patterns a gather-copy can take
// on gfx950:
//   ONE_SHOT  every thread moves one 16-byte piece of a K row and the same piece of its V
//             row, then exits (no thread waits for its own stores);
//   LOOP      a wavefront moves 64 consecutive list entries, 16 rows a batch (four rows per
//             16-lane group), with the next batch's loads issued before this batch's stores,
//             the pattern of a kernel that also consumes the rows it moves (the fused
//             rewrite and attention).
// Built into its own library; the step's library does not use it.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int ROWB = 256;  // bytes of a bf16 row of 128 elements
constexpr int NTHREADS = 256;
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4u32 ld_nt(const char *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4u32 *>(p));
}
__device__ __forceinline__ void st_nt(char *p, v4u32 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<v4u32 *>(p));
}

__global__ __launch_bounds__(NTHREADS) void probe_one_shot(const char *__restrict__ sk, const char *__restrict__ sv,
                                                           char *__restrict__ dk, char *__restrict__ dv,
                                                           const int32_t *__restrict__ rows, int64_t nrows) {
  const int64_t i = (int64_t)blockIdx.x * NTHREADS + threadIdx.x;
  const int64_t r = i >> 4;  // 16 pieces per row
  if (r >= nrows) return;
  const int piece = (int)(i & 15);
  const size_t src = (size_t)rows[r] * ROWB + piece * 16, dst = (size_t)r * ROWB + piece * 16;
  const v4u32 k = ld_nt(sk + src), v = ld_nt(sv + src);
  st_nt(dk + dst, k);
  st_nt(dv + dst, v);
}

__global__ __launch_bounds__(NTHREADS) void probe_loop(const char *__restrict__ sk, const char *__restrict__ sv,
                                                       char *__restrict__ dk, char *__restrict__ dv,
                                                       const int32_t *__restrict__ rows, int64_t nrows) {
  const int lane = threadIdx.x & 63, sub = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * 64;
  if (r0 >= nrows) return;
  const int n = (int)(nrows - r0 < 64 ? nrows - r0 : 64);
  const int nb = (n + 15) / 16;
  v4u32 kA[4], vA[4], kB[4], vB[4];
  // rows past the wavefront's entries load its first row and store nothing
  auto issue = [&](int it, v4u32 (&k)[4], v4u32 (&v)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = it * 16 + j * 4 + grp;
      const size_t src = (size_t)rows[r0 + (e < n ? e : 0)] * ROWB + sub * 16;
      k[j] = ld_nt(sk + src);
      v[j] = ld_nt(sv + src);
    }
  };
  auto put = [&](int it, const v4u32 (&k)[4], const v4u32 (&v)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = it * 16 + j * 4 + grp;
      if (e < n) {
        const size_t dst = (size_t)(r0 + e) * ROWB + sub * 16;
        st_nt(dk + dst, k[j]);
        st_nt(dv + dst, v[j]);
      }
    }
  };
  issue(0, kA, vA);
  int it = 0;
  for (; it + 2 <= nb; it += 2) {
    issue(it + 1, kB, vB);
    put(it, kA, vA);
    if (it + 2 < nb) issue(it + 2, kA, vA);
    put(it + 1, kB, vB);
  }
  if (it < nb) put(it, kA, vA);
}

}  // namespace

extern "C" {

// Gathers rows[0 .. nrows) of src_k / src_v (rows of 256 bytes) into rows 0 .. nrows of
// dst_k / dst_v on `stream`.  mode 0: ONE_SHOT, 1: LOOP.  Every entry of rows must index a
// row of the source buffers (not checked on the device).  Returns 0, or -1 on a bad argument
// (null or unaligned pointer, nrows outside [0, 2^27], unknown mode), or the HIP error of the
// launch.
int32_t hardkv_probe_gather_copy(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                                 const int32_t *rows, int64_t nrows, int32_t mode, void *stream) {
  const void *ptrs[] = {src_k, src_v, dst_k, dst_v};
  for (const void *p : ptrs)
    if (!p || ((uintptr_t)p & 15u)) return -1;
  if (!rows || ((uintptr_t)rows & 3u) || nrows < 0 || nrows > ((int64_t)1 << 27) || (mode != 0 && mode != 1))
    return -1;
  if (nrows == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  const char *sk = (const char *)src_k, *sv = (const char *)src_v;
  char *dk = (char *)dst_k, *dv = (char *)dst_v;
  if (mode == 0) {
    const int64_t threads = nrows * 16;
    hipLaunchKernelGGL(probe_one_shot, dim3((unsigned)((threads + NTHREADS - 1) / NTHREADS)), dim3(NTHREADS), 0, s,
                       sk, sv, dk, dv, rows, nrows);
  } else {
    const int64_t waves = (nrows + 63) / 64;
    hipLaunchKernelGGL(probe_loop, dim3((unsigned)((waves + 3) / 4)), dim3(NTHREADS), 0, s, sk, sv, dk, dv, rows,
                       nrows);
  }
  return (int32_t)hipGetLastError();
}

}  // extern "C"
