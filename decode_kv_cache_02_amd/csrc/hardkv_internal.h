// hardkv_internal.h -- shared definitions of the HIP kernels and the host entry points.
#pragma once
#include <cstddef>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hardkv.h"

namespace hardkv {

constexpr int BK = 64;        // tokens per block: one wavefront, one mask word
constexpr int HD = 128;       // head dim
constexpr int NCOEFF = 10;    // Taylor coefficients of 2^f on [0, 1)
constexpr int NTHREADS = 256; // threads per workgroup of every kernel
constexpr int NB1 = 3073;     // level-1 buckets of the mass radix select (key >> 16)
constexpr int SEL_THREADS = 1024;     // threads of the select workgroup (one per head)
constexpr int MAX_POOL_BLOCKS = HARDKV_MAX_POOL_BLOCKS; // pool ring blocks per head the select LDS can index
constexpr int CAND_CAP = 8192;        // cut-bucket candidates resolved in LDS
constexpr int SEL_SLICE_BLOCKS = 256; // pool blocks per workgroup when a head's select is split
constexpr int SEL_SPLIT_MIN = 4;      // slices per head from which the select is split
constexpr int FUSE_COND_BLOCKS = 4;   // blocks per step up to which the step's select condenses
constexpr int SCORE_LIVE_BLOCKS = 32; // most blocks per score workgroup under destructive selection

// Per-head values that the split select passes between its kernels.
struct alignas(128) SelHead {
  unsigned long long w_all, w_u, T, R1;  // masses, the top-p target, mass needed from the cut bucket
  int32_t b1;                            // level-1 bucket that holds the cut
  int32_t pad_[7];
  // candidates of that bucket (a counter, may exceed CAND_CAP); on a 64-byte line of its
  // own, apart from the fields above, which one workgroup stores while the others add here
  uint32_t ncand;
};
static_assert(offsetof(SelHead, ncand) == 64, "ncand on its own line");

// Entropy fit of the calibration temperature: rounds of a grid on log2 tau.
constexpr int FIT_POINTS = 17;          // grid points per round (16 intervals)
constexpr int FIT_ROUNDS = 5;
constexpr int FIT_SPLIT_ROWS = 4096;    // pool rows per workgroup when a head's fit is split
constexpr int FIT_SPLIT_MIN_ROWS = 2 * FIT_SPLIT_ROWS;  // pool capacity from which it may be split
constexpr int FIT_MAX_SLICES = (MAX_POOL_BLOCKS * 64 + FIT_SPLIT_ROWS - 1) / FIT_SPLIT_ROWS;  // per head

// Per-head values that the split fit passes between its kernels.
struct FitHead {
  double H;                                   // target entropy (nats)
  float m;                                    // max score
  int32_t pad_;
  double lo[FIT_ROUNDS], hi[FIT_ROUNDS];      // bracket of each round (log2 tau)
};

// Per-head plan of the current step, written by the select kernel and read by the
// kernels after it (rewrite, condense), so that they see the pool as select saw it.
struct alignas(64) HeadInfo {
  int64_t t_plan;   // t after the append
  int64_t c_plan;   // pool head before condensation
  uint32_t w_th;    // threshold weight of the top-p cut
  uint32_t r;       // tokens of weight w_th that are kept (lowest positions first)
  int32_t kstar;
  int32_t E;        // blocks to condense
  int32_t nu_plan;  // condensed-slot cursor before condensation
  int32_t rw;       // 1: the head's kept rows are rewritten into its view this step
  uint64_t w_all;
  int64_t voff;     // first view row of the head (row index into the view arrays)
  float kappa;      // calibration slope of the step (fitted temperature)
  float tau;        // the fitted temperature
};

// Everything a kernel needs, passed by value.
struct Args {
  // inputs and outputs of the call
  const void *q, *k_new, *v_new;
  float *out;
  // state
  void *dense_k, *dense_v, *pool_k, *pool_v, *view_k, *view_v;
  void *sink_k, *sink_v;    // [BH][S][D] (S > 0)
  int32_t *view_pos;
  float *cond_kn, *cond_vn, *cond_omega;
  int32_t *cond_n, *cond_cursor;
  int64_t *seq_len, *pool_head;
  float *scores;
  uint32_t *weights;
  uint64_t *mask;
  int32_t *budget, *n_condense;
  uint64_t *w_all, *w_u, *thresh;
  int32_t *regularized;     // may be null
  int32_t *view_off;        // [BH + 1] CSR offsets (SUM layout)
  float *tau_fit;           // [BH] fitted temperatures (may be null)
  uint32_t *error_word;
  // workspace
  HeadInfo *head;
  float *cmax;        // [BH][nch_score] max score of each score workgroup
  float *ent;         // [BH][nch_score][G][3] per query: (max, sum 2^(l-max), sum 2^(l-max)(l-max)),
                      // l = q . k log2(e) / sqrt(D) (entropy calibration)
  uint2 *blkinfo;     // [BH][P] per ring block: (first view row, ties before the block)
  float *part;        // [BH][npart][G][2 + HD] attention partials (m, l, acc)
  // split select (nsp > 1 slices per head)
  unsigned long long *phist;  // [BH][nsp][NB1] level-1 mass histogram of each slice
  unsigned long long *psum;   // [BH][nsp][2] (pool mass, survivor mass) of each slice
  SelHead *selh;              // [BH]
  uint32_t *cand_g;           // [BH][CAND_CAP] candidates of the cut bucket
  FitHead *fith;      // [BH] split fit: target, max, brackets
  double *fitp;       // [FIT_ROUNDS][BH][nfs][2 * FIT_POINTS] split fit: each slice's sums
  uint32_t *kx;       // [BH] nonzero once a 16-bit key outside KEY_SAFE has entered the head's
                      // pool (since its prefill): its scores then take the unfused products
  int kx_unknown;     // 1: kx is not kept for this state (the no-alloc step): every head's
                      // scores take the unfused products
  // the shared head-wise block pool (pool_shared): pool_k / pool_v hold NB physical blocks of
  // 64 rows; btab maps ring block pb of unit bh to its physical block (-1: none); the free
  // blocks are free_list[0 .. *free_top)
  int pool_shared, NB;
  // destructive selection: a pool row is in play iff it arrived after the last selection
  // (at or past the pool end of its plan) or that selection kept it (its mask bit)
  int destructive;
  int32_t *btab, *free_list, *free_top;
  int64_t *tsnap;     // [B] t of the step a selection made ahead is for (the pipeline)
  const uint32_t *kx_src;  // the current state's kx, copied by the pipeline's fork
  // prefill
  const void *k_ctx, *v_ctx;
  const int64_t *ctx_len;
  int64_t max_len;
  // sizes
  int B, Hq, Hkv, G, W, P, S_cap, V_cap, C, mode, merge_bias;
  int S;                    // sink prefix tokens (0: none)
  int cb_score, nch_score;  // score: blocks per workgroup, workgroups per head
  int nsp;                  // select: slices per head (1: one workgroup does the whole select)
  int nfs;                  // entropy fit: slices per head (1: one workgroup does the whole fit)
  int cond_small;           // at most FUSE_COND_BLOCKS blocks can condense per step
  int fuse_cond;            // this select launch also condenses (the fused step, cond_small)
  int cb_reg, nch_reg;      // rewrite: blocks per workgroup, workgroups per head
  int rv_att, nv_att;       // attention over the view (standalone): rows per workgroup, count
  int rc_att, nc_att;       // attention over condensed slots
  int rd_att, nd_att;       // attention over the dense window
  int rs_att, ns_att;       // attention over the sink rows
  int rt_att, nt_att;       // attention over the pool positions since the last selection
  int ntp;                  // tail segments in this call's partials (0 or nt_att)
  int nvp;                  // view partial slots written by this call
  int npart, part_cd_base;  // partial slots per head; first condensed/dense slot
  int xp_base, nxp;         // gathered-row partial slots of the standalone attention
  int reg_policy, mti_lower, mti_upper;  // regularize policy and its budget thresholds
  int reg_launch;           // the policy the launches are shaped for: reg_policy, or for the
                            // memory-time controller REWRITE / SPARSE when its choice is the same
                            // for every head that keeps a row
  // the memory-time controller (policy MTI_AUTO): H, per-row costs (fs), fixed cost
  int mti_horizon;
  uint32_t mti_c_view, mti_c_write, mti_c_scan, mti_c_hold;
  uint32_t mti_c_gather[9];
  int64_t mti_fixed;
  int gather_mode;          // rewrite kernel: GATHER_* below
  int view_sum;             // 1: Flatten Index to the sum (packed views)
  int calibration;          // HARDKV_CAL_*
  int64_t view_rows;        // rows of the view arrays: B * Hkv * V_cap, or view_total
  int ncs;                  // condense workgroups per head
  int bh0, nbh;             // (sequence, KV head) units this launch covers: [bh0, bh0 + nbh)
  uint32_t pq;
  float coeff[NCOEFF];
  float kappa[HARDKV_MAX_KV_HEADS];
  float att_scale;          // log2(e) / sqrt(D): logits in base 2
};

// What the rewrite kernel does with the kept rows it gathers from the pool:
//   GATHER_STEP       fused step: attend them; store them into the view if the head's rw
//   GATHER_REWRITE    standalone regularize: store them if rw
//   GATHER_ATTEND_NRW standalone attention: attend them for heads with rw == 0 only
//   GATHER_ATTEND_ALL Sparse Loading attention: attend them for every head
// The attending modes other than GATHER_STEP write their partials at xp_base + chunk.
enum { GATHER_STEP = 0, GATHER_REWRITE = 1, GATHER_ATTEND_NRW = 2, GATHER_ATTEND_ALL = 3 };

// launchers (one per kernel); each returns a hipError_t
hipError_t launch_prefill(const Args &a, hipStream_t s, bool bf16);
hipError_t launch_append(const Args &a, hipStream_t s, bool bf16);
// the pipeline's fork: t of every sequence and the current state's key-magnitude flags into
// the state of the selection made ahead
hipError_t launch_fork(const Args &a, hipStream_t s);
hipError_t launch_score(const Args &a, hipStream_t s, bool bf16);
hipError_t launch_select(const Args &a, hipStream_t s, bool bf16);
// exclusive scan of the rewritten budgets into view_off and each head's voff (SUM layout)
hipError_t launch_flatten(const Args &a, hipStream_t s);
// entropy-matched temperature of every head (calibration ENTROPY), before the select
hipError_t launch_fit(const Args &a, hipStream_t s);
// rewrite kernel: `mask` writes the mask words, `copy` copies the kept rows into the view,
// `attend` adds the view attention and the condensed/dense attention segments
hipError_t launch_rewrite(const Args &a, hipStream_t s, bool bf16, bool mask, bool copy, bool attend);
hipError_t launch_condense(const Args &a, hipStream_t s, bool bf16);
hipError_t launch_attend(const Args &a, hipStream_t s, bool bf16);
hipError_t launch_combine(const Args &a, hipStream_t s);

// The memory-time controller's choice for a head with kstar kept rows out of n survivors:
// rewrite iff k* c_write + H k* (c_view + c_hold) + F < H (k* g[b] + n c_scan), b the kept
// eighth (the terms both policies share cancel); exact in 64-bit integers for k*, n < 2^20,
// H < 2^16, costs < 2^24, F < 2^41.
__host__ __device__ inline bool mti_rewrites(int64_t kstar, int64_t n, int64_t H, uint32_t c_view,
                                             uint32_t c_write, uint32_t c_scan, uint32_t c_hold,
                                             const uint32_t *c_gather, int64_t fixed) {
  if (kstar <= 0 || n <= 0) return false;
  const int64_t b = (8 * kstar) / n < 8 ? (8 * kstar) / n : 8;
  const int64_t lhs = kstar * (int64_t)c_write + H * kstar * ((int64_t)c_view + (int64_t)c_hold) + fixed;
  const int64_t rhs = H * (kstar * (int64_t)c_gather[b] + n * (int64_t)c_scan);
  return lhs < rhs;
}

// ---------------------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------------------
#define HK_DEV __device__ __forceinline__

// Magnitudes for which every product of a 16-bit query element and a 16-bit key element
// is exact in fp32 (KEY_SAFE: biased exponent in [64, 192), |k| in [2^-63, 2^65); the
// query: |q| in [2^-72, 2^62); zeros always).  A product of two 8-bit significands has at
// most 16 significant bits, its lowest at 2^(eq + ek - 14) >= 2^-149, and it stays below
// 2^127.  With exact products, fl(fl(q0 k0) + fl(q1 k1)) equals fma(q0, k0, fl(q1 k1)).
constexpr uint32_t KEY_EXP_LO = 64, KEY_EXP_HI = 192;
constexpr float Q_SAFE_LO = 0x1p-72f, Q_SAFE_HI = 0x1p62f;

// whether a 32-bit word holds a nonzero 16-bit key element outside KEY_SAFE
HK_DEV bool key_word_unsafe(uint32_t w) {
  const uint32_t e0 = (w >> 7) & 0xFFu, e1 = (w >> 23) & 0xFFu;
  const bool b0 = (w & 0x7FFFu) != 0u && (e0 < KEY_EXP_LO || e0 >= KEY_EXP_HI);
  const bool b1 = (w & 0x7FFF0000u) != 0u && (e1 < KEY_EXP_LO || e1 >= KEY_EXP_HI);
  return b0 || b1;
}
HK_DEV bool key_piece_unsafe(const uint4 &x) {
  return key_word_unsafe(x.x) || key_word_unsafe(x.y) || key_word_unsafe(x.z) || key_word_unsafe(x.w);
}

HK_DEV float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

HK_DEV float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
HK_DEV float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// 8 consecutive elements of a row as floats; T is the storage type tag.
struct BF16 {};
struct F32 {};

HK_DEV void load8(const void *p, float (&f)[8], BF16) {
  uint4 u = *reinterpret_cast<const uint4 *>(p);
  f[0] = bf_lo(u.x); f[1] = bf_hi(u.x); f[2] = bf_lo(u.y); f[3] = bf_hi(u.y);
  f[4] = bf_lo(u.z); f[5] = bf_hi(u.z); f[6] = bf_lo(u.w); f[7] = bf_hi(u.w);
}
HK_DEV void load8(const void *p, float (&f)[8], F32) {
  float4 a = reinterpret_cast<const float4 *>(p)[0];
  float4 b = reinterpret_cast<const float4 *>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

template <typename T> struct Elem;
template <> struct Elem<BF16> { static constexpr int bytes = 2; };
template <> struct Elem<F32> { static constexpr int bytes = 4; };

// raw copy of the 8 elements a lane owns in a row
template <typename T> struct Raw8;
template <> struct Raw8<BF16> { uint4 v; };
template <> struct Raw8<F32> { float4 a, b; };

// Streaming accesses: keys and values are read once per step and view rows written once,
// so they bypass cache retention (non-temporal), which raises sustained HBM bandwidth.
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
HK_DEV uint4 nt_load16(const void *p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4u32 *>(p)));
}
HK_DEV void nt_store16(void *p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(v4u32, v), reinterpret_cast<v4u32 *>(p));
}
HK_DEV void raw_load_nt(const void *p, Raw8<BF16> &r) { r.v = nt_load16(p); }
HK_DEV void raw_load_nt(const void *p, Raw8<F32> &r) {
  r.a = __builtin_bit_cast(float4, nt_load16(p));
  r.b = __builtin_bit_cast(float4, nt_load16((const char *)p + 16));
}
HK_DEV void raw_store_nt(void *p, const Raw8<BF16> &r) { nt_store16(p, r.v); }
HK_DEV void raw_store_nt(void *p, const Raw8<F32> &r) {
  nt_store16(p, __builtin_bit_cast(uint4, r.a));
  nt_store16((char *)p + 16, __builtin_bit_cast(uint4, r.b));
}

HK_DEV void raw_load(const void *p, Raw8<BF16> &r) { r.v = *reinterpret_cast<const uint4 *>(p); }
HK_DEV void raw_load(const void *p, Raw8<F32> &r) {
  r.a = reinterpret_cast<const float4 *>(p)[0];
  r.b = reinterpret_cast<const float4 *>(p)[1];
}
HK_DEV void raw_store(void *p, const Raw8<BF16> &r) { *reinterpret_cast<uint4 *>(p) = r.v; }
HK_DEV void raw_store(void *p, const Raw8<F32> &r) {
  reinterpret_cast<float4 *>(p)[0] = r.a;
  reinterpret_cast<float4 *>(p)[1] = r.b;
}
// Raw buffer resources (stride 0, byte offsets).  The hardware drops an access whose
// offset lies outside the resource's range: a load returns zeros, a store writes
// nothing.  Rows a lane must skip get the offset BUF_SKIP, outside every range made
// here, instead of a branch around the access: with no branches the compiler can count
// the accesses in flight and waits only for those whose data it needs next.
typedef __amdgpu_buffer_rsrc_t BufRes;
constexpr uint32_t BUF_SKIP = 0x80000000u;
constexpr uint64_t BUF_MAX_BYTES = 0x7FFFFFF0u;  // every range stays below BUF_SKIP
constexpr int BUF_NT = 2;                       // cache policy bits: non-temporal
HK_DEV BufRes make_buf(const void *base, uint64_t bytes) {
  const uint32_t n = (uint32_t)(bytes < BUF_MAX_BYTES ? bytes : BUF_MAX_BYTES);
  // word 3 of a gfx9-family raw buffer: 32-bit data format, no swizzle or index stride
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)n, 0x00020000);
}
static_assert((uint64_t)MAX_POOL_BLOCKS * 64 * 128 * 4 <= BUF_MAX_BYTES, "a head's pool rows fit one buffer range");
HK_DEV uint4 buf_load16_nt(BufRes r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, BUF_NT));
}
HK_DEV void buf_store16_nt(BufRes r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, v), r, off, 0, BUF_NT);
}
// a lane's 8 elements of a row at byte offset off (BUF_SKIP: zeros / nothing written)
HK_DEV void buf_load_nt(BufRes r, uint32_t off, Raw8<BF16> &x) { x.v = buf_load16_nt(r, off); }
HK_DEV void buf_load_nt(BufRes r, uint32_t off, Raw8<F32> &x) {
  x.a = __builtin_bit_cast(float4, buf_load16_nt(r, off));
  x.b = __builtin_bit_cast(float4, buf_load16_nt(r, off + 16));
}
HK_DEV void buf_store_nt(BufRes r, uint32_t off, const Raw8<BF16> &x) { buf_store16_nt(r, off, x.v); }
HK_DEV void buf_store_nt(BufRes r, uint32_t off, const Raw8<F32> &x) {
  buf_store16_nt(r, off, __builtin_bit_cast(uint4, x.a));
  buf_store16_nt(r, off + 16, __builtin_bit_cast(uint4, x.b));
}

HK_DEV void raw_to_f(const Raw8<BF16> &r, float (&f)[8]) {
  f[0] = bf_lo(r.v.x); f[1] = bf_hi(r.v.x); f[2] = bf_lo(r.v.y); f[3] = bf_hi(r.v.y);
  f[4] = bf_lo(r.v.z); f[5] = bf_hi(r.v.z); f[6] = bf_lo(r.v.w); f[7] = bf_hi(r.v.w);
}
HK_DEV void raw_to_f(const Raw8<F32> &r, float (&f)[8]) {
  f[0] = r.a.x; f[1] = r.a.y; f[2] = r.a.z; f[3] = r.a.w;
  f[4] = r.b.x; f[5] = r.b.y; f[6] = r.b.z; f[7] = r.b.w;
}

// DPP lane exchanges inside a row of 16 lanes
template <int CTRL> HK_DEV float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;

// ordered encoding of finite floats into uint32 (> 0), for atomicMax
HK_DEV uint32_t f2ord(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
HK_DEV float ord2f(uint32_t e) { return __uint_as_float((e & 0x80000000u) ? (e & 0x7fffffffu) : ~e); }

HK_DEV uint32_t lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }
HK_DEV uint32_t popc_below(uint64_t m) {  // set bits of m below this lane
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}
HK_DEV uint64_t ballot(bool p) { return __ballot(p); }

// Workgroups of a launch are dispatched round-robin over the 8 XCDs (workgroup i to XCD
// i mod 8).  xcd_swizzle maps the k-th workgroup that XCD x receives to position k of a
// contiguous range of the linear work index (XCD x gets range x), so that the chunks one
// XCD streams are neighbours in memory.  A bijection on [0, total).
HK_DEV int xcd_swizzle(int lin, int total) {
  const int q = total >> 3, r = total & 7, x = lin & 7, k = lin >> 3;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + k;
}

// the pool ends where the dense window starts: max(S, t - W) with a sink prefix of S
// tokens (the pool then starts at S); the dense window is [dense_lo, t)
HK_DEV int64_t pool_end(int64_t t, int W, int S) { return t - W > S ? t - W : (int64_t)S; }
HK_DEV int64_t dense_lo_of(int64_t t, int W, int S) {
  const int64_t lo = pool_end(t, W, S);
  return lo < t ? lo : t;
}
// Row 0 of ring block pb of unit bh in the pool arrays: the unit's own ring, or the physical
// block the block table gives it in the shared pool.
HK_DEV size_t pool_row0(const Args &a, int bh, int pb) {
  if (a.pool_shared) {
    const int32_t phys = a.btab[(size_t)bh * a.P + pb];
    return (size_t)(phys < 0 ? 0 : phys) * BK;
  }
  return ((size_t)bh * a.P + pb) * BK;
}

// Destructive selection: the pool end when the last selection ran (positions from here on
// arrived since), read before this step's selection replaces the plan; and whether position
// p of a block whose mask word is mw is in play.
HK_DEV int64_t pend_last_selection(const Args &a, int bh) { return pool_end(a.head[bh].t_plan, a.W, a.S); }
HK_DEV bool in_play(int64_t p, int64_t pend_last, uint64_t mw) {
  return p >= pend_last || ((mw >> (p & (BK - 1))) & 1ull) != 0ull;
}

HK_DEV int64_t plan_E(int64_t N, int mode, int S_cap) {
  return (mode != HARDKV_COND_OFF && N > S_cap) ? (N - S_cap + BK - 1) / BK : 0;
}

// agent-scope atomics and fences (cross-XCD visibility)
HK_DEV uint32_t atomic_add_acq_rel(uint32_t *p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
HK_DEV uint32_t atomic_load_acq(uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
HK_DEV void fence_agent() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent"); }
HK_DEV void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace hardkv
