// hardkv_api.hip -- the C ABI: argument checks, launch geometry, workspace layout and the
// stream-ordered kernel sequences of each entry point.  Nothing here allocates, frees,
// synchronizes, or touches device memory from the host.
#include <math.h>
#include <string.h>

#include <mutex>

#include "hardkv_internal.h"

// Scratch of hardkv_step_noalloc, one copy per GPU (zero-filled at load; nothing in it has to
// start at zero).  Host code never passes this name to a kernel: it stands for the array
// only on the device; the host uses the address looked up per device below.
static __device__ __align__(256) unsigned char scratch[HARDKV_STATIC_SCRATCH_BYTES];

namespace hardkv {
namespace {

constexpr int MAX_DEVICES = 64;

// The device address of `scratch` on the current device, looked up once per device with
// that device current.
int32_t scratch_address(void **out) {
  static std::mutex mu;
  static void *addr[MAX_DEVICES] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return HARDKV_EHIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HARDKV_EHIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return HARDKV_OK;
}

constexpr double LOG2E = 1.4426950408889634074;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void *p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

// the memory-time controller's inputs stay inside the ranges its exact integer comparison
// covers
bool mti_config_ok(const hardkv_config *cfg) {
  if (cfg->mti_horizon < 0 || cfg->mti_horizon > HARDKV_MTI_MAX_HORIZON) return false;
  const uint32_t c[] = {cfg->mti_c_view, cfg->mti_c_write, cfg->mti_c_scan, cfg->mti_c_hold, cfg->mti_c_score};
  for (uint32_t x : c)
    if (x >= HARDKV_MTI_MAX_COST) return false;
  for (int i = 0; i < 9; ++i)
    if (cfg->mti_c_gather[i] >= HARDKV_MTI_MAX_COST) return false;
  return cfg->mti_fixed >= 0 && cfg->mti_fixed <= HARDKV_MTI_MAX_FIXED;
}

bool mti_rewrites_cfg(const hardkv_config *cfg, int64_t H, int64_t kstar, int64_t n) {
  return mti_rewrites(kstar, n, H, cfg->mti_c_view, cfg->mti_c_write, cfg->mti_c_scan, cfg->mti_c_hold,
                      cfg->mti_c_gather, cfg->mti_fixed);
}

// The launches a policy needs: the memory-time controller decides per head on the device,
// but without a scan cost or a fixed cost its choice for a head that keeps a row depends
// only on the kept eighth b (k* cancels); when it is the same for all nine, the step is
// shaped like REWRITE (no gather of views' rows) or SPARSE (no store path).  The device
// still applies the controller (a head keeping nothing is never rewritten).
int launch_policy(const hardkv_config *cfg) {
  if (cfg->regularize != HARDKV_REG_MTI_AUTO || cfg->mti_c_scan != 0 || cfg->mti_fixed != 0)
    return cfg->regularize;
  const int64_t H = cfg->mti_horizon;
  const int64_t lhs = (int64_t)cfg->mti_c_write + H * ((int64_t)cfg->mti_c_view + (int64_t)cfg->mti_c_hold);
  int n_rw = 0;
  for (int b = 0; b < 9; ++b) n_rw += lhs < H * (int64_t)cfg->mti_c_gather[b] ? 1 : 0;
  return n_rw == 9 ? HARDKV_REG_REWRITE : n_rw == 0 ? HARDKV_REG_SPARSE : HARDKV_REG_MTI_AUTO;
}

struct Plan {
  Args a;
  size_t off_head, off_cmax, off_ent, off_blkinfo, off_part, off_phist, off_psum, off_selh, off_cand, off_kx,
      off_fith, off_fitp, off_tsnap, ws_bytes;
};

// Checks the configuration and derives every size; fills the size fields of p.a.
int32_t plan(const hardkv_config *cfg, Plan &p) {
  if (!cfg) return HARDKV_EINVAL;
  Args &a = p.a;
  memset(&a, 0, sizeof(a));
  if (cfg->batch < 1 || cfg->num_kv_heads < 1 || cfg->num_q_heads < 1) return HARDKV_EINVAL;
  if (cfg->num_kv_heads > HARDKV_MAX_KV_HEADS) return HARDKV_EUNSUPPORTED;
  if ((int64_t)cfg->batch * cfg->num_kv_heads > HARDKV_MAX_UNITS) return HARDKV_EUNSUPPORTED;
  if (cfg->num_q_heads % cfg->num_kv_heads) return HARDKV_EINVAL;
  const int G = cfg->num_q_heads / cfg->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return HARDKV_EUNSUPPORTED;
  if (cfg->head_dim != HD) return HARDKV_EUNSUPPORTED;
  if (cfg->dtype != HARDKV_BF16 && cfg->dtype != HARDKV_F32) return HARDKV_EINVAL;
  if (cfg->dense_window < 1) return HARDKV_EINVAL;
  if (cfg->sparse_cap < BK || cfg->sparse_cap % BK) return HARDKV_EINVAL;
  if (cfg->pool_blocks < 1) return HARDKV_EINVAL;
  if (cfg->pool_blocks > MAX_POOL_BLOCKS) return HARDKV_EUNSUPPORTED;
  if ((int64_t)cfg->pool_blocks * BK < (int64_t)cfg->sparse_cap + BK) return HARDKV_EINVAL;
  if (cfg->cond_mode < HARDKV_COND_OFF || cfg->cond_mode > HARDKV_COND_MERGE) return HARDKV_EINVAL;
  if (cfg->view_cap < cfg->sparse_cap) return HARDKV_EINVAL;
  if (cfg->cond_mode == HARDKV_COND_OFF && (int64_t)cfg->view_cap < (int64_t)cfg->pool_blocks * BK)
    return HARDKV_EINVAL;
  if (cfg->condensed_slots < 1) return HARDKV_EINVAL;
  if (!(cfg->top_p > 0.0 && cfg->top_p <= 1.0)) return HARDKV_EINVAL;
  const double pq = rint(cfg->top_p * 65536.0);
  if (pq < 1.0) return HARDKV_EINVAL;
  if (!cfg->tau) return HARDKV_EINVAL;
  for (int h = 0; h < cfg->num_kv_heads; ++h)
    if (!(cfg->tau[h] > 0.0f)) return HARDKV_EINVAL;
  if (cfg->regularize < HARDKV_REG_REWRITE || cfg->regularize > HARDKV_REG_MTI_AUTO) return HARDKV_EINVAL;
  if (cfg->regularize == HARDKV_REG_MTI_AUTO && !mti_config_ok(cfg)) return HARDKV_EINVAL;
  if (cfg->regularize == HARDKV_REG_MTI && (cfg->mti_lower < 0 || cfg->mti_upper < cfg->mti_lower))
    return HARDKV_EINVAL;
  if (cfg->view_layout != HARDKV_VIEW_MAXLEN && cfg->view_layout != HARDKV_VIEW_SUM) return HARDKV_EINVAL;
  if (cfg->view_layout == HARDKV_VIEW_SUM && cfg->view_total < 0) return HARDKV_EINVAL;
  if (cfg->calibration != HARDKV_CAL_FIXED && cfg->calibration != HARDKV_CAL_ENTROPY) return HARDKV_EINVAL;
  if (cfg->sink < 0 || cfg->sink % BK || cfg->sink > HARDKV_MAX_SINK) return HARDKV_EINVAL;
  if (cfg->pool_layout != HARDKV_POOL_RING && cfg->pool_layout != HARDKV_POOL_SHARED) return HARDKV_EINVAL;
  if (cfg->selection != HARDKV_SEL_VIEW && cfg->selection != HARDKV_SEL_DESTRUCTIVE) return HARDKV_EINVAL;
  if (cfg->selection == HARDKV_SEL_DESTRUCTIVE && cfg->calibration != HARDKV_CAL_FIXED) return HARDKV_EUNSUPPORTED;
  if (cfg->pool_layout == HARDKV_POOL_SHARED && (cfg->pool_total_blocks < 1 || cfg->pool_total_blocks >= (1 << 26)))
    return HARDKV_EINVAL;

  a.B = cfg->batch;
  a.Hq = cfg->num_q_heads;
  a.Hkv = cfg->num_kv_heads;
  a.G = G;
  a.W = cfg->dense_window;
  a.P = cfg->pool_blocks;
  a.S_cap = cfg->sparse_cap;
  a.V_cap = cfg->view_cap;
  a.C = cfg->condensed_slots;
  a.S = cfg->sink;
  a.mode = cfg->cond_mode;
  a.merge_bias = cfg->merge_bias ? 1 : 0;
  a.view_sum = cfg->view_layout == HARDKV_VIEW_SUM ? 1 : 0;
  a.calibration = cfg->calibration;
  a.view_rows = a.view_sum ? (int64_t)cfg->view_total
                           : (int64_t)cfg->batch * cfg->num_kv_heads * cfg->view_cap;
  a.destructive = cfg->selection == HARDKV_SEL_DESTRUCTIVE ? 1 : 0;
  a.pool_shared = cfg->pool_layout == HARDKV_POOL_SHARED ? 1 : 0;
  a.NB = a.pool_shared ? cfg->pool_total_blocks : 0;
  a.reg_policy = cfg->regularize;
  a.reg_launch = launch_policy(cfg);
  a.mti_lower = cfg->mti_lower;
  a.mti_upper = cfg->mti_upper;
  a.mti_horizon = cfg->mti_horizon;
  a.mti_c_view = cfg->mti_c_view;
  a.mti_c_write = cfg->mti_c_write;
  a.mti_c_scan = cfg->mti_c_scan;
  a.mti_c_hold = cfg->mti_c_hold;
  for (int i = 0; i < 9; ++i) a.mti_c_gather[i] = cfg->mti_c_gather[i];
  a.mti_fixed = cfg->mti_fixed;
  a.pq = (uint32_t)pq;
  {
    // Taylor coefficients (ln 2)^i / i! of 2^f, rounded once to fp32
    const long double ln2 = 0.693147180559945309417232121458176568L;
    long double term = 1.0L;
    for (int i = 0; i < NCOEFF; ++i) {
      if (i > 0) term = term * ln2 / (long double)i;
      a.coeff[i] = (float)term;
    }
  }
  for (int h = 0; h < a.Hkv; ++h)
    a.kappa[h] = (float)(LOG2E / (sqrt((double)HD) * (double)cfg->tau[h]));
  a.att_scale = (float)(LOG2E / sqrt((double)HD));

  const int64_t BH = (int64_t)a.B * a.Hkv;
  const int64_t work = (int64_t)a.P * BH;
  // (destructive selection scores only the rows in play, so its chunks span more blocks)
  const int cb_max = a.destructive ? SCORE_LIVE_BLOCKS : 8;
  const int cb = (int)std::max<int64_t>(1, std::min<int64_t>(cb_max, work / 1024));
  a.cb_score = cb;
  a.nch_score = (a.P + cb - 1) / cb;
  // rewrite chunks of 4 blocks (one per wavefront) over the survivor blocks only: at most
  // S_cap / 64 of them after condensation, the whole ring in mode OFF
  const int max_survivor_blocks = a.mode == HARDKV_COND_OFF ? a.P : std::min(a.P, a.S_cap / BK);
  a.cb_reg = 4;
  a.nch_reg = (max_survivor_blocks + a.cb_reg - 1) / a.cb_reg;
  a.rv_att = 512;
  a.nv_att = (a.V_cap + a.rv_att - 1) / a.rv_att;
  a.rc_att = 64;
  a.nc_att = (a.C + a.rc_att - 1) / a.rc_att;
  a.rd_att = 128;
  a.nd_att = (a.W + a.rd_att - 1) / a.rd_att;
  a.rs_att = 128;
  a.ns_att = (a.S + a.rs_att - 1) / a.rs_att;
  a.part_cd_base = std::max(a.nch_reg, a.nv_att);
  // a step without selection attends the pool positions since the last one in nt_att
  // segments that stride over them in pieces of rt_att rows
  a.rt_att = 128;
  a.nt_att = 4;
  a.ntp = 0;
  a.xp_base = a.part_cd_base + a.nc_att + a.nd_att + a.ns_att + a.nt_att;  // then one slot per rewrite chunk
  a.npart = a.xp_base + a.nch_reg;
  // at most emax blocks condense in a step (a pool never exceeds its P*64 rows)
  const int emax = std::max(1, a.P - a.S_cap / BK);
  a.ncs = a.mode == HARDKV_COND_MERGE ? std::min(a.C, emax) : 1;
  a.cond_small = a.mode != HARDKV_COND_OFF && emax <= FUSE_COND_BLOCKS;
  a.fuse_cond = 0;

  // the select of a long pool is split over slices of SEL_SLICE_BLOCKS blocks
  a.nsp = (a.P + SEL_SLICE_BLOCKS - 1) / SEL_SLICE_BLOCKS;
  if (a.nsp < SEL_SPLIT_MIN) a.nsp = 1;
  // The entropy fit of long pools is split over slices of FIT_SPLIT_ROWS rows when the
  // heads alone would leave half the chip's 256 compute units idle (one workgroup per
  // head spends most of the fit on its own vector ALUs); otherwise its six extra launches
  // cost more than they save.
  a.nfs = 1;
  if (a.calibration && BH * 2 <= 256 && (int64_t)a.P * BK >= FIT_SPLIT_MIN_ROWS)
    a.nfs = (int)(((int64_t)a.P * BK + FIT_SPLIT_ROWS - 1) / FIT_SPLIT_ROWS);
  a.bh0 = 0;
  a.nbh = (int)BH;

  p.off_head = 0;
  p.off_cmax = align256(p.off_head + (size_t)BH * sizeof(HeadInfo));
  p.off_ent = align256(p.off_cmax + (size_t)BH * a.nch_score * sizeof(float));
  p.off_blkinfo = align256(p.off_ent + (a.calibration ? (size_t)BH * a.nch_score * G * 3 * sizeof(float) : 0));
  p.off_part = align256(p.off_blkinfo + (size_t)BH * a.P * sizeof(uint2));
  const size_t split = a.nsp > 1 ? 1 : 0;  // the split select's scratch
  p.off_phist = align256(p.off_part + (size_t)BH * a.npart * G * (2 + HD) * sizeof(float));
  p.off_psum = align256(p.off_phist + split * (size_t)BH * a.nsp * NB1 * sizeof(unsigned long long));
  p.off_selh = align256(p.off_psum + split * (size_t)BH * a.nsp * 2 * sizeof(unsigned long long));
  p.off_cand = align256(p.off_selh + split * (size_t)BH * sizeof(SelHead));
  p.off_kx = align256(p.off_cand + split * (size_t)BH * CAND_CAP * sizeof(uint32_t));
  p.off_fith = align256(p.off_kx + (size_t)BH * sizeof(uint32_t));
  const size_t fsplit = a.nfs > 1 ? 1 : 0;  // the split fit's scratch
  p.off_fitp = align256(p.off_fith + fsplit * (size_t)BH * sizeof(FitHead));
  p.off_tsnap = align256(p.off_fitp + fsplit * (size_t)FIT_ROUNDS * BH * a.nfs * 2 * FIT_POINTS * sizeof(double));
  p.ws_bytes = align256(p.off_tsnap + (size_t)a.B * sizeof(int64_t));
  return HARDKV_OK;
}

// Checks the state's pointers and points the kernel arguments at it.
int32_t bind(const hardkv_state *st, Plan &p) {
  if (!st) return HARDKV_EINVAL;
  const void *ptrs[] = {st->dense_k, st->dense_v, st->pool_k, st->pool_v, st->view_k, st->view_v,
                        st->view_pos, st->cond_kn, st->cond_vn, st->cond_omega, st->cond_n,
                        st->cond_cursor, st->seq_len, st->pool_head, st->scores, st->weights,
                        st->mask, st->budget, st->n_condense, st->w_all, st->w_u, st->thresh,
                        st->workspace};
  for (const void *q : ptrs)
    if (!aligned16(q)) return HARDKV_EINVAL;
  if (!st->error_word || ((uintptr_t)st->error_word & 3u)) return HARDKV_EINVAL;
  if (st->workspace_bytes < p.ws_bytes) return HARDKV_ECAPACITY;
  Args &a = p.a;
  if (a.pool_shared) {
    if (!aligned16(st->block_table) || !aligned16(st->free_list) || !st->free_top ||
        ((uintptr_t)st->free_top & 3u))
      return HARDKV_EINVAL;
    a.btab = st->block_table;
    a.free_list = st->free_list;
    a.free_top = st->free_top;
  }
  a.dense_k = st->dense_k;
  a.dense_v = st->dense_v;
  a.pool_k = st->pool_k;
  a.pool_v = st->pool_v;
  a.view_k = st->view_k;
  a.view_v = st->view_v;
  a.view_pos = st->view_pos;
  a.cond_kn = st->cond_kn;
  a.cond_vn = st->cond_vn;
  a.cond_omega = st->cond_omega;
  a.cond_n = st->cond_n;
  a.cond_cursor = st->cond_cursor;
  a.seq_len = st->seq_len;
  a.pool_head = st->pool_head;
  a.scores = st->scores;
  a.weights = st->weights;
  a.mask = st->mask;
  a.budget = st->budget;
  a.n_condense = st->n_condense;
  a.w_all = st->w_all;
  a.w_u = st->w_u;
  a.thresh = st->thresh;
  if (st->regularized && ((uintptr_t)st->regularized & 3u)) return HARDKV_EINVAL;
  a.regularized = st->regularized;
  if (p.a.view_sum && (!st->view_off || ((uintptr_t)st->view_off & 3u))) return HARDKV_EINVAL;
  if (st->view_off && ((uintptr_t)st->view_off & 3u)) return HARDKV_EINVAL;
  a.view_off = st->view_off;
  if (st->tau_fit && ((uintptr_t)st->tau_fit & 3u)) return HARDKV_EINVAL;
  a.tau_fit = st->tau_fit;
  if (a.S > 0 && (!aligned16(st->sink_k) || !aligned16(st->sink_v))) return HARDKV_EINVAL;
  a.sink_k = st->sink_k;
  a.sink_v = st->sink_v;
  a.error_word = st->error_word;
  char *ws = (char *)st->workspace;
  a.head = reinterpret_cast<HeadInfo *>(ws + p.off_head);
  a.cmax = reinterpret_cast<float *>(ws + p.off_cmax);
  a.ent = reinterpret_cast<float *>(ws + p.off_ent);
  a.blkinfo = reinterpret_cast<uint2 *>(ws + p.off_blkinfo);
  a.part = reinterpret_cast<float *>(ws + p.off_part);
  a.phist = reinterpret_cast<unsigned long long *>(ws + p.off_phist);
  a.psum = reinterpret_cast<unsigned long long *>(ws + p.off_psum);
  a.selh = reinterpret_cast<SelHead *>(ws + p.off_selh);
  a.cand_g = reinterpret_cast<uint32_t *>(ws + p.off_cand);
  a.kx = reinterpret_cast<uint32_t *>(ws + p.off_kx);
  a.fith = reinterpret_cast<FitHead *>(ws + p.off_fith);
  a.fitp = reinterpret_cast<double *>(ws + p.off_fitp);
  a.tsnap = reinterpret_cast<int64_t *>(ws + p.off_tsnap);
  return HARDKV_OK;
}

int32_t setup(const hardkv_config *cfg, const hardkv_state *st, Plan &p) {
  int32_t rc = plan(cfg, p);
  if (rc != HARDKV_OK) return rc;
  return bind(st, p);
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? HARDKV_OK : HARDKV_EHIP; }

bool is_bf16(const hardkv_config *cfg) { return cfg->dtype == HARDKV_BF16; }

constexpr int NSTAGES = 6;
const char *const kStageNames[NSTAGES] = {"append", "score", "select", "condense", "rewrite_attend",
                                          "combine"};

// Kernel `stage` of the fused step.  In the whole step (whole_step) the select launch
// also condenses when at most FUSE_COND_BLOCKS blocks can condense per step, and stage 3
// launches nothing; one stage at a time (timing) they stay apart.
hipError_t step_stage(const hardkv_config *cfg, Args &a, int stage, hipStream_t s, bool whole_step) {
  const bool bf = is_bf16(cfg);
  a.nvp = a.nch_reg;
  a.nxp = 0;
  a.ntp = 0;  // the step's own selection leaves no pool position unselected
  a.gather_mode = GATHER_STEP;
  const bool fuse = whole_step && a.cond_small;
  switch (stage) {
    case 0: return launch_append(a, s, bf);
    case 1: return launch_score(a, s, bf);
    case 2: {
      hipError_t e = a.calibration ? launch_fit(a, s) : hipSuccess;
      a.fuse_cond = fuse ? 1 : 0;
      if (e == hipSuccess) e = launch_select(a, s, bf);
      a.fuse_cond = 0;
      if (e == hipSuccess && a.view_sum) e = launch_flatten(a, s);
      return e;
    }
    case 3: return fuse ? hipSuccess : launch_condense(a, s, bf);
    case 4: return launch_rewrite(a, s, bf, true, true, true);
    case 5: return launch_combine(a, s);
    default: return hipErrorInvalidValue;
  }
}

// The standalone attention: the tier kernel attends the view segments of the rewritten
// heads (none under SPARSE, or when `sparse` asks for Sparse Loading everywhere) and the
// condensed and dense segments; the rewrite kernel gathers and attends the kept rows of
// the other heads (none under REWRITE) from the pool; the combine reduces both.
hipError_t attend_calls(const hardkv_config *cfg, Args &a, hipStream_t s, bool sparse) {
  const bool bf = is_bf16(cfg);
  const bool views = !sparse && a.reg_launch != HARDKV_REG_SPARSE;
  const bool gather = sparse || a.reg_launch != HARDKV_REG_REWRITE;
  if (!views) a.nv_att = 0;
  a.nvp = a.nv_att;
  a.ntp = a.nt_att;
  a.nxp = gather ? a.nch_reg : 0;
  a.gather_mode = sparse ? GATHER_ATTEND_ALL : GATHER_ATTEND_NRW;
  hipError_t e = launch_attend(a, s, bf);
  if (e == hipSuccess && gather) e = launch_rewrite(a, s, bf, false, true, true);
  if (e == hipSuccess) e = launch_combine(a, s);
  return e;
}

// The fused step: every stage over all units, in stream order.
hipError_t step_all(const hardkv_config *cfg, Args &a, hipStream_t s) {
  hipError_t e = hipSuccess;
  for (int stage = 0; stage < NSTAGES && e == hipSuccess; ++stage) e = step_stage(cfg, a, stage, s, true);
  return e;
}

}  // namespace
}  // namespace hardkv

using namespace hardkv;

extern "C" {

int32_t hardkv_workspace_size(const hardkv_config *cfg, size_t *bytes) {
  if (!bytes) return HARDKV_EINVAL;
  Plan p;
  int32_t rc = plan(cfg, p);
  if (rc != HARDKV_OK) return rc;
  *bytes = p.ws_bytes;
  return HARDKV_OK;
}

int32_t hardkv_prefill(const hardkv_config *cfg, hardkv_state *st, const void *k_ctx,
                       const void *v_ctx, const int64_t *ctx_len_dev, int64_t max_len, void *stream) {
  Plan p;
  int32_t rc = setup(cfg, st, p);
  if (rc != HARDKV_OK) return rc;
  if (max_len < 0 || !ctx_len_dev || ((uintptr_t)ctx_len_dev & 7u)) return HARDKV_EINVAL;
  if (max_len > 0 && (!aligned16(k_ctx) || !aligned16(v_ctx))) return HARDKV_EINVAL;
  if (max_len - cfg->dense_window + 1 - cfg->sink > (int64_t)cfg->pool_blocks * BK) return HARDKV_ECAPACITY;
  p.a.k_ctx = k_ctx;
  p.a.v_ctx = v_ctx;
  p.a.ctx_len = ctx_len_dev;
  p.a.max_len = max_len;
  return hip_status(launch_prefill(p.a, (hipStream_t)stream, is_bf16(cfg)));
}

int32_t hardkv_append(const hardkv_config *cfg, hardkv_state *st, const void *k_new,
                      const void *v_new, void *stream) {
  Plan p;
  int32_t rc = setup(cfg, st, p);
  if (rc != HARDKV_OK) return rc;
  if (!aligned16(k_new) || !aligned16(v_new)) return HARDKV_EINVAL;
  p.a.k_new = k_new;
  p.a.v_new = v_new;
  return hip_status(launch_append(p.a, (hipStream_t)stream, is_bf16(cfg)));
}

int32_t hardkv_select(const hardkv_config *cfg, hardkv_state *st, const void *q, void *stream) {
  Plan p;
  int32_t rc = setup(cfg, st, p);
  if (rc != HARDKV_OK) return rc;
  if (!aligned16(q)) return HARDKV_EINVAL;
  p.a.q = q;
  hipStream_t s = (hipStream_t)stream;
  const bool bf = is_bf16(cfg);
  hipError_t e = launch_score(p.a, s, bf);
  if (e == hipSuccess && p.a.calibration) e = launch_fit(p.a, s);
  if (e == hipSuccess) e = launch_select(p.a, s, is_bf16(cfg));
  if (e == hipSuccess && p.a.view_sum) e = launch_flatten(p.a, s);
  if (e == hipSuccess) e = launch_rewrite(p.a, s, bf, true, false, false);  // mask words
  return hip_status(e);
}

int32_t hardkv_regularize(const hardkv_config *cfg, hardkv_state *st, void *stream) {
  Plan p;
  int32_t rc = setup(cfg, st, p);
  if (rc != HARDKV_OK) return rc;
  p.a.gather_mode = GATHER_REWRITE;
  return hip_status(launch_rewrite(p.a, (hipStream_t)stream, is_bf16(cfg), false, true, false));
}

int32_t hardkv_condense(const hardkv_config *cfg, hardkv_state *st, void *stream) {
  Plan p;
  int32_t rc = setup(cfg, st, p);
  if (rc != HARDKV_OK) return rc;
  return hip_status(launch_condense(p.a, (hipStream_t)stream, is_bf16(cfg)));
}

int32_t hardkv_attend(const hardkv_config *cfg, hardkv_state *st, const void *q, float *out,
                      void *stream) {
  Plan p;
  int32_t rc = setup(cfg, st, p);
  if (rc != HARDKV_OK) return rc;
  if (!aligned16(q) || !aligned16(out)) return HARDKV_EINVAL;
  p.a.q = q;
  p.a.out = out;
  return hip_status(attend_calls(cfg, p.a, (hipStream_t)stream, false));
}

int32_t hardkv_attend_sparse(const hardkv_config *cfg, hardkv_state *st, const void *q, float *out,
                             void *stream) {
  Plan p;
  int32_t rc = setup(cfg, st, p);
  if (rc != HARDKV_OK) return rc;
  if (!aligned16(q) || !aligned16(out)) return HARDKV_EINVAL;
  p.a.q = q;
  p.a.out = out;
  return hip_status(attend_calls(cfg, p.a, (hipStream_t)stream, true));
}

int32_t hardkv_step(const hardkv_config *cfg, hardkv_state *st, const void *q, const void *k_new,
                    const void *v_new, float *out, void *stream) {
  Plan p;
  int32_t rc = setup(cfg, st, p);
  if (rc != HARDKV_OK) return rc;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out)) return HARDKV_EINVAL;
  p.a.q = q;
  p.a.k_new = k_new;
  p.a.v_new = v_new;
  p.a.out = out;
  return hip_status(step_all(cfg, p.a, (hipStream_t)stream));
}

int32_t hardkv_step_reuse(const hardkv_config *cfg, hardkv_state *st, const void *q, const void *k_new,
                          const void *v_new, float *out, void *stream) {
  Plan p;
  int32_t rc = setup(cfg, st, p);
  if (rc != HARDKV_OK) return rc;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out)) return HARDKV_EINVAL;
  p.a.q = q;
  p.a.k_new = k_new;
  p.a.v_new = v_new;
  p.a.out = out;
  hipError_t e = launch_append(p.a, (hipStream_t)stream, is_bf16(cfg));
  if (e == hipSuccess) e = attend_calls(cfg, p.a, (hipStream_t)stream, false);
  return hip_status(e);
}

int32_t hardkv_step_noalloc(const hardkv_config *cfg, hardkv_state *st, const void *q, const void *k_new,
                            const void *v_new, float *out, void *stream) {
  Plan p;
  int32_t rc = plan(cfg, p);
  if (rc != HARDKV_OK) return rc;
  if (!st) return HARDKV_EINVAL;
  if (p.ws_bytes > (size_t)HARDKV_STATIC_SCRATCH_BYTES) return HARDKV_ESCRATCH;
  // (a destructive selection reads the last selection's plan, which the shared scratch does
  // not keep)
  if (p.a.destructive) return HARDKV_EUNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out)) return HARDKV_EINVAL;
  // the state's own buffers, with the library's scratch in place of its workspace; the
  // pointer checks of bind() run on a stand-in address first, so that a bad state is
  // rejected before the array's address is looked up
  hardkv_state sc = *st;
  sc.workspace = reinterpret_cast<void *>((uintptr_t)256);
  sc.workspace_bytes = HARDKV_STATIC_SCRATCH_BYTES;
  rc = bind(&sc, p);
  if (rc != HARDKV_OK) return rc;
  void *ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != HARDKV_OK) return rc;
  sc.workspace = ws;
  rc = bind(&sc, p);
  if (rc != HARDKV_OK) return rc;
  p.a.kx_unknown = 1;
  p.a.q = q;
  p.a.k_new = k_new;
  p.a.v_new = v_new;
  p.a.out = out;
  return hip_status(step_all(cfg, p.a, (hipStream_t)stream));
}

// The pipeline's two states: the buffers that hold the cache itself are shared, those a
// selection writes are not.
int32_t check_pipeline_pair(const hardkv_state *nx, const hardkv_state *cur) {
  if (!nx || !cur) return HARDKV_EINVAL;
  const void *shared[][2] = {{nx->dense_k, cur->dense_k}, {nx->dense_v, cur->dense_v}, {nx->pool_k, cur->pool_k},
                             {nx->pool_v, cur->pool_v}, {nx->cond_kn, cur->cond_kn}, {nx->cond_vn, cur->cond_vn},
                             {nx->cond_omega, cur->cond_omega}, {nx->cond_n, cur->cond_n},
                             {nx->cond_cursor, cur->cond_cursor}, {nx->seq_len, cur->seq_len},
                             {nx->pool_head, cur->pool_head}, {nx->sink_k, cur->sink_k}, {nx->sink_v, cur->sink_v},
                             {nx->block_table, cur->block_table}, {nx->free_list, cur->free_list},
                             {nx->free_top, cur->free_top}};
  for (auto &pr : shared)
    if (pr[0] != pr[1]) return HARDKV_EINVAL;
  const void *own[][2] = {{nx->view_k, cur->view_k}, {nx->view_v, cur->view_v}, {nx->view_pos, cur->view_pos},
                          {nx->scores, cur->scores}, {nx->weights, cur->weights}, {nx->mask, cur->mask},
                          {nx->budget, cur->budget}, {nx->n_condense, cur->n_condense}, {nx->w_all, cur->w_all},
                          {nx->w_u, cur->w_u}, {nx->thresh, cur->thresh}, {nx->workspace, cur->workspace}};
  for (auto &pr : own)
    if (pr[0] == pr[1]) return HARDKV_EINVAL;
  if (nx->regularized && nx->regularized == cur->regularized) return HARDKV_EINVAL;
  if (nx->tau_fit && nx->tau_fit == cur->tau_fit) return HARDKV_EINVAL;
  return HARDKV_OK;
}

int32_t hardkv_select_fork(const hardkv_config *cfg, hardkv_state *st_next, const hardkv_state *st_cur,
                           void *stream) {
  Plan p, pc;
  int32_t rc = setup(cfg, st_next, p);
  if (rc != HARDKV_OK) return rc;
  rc = setup(cfg, st_cur, pc);
  if (rc != HARDKV_OK) return rc;
  rc = check_pipeline_pair(st_next, st_cur);
  if (rc != HARDKV_OK) return rc;
  if (p.a.destructive) return HARDKV_EUNSUPPORTED;
  p.a.kx_src = pc.a.kx;
  return hip_status(launch_fork(p.a, (hipStream_t)stream));
}

int32_t hardkv_select_ahead(const hardkv_config *cfg, hardkv_state *st_next, const void *q, int32_t unit_begin,
                            int32_t unit_count, void *stream) {
  Plan p;
  int32_t rc = setup(cfg, st_next, p);
  if (rc != HARDKV_OK) return rc;
  if (p.a.view_sum || p.a.destructive) return HARDKV_EUNSUPPORTED;
  if (!aligned16(q)) return HARDKV_EINVAL;
  if (unit_begin < 0 || unit_count < 0 || (int64_t)unit_begin + unit_count > (int64_t)p.a.B * p.a.Hkv)
    return HARDKV_EINVAL;
  if (unit_count == 0) return HARDKV_OK;
  p.a.bh0 = unit_begin;  // every kernel below covers units [bh0, bh0 + nbh)
  p.a.nbh = unit_count;
  p.a.q = q;
  p.a.seq_len = p.a.tsnap;  // the pool as it stood at the forked step
  p.a.gather_mode = GATHER_REWRITE;
  hipStream_t s = (hipStream_t)stream;
  const bool bf = is_bf16(cfg);
  hipError_t e = launch_score(p.a, s, bf);
  if (e == hipSuccess && p.a.calibration) e = launch_fit(p.a, s);
  if (e == hipSuccess) e = launch_select(p.a, s, bf);
  if (e == hipSuccess) e = launch_rewrite(p.a, s, bf, true, true, false);  // mask words and views
  return hip_status(e);
}

int32_t hardkv_step_stage(const hardkv_config *cfg, hardkv_state *st, const void *q,
                          const void *k_new, const void *v_new, float *out, int32_t stage,
                          void *stream) {
  Plan p;
  int32_t rc = setup(cfg, st, p);
  if (rc != HARDKV_OK) return rc;
  if (stage < 0 || stage >= NSTAGES) return HARDKV_EINVAL;
  if (stage == 0 && (!aligned16(k_new) || !aligned16(v_new))) return HARDKV_EINVAL;
  if ((stage == 1 || stage == 4) && !aligned16(q)) return HARDKV_EINVAL;
  if (stage == 5 && !aligned16(out)) return HARDKV_EINVAL;
  p.a.q = q;
  p.a.k_new = k_new;
  p.a.v_new = v_new;
  p.a.out = out;
  return hip_status(step_stage(cfg, p.a, stage, (hipStream_t)stream, false));
}

int32_t hardkv_step_num_stages(void) { return NSTAGES; }

const char *hardkv_step_stage_name(int32_t stage) {
  return (stage >= 0 && stage < NSTAGES) ? kStageNames[stage] : "unknown";
}

int32_t hardkv_mti_thresholds(const hardkv_config *cfg, int64_t n_survivors, int32_t *l_lower,
                              int32_t *l_upper) {
  if (!cfg || !l_lower || !l_upper || !mti_config_ok(cfg)) return HARDKV_EINVAL;
  if (n_survivors < 0 || n_survivors >= (1 << 20)) return HARDKV_EINVAL;
  // the policy's choice at every budget, smallest and largest rewritten
  int32_t lo = 0, hi = -1;
  for (int64_t k = 1; k <= n_survivors; ++k)
    if (mti_rewrites_cfg(cfg, cfg->mti_horizon, k, n_survivors)) {
      if (lo == 0) lo = (int32_t)k;
      hi = (int32_t)k;
    }
  *l_lower = lo;
  *l_upper = hi;
  return HARDKV_OK;
}

int32_t hardkv_shared_pool_blocks(const hardkv_config *cfg, const int64_t *ctx_len, int64_t steps,
                                  int64_t *blocks) {
  Plan p;
  if (!cfg || !ctx_len || !blocks || steps < 0 || steps > ((int64_t)1 << 40)) return HARDKV_EINVAL;
  const int32_t rc = plan(cfg, p);
  if (rc != HARDKV_OK) return rc;
  int64_t total = 0;
  for (int b = 0; b < cfg->batch; ++b) {
    if (ctx_len[b] < 0 || ctx_len[b] > ((int64_t)1 << 40)) return HARDKV_EINVAL;
    const int64_t t = ctx_len[b] + steps;
    const int64_t pend = t - cfg->dense_window > cfg->sink ? t - cfg->dense_window : (int64_t)cfg->sink;
    const int64_t need = pend > cfg->sink ? (pend + BK - 1) / BK - cfg->sink / BK : 0;
    total += std::min<int64_t>(need, cfg->pool_blocks) * cfg->num_kv_heads;
  }
  *blocks = total;
  return HARDKV_OK;
}

int32_t hardkv_mti_period(const hardkv_config *cfg, int64_t n_pool, int64_t n_survivors, int64_t kstar,
                          int32_t max_period, int32_t *period) {
  if (!cfg || !period || !mti_config_ok(cfg)) return HARDKV_EINVAL;
  if (n_pool < 0 || n_pool >= (1 << 20) || n_survivors < 0 || n_survivors > n_pool || kstar < 0 ||
      kstar > n_survivors || max_period < 1 || max_period > HARDKV_MTI_MAX_HORIZON + 1)
    return HARDKV_EINVAL;
  // memory time of one period of R steps: the score, the cheaper policy at H = R - 1, and the
  // rows that arrived since the selection (1 + 2 + ... + (R - 1) of them), in 128 bits
  typedef unsigned __int128 u128;
  const int64_t b = n_survivors > 0 ? std::min<int64_t>(8, (8 * kstar) / n_survivors) : 0;
  const u128 per_gather = (u128)kstar * cfg->mti_c_gather[b] + (u128)n_survivors * cfg->mti_c_scan;
  auto cost = [&](int64_t R) -> u128 {
    const u128 H = (u128)(R - 1);
    const u128 sparse = (H + 1) * per_gather;
    const u128 rewrite = per_gather + (u128)kstar * cfg->mti_c_write +
                         H * (u128)kstar * ((u128)cfg->mti_c_view + cfg->mti_c_hold) + (u128)cfg->mti_fixed;
    const u128 pol = mti_rewrites_cfg(cfg, R - 1, kstar, n_survivors) ? rewrite : sparse;
    return (u128)n_pool * cfg->mti_c_score + pol + (u128)cfg->mti_c_view * (H * (H + 1) / 2);
  };
  int64_t best = 1;
  u128 best_cost = cost(1);
  for (int64_t R = 2; R <= max_period; ++R) {
    const u128 c = cost(R);
    if (c * (u128)best < best_cost * (u128)R) {  // c / R < best_cost / best
      best = R;
      best_cost = c;
    }
  }
  *period = (int32_t)best;
  return HARDKV_OK;
}

const char *hardkv_strerror(int32_t code) {
  switch (code) {
    case HARDKV_OK: return "ok";
    case HARDKV_EINVAL: return "invalid argument";
    case HARDKV_EUNSUPPORTED: return "unsupported configuration";
    case HARDKV_ECAPACITY: return "capacity too small";
    case HARDKV_EHIP: return "HIP launch failed";
    case HARDKV_ESCRATCH: return "scratch needed exceeds the library's static scratch";
    default: return "unknown status";
  }
}

}  // extern "C"
