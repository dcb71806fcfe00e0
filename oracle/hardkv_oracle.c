/* hardkv_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain CPU definition of one HARD-KV decode step, written from the HARD-KV
 * explainer pages ("HARD-KV: Head-Adaptive Regularization for Decoding-time KV
 * Compression", technical summary section 2).  Every step is a scalar loop in
 * the order the definition states; only qsort (for the ranking) is a library
 * primitive.  Float work that must match the GPU bit for bit is done in single
 * precision with one rounding per operation (build with -ffp-contract=off,
 * never -ffast-math); attention and the condensed sums are done in binary64.
 *
 * Points the pages leave open are settled by the readings listed in the
 * design notes (per-step view over a fixed pool, max over the GQA group of the
 * current queries, tau-scaled softmax calibration with integer weights, top-p
 * with ties to the lower position, one condensed slot per merged block, a
 * ln(n) logit bias for merged slots).
 */
#include "hardkv_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define BK 64
#define ORC_LOG2E 1.4426950408889634074 /* binary64 nearest log2(e) */

/* ------------------------------------------------------------------------------------
 * storage elements
 * ---------------------------------------------------------------------------------- */
static float elem_get(const void *base, int64_t i, int eb) {
  if (eb == 4) return ((const float *)base)[i];
  uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16; /* bf16 widens exactly */
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static void row_copy(void *dst, int64_t drow, const void *src, int64_t srow, int D, int eb) {
  memcpy((char *)dst + drow * D * eb, (const char *)src + srow * D * eb, (size_t)D * eb);
}

/* ------------------------------------------------------------------------------------
 * System-aware index regularization (section 2.C): the trade-off between Rewrite Cache and
 * Sparse Loading is weighed by a memory-time integral, switched by budget thresholds
 * L_lower and L_upper.  Reading: the memory time a head's kept rows cost over a horizon of
 * the selection step and the H later steps that reuse it, in femtoseconds,
 *   Sparse Loading: every one of the H + 1 steps gathers the k* kept rows through the
 *     mask, g(b) each (b = floor(8 k* / n), the kept eighth of the n survivors), and walks
 *     the mask over the n survivors, c_scan each;
 *   Rewrite Cache: the selection step gathers them and writes the view, c_write each;
 *     each later step reads them from the view, c_view each, while the view holds them,
 *     c_hold per row and step; plus a fixed F per rewritten head.
 * The head is rewritten iff the rewrite's integral is the smaller one.  The selection
 * step's gather appears on both sides and cancels; what remains is compared exactly in
 * 64-bit integers (k*, n < 2^20, H < 2^16, costs < 2^24).
 * ---------------------------------------------------------------------------------- */
int32_t orc_mti_rewrite(const orc_cfg *cfg, int64_t kstar, int64_t n) {
  if (kstar <= 0 || n <= 0) return 0;
  int64_t b = (8 * kstar) / n;
  if (b > 8) b = 8;
  const int64_t H = cfg->mti_horizon;
  const int64_t g = cfg->mti_c_gather[b];
  /* sparse: (H + 1) (k g + n c_scan);  rewrite: k g + n c_scan + k c_write
   * + H k (c_view + c_hold) + F */
  const int64_t rewrite_extra = kstar * (int64_t)cfg->mti_c_write +
                                H * kstar * ((int64_t)cfg->mti_c_view + (int64_t)cfg->mti_c_hold) + cfg->mti_fixed;
  const int64_t sparse_extra = H * (kstar * g + n * (int64_t)cfg->mti_c_scan);
  return rewrite_extra < sparse_extra ? 1 : 0;
}

void orc_mti_thresholds(const orc_cfg *cfg, int64_t n, int64_t *lo, int64_t *hi) {
  *lo = 0;
  *hi = -1;
  for (int64_t k = 1; k <= n; ++k)
    if (orc_mti_rewrite(cfg, k, n)) {
      if (*lo == 0) *lo = k;
      *hi = k;
    }
}

/* Steps per selection (a reading of when to select again, by the same integral): a head
 * that selects every R steps pays, per period, the score over its n_pool pool rows
 * (c_score each), the cheaper of the two policies above for H = R - 1, and, at the j-th
 * step after the selection, the j pool rows that arrived since it, attended from the pool
 * (c_view each, contiguous rows).  R minimises that cost over R (the smallest R on ties),
 * compared exactly as cost(R1) R2 against cost(R2) R1. */
static unsigned __int128 mti_period_cost(const orc_cfg *cfg, int64_t n_pool, int64_t n, int64_t k, int64_t R) {
  orc_cfg c2 = *cfg;
  c2.mti_horizon = (int32_t)(R - 1);
  int64_t b = n > 0 ? (8 * k) / n : 0;
  if (b > 8) b = 8;
  const unsigned __int128 H = (unsigned __int128)(R - 1);
  const unsigned __int128 kk = (unsigned __int128)k, nn = (unsigned __int128)n;
  const unsigned __int128 sparse = (H + 1) * (kk * cfg->mti_c_gather[b] + nn * cfg->mti_c_scan);
  const unsigned __int128 rewrite = kk * cfg->mti_c_gather[b] + nn * cfg->mti_c_scan + kk * cfg->mti_c_write +
                                    H * kk * ((unsigned __int128)cfg->mti_c_view + cfg->mti_c_hold) +
                                    (unsigned __int128)cfg->mti_fixed;
  const unsigned __int128 policy = orc_mti_rewrite(&c2, k, n) ? rewrite : sparse;
  const unsigned __int128 tail = (unsigned __int128)cfg->mti_c_view * (H * (H + 1) / 2);
  return (unsigned __int128)n_pool * cfg->mti_c_score + policy + tail;
}

int32_t orc_mti_period(const orc_cfg *cfg, int64_t n_pool, int64_t n, int64_t kstar, int32_t max_period) {
  if (max_period < 1) return 0;
  int64_t best = 1;
  unsigned __int128 best_cost = mti_period_cost(cfg, n_pool, n, kstar, 1);
  for (int64_t R = 2; R <= max_period; ++R) {
    const unsigned __int128 cst = mti_period_cost(cfg, n_pool, n, kstar, R);
    if (cst * (unsigned __int128)best < best_cost * (unsigned __int128)R) {
      best = R;
      best_cost = cst;
    }
  }
  return (int32_t)best;
}

/* whether head u keeps a rewritten view this selection (the regularize policy) */
static int head_rewritten(const orc_cfg *cfg, int64_t kstar, int64_t n_survivors) {
  switch (cfg->regularize) {
    case 0: return 1;
    case 1: return 0;
    case 2: return (kstar >= cfg->mti_lower && kstar <= cfg->mti_upper) ? 1 : 0;
    default: return orc_mti_rewrite(cfg, kstar, n_survivors);
  }
}

/* pool ring row of position p for unit u (rows counted over the whole buffer) */
static int64_t pool_row(const orc_cfg *cfg, int64_t u, int64_t p) {
  int64_t P = cfg->pool_blocks;
  return (u * P + (p / BK) % P) * BK + p % BK;
}

/* ------------------------------------------------------------------------------------
 * Score: max-pooled logits (section 2.B names "max-pooled logits" as an importance
 * metric; the pooling runs over the GQA group of the current step's queries).
 * Each query-key logit is a dot product taken as a canonical pairwise tree:
 * products in index order, then level l+1 element i = level l [2i] + [2i+1].
 * ---------------------------------------------------------------------------------- */
/* Sink prefix (a reading of the dense tier's role of keeping attention sinks): the first S
 * positions of a sequence stay in a tier of their own, attended at every step and never
 * scored, condensed or rewritten.  The dense window then holds the W latest positions
 * after them, [max(S, t - W), t), and the pool the positions between, [c, max(S, t - W)),
 * its head c starting at S.  With S = 0 these are the plain windows. */
static int64_t pool_end_of(const orc_cfg *cfg, int64_t t) {
  const int64_t e = t - cfg->dense_window;
  return e > cfg->sink ? e : cfg->sink;
}
static int64_t dense_lo_of(const orc_cfg *cfg, int64_t t) {
  const int64_t lo = pool_end_of(cfg, t);
  return lo < t ? lo : t;
}

float orc_dot_pairwise(const float *a, const float *b, int32_t n) {
  float lvl[1024];
  if (n < 1 || n > 1024) return NAN; /* head dims up to 1024 */
  for (int i = 0; i < n; ++i) {
    float p = a[i] * b[i];
    lvl[i] = p;
  }
  for (int m = n; m > 1; m /= 2) {
    for (int i = 0; i < m / 2; ++i) {
      float s = lvl[2 * i] + lvl[2 * i + 1];
      lvl[i] = s;
    }
  }
  return lvl[0];
}

float orc_score_row(const float *q, int32_t G, const float *k, int32_t D) {
  float s = orc_dot_pairwise(q, k, D);
  for (int g = 1; g < G; ++g) {
    float d = orc_dot_pairwise(q + (int64_t)g * D, k, D);
    if (d > s) s = d;
  }
  return s + 0.0f; /* a zero score is +0 whatever the signs of the group's zeros */
}

/* ------------------------------------------------------------------------------------
 * Logits Calibration (section 2.B): the scores are mapped to one softmax by a
 * temperature, softmax(s / (sqrt(D) tau)), evaluated in base 2 with
 * kappa = log2(e) / (sqrt(D) tau).  Probabilities are carried as integer
 * weights w = max(1, floor(2^24 * 2^((s - m) kappa))), so masses add exactly.
 * 2^t uses t = n + f with n = floor(t) and f = t - n in [0, 1), and the degree-9
 * Taylor polynomial of 2^f = sum (f ln 2)^i / i! in Horner form.  With f >= 0
 * every Horner step multiplies and adds non-negative numbers, so each rounding
 * is monotone and 2^t, hence w, never decreases as the score grows: the
 * calibration keeps the order of the scores.
 * ---------------------------------------------------------------------------------- */
#define ORC_NCOEFF 10
static float g_coeff[ORC_NCOEFF];

__attribute__((constructor)) static void init_coeffs(void) {
  const long double ln2 = 0.693147180559945309417232121458176568L;
  long double v = 1.0L;
  for (int i = 0; i < ORC_NCOEFF; ++i) {
    if (i > 0) v = v * ln2 / (long double)i;
    g_coeff[i] = (float)v;
  }
}

float orc_poly_coeff(int32_t i) { return (i >= 0 && i < ORC_NCOEFF) ? g_coeff[i] : 0.0f; }

float orc_kappa(int32_t D, float tau) {
  return (float)(ORC_LOG2E / (sqrt((double)D) * (double)tau));
}

/* ------------------------------------------------------------------------------------
 * Calibration temperature fitted by entropy (section 2.B says the scores are calibrated
 * by the temperature of the attention scores; one reading of "the temperature of the
 * attention": the calibrated softmax of the max-pooled scores gets the mean entropy of
 * the group's raw attention over the same tokens).  Entropy grows with the temperature,
 * so a bracket search on log2 tau finds it: five rounds of a 17-point grid on [-12, 12].
 * ---------------------------------------------------------------------------------- */
double orc_calibrated_entropy(const float *s, int64_t n, int32_t D, double tau) {
  if (n <= 0) return 0.0;
  float m = s[0];
  for (int64_t j = 1; j < n; ++j)
    if (s[j] > m) m = s[j];
  const double c = 1.0 / (sqrt((double)D) * tau);
  double Z = 0.0, A = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    double x = ((double)s[j] - (double)m) * c;
    double e = exp(x);
    Z += e;
    A += e * x;
  }
  return log(Z) - A / Z;
}

static double raw_entropy(const float *d, int64_t n, int32_t D) {
  const double r = 1.0 / sqrt((double)D);
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j)
    if ((double)d[j] * r > m) m = (double)d[j] * r;
  double Z = 0.0, A = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    double x = (double)d[j] * r - m;
    double e = exp(x);
    Z += e;
    A += e * x;
  }
  return log(Z) - A / Z;
}

float orc_fit_tau(const float *d, int32_t G, const float *s, int64_t n, int32_t D, double *h_target) {
  double H = 0.0;
  for (int g = 0; g < G; ++g) H += raw_entropy(d + (int64_t)g * n, n, D);
  H /= (double)G;
  if (h_target) *h_target = H;
  if (n <= 0) return 1.0f;
  double lo = -12.0, hi = 12.0;
  for (int round = 0; round < 5; ++round) {
    const double step = (hi - lo) / 16.0;
    int k = 0;
    while (k <= 16 && orc_calibrated_entropy(s, n, D, exp2(lo + k * step)) < H) ++k;
    if (k == 0) {
      hi = lo;
    } else if (k > 16) {
      lo = hi;
    } else {
      const double a = lo + (k - 1) * step, b = lo + k * step;
      lo = a;
      hi = b;
    }
  }
  return (float)exp2(0.5 * (lo + hi));
}

float orc_exp2_poly(float f) {
  float y = g_coeff[ORC_NCOEFF - 1];
  for (int i = ORC_NCOEFF - 2; i >= 0; --i) {
    float p = y * f;
    y = p + g_coeff[i];
  }
  return y;
}

void orc_exp2_poly_batch(const float *f, float *y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_exp2_poly(f[i]);
}

static uint32_t weight_from_t(float t) {
  if (!(t >= -60.0f)) return 1u;
  float n = floorf(t);
  float f = t - n; /* in [0, 1); rounded only when n = -1 */
  float y = orc_exp2_poly(f);
  float e = ldexpf(y, (int)n);
  float big = e * 16777216.0f; /* exact: scaling by 2^24 */
  uint32_t w = (uint32_t)floorf(big);
  return w < 1u ? 1u : w;
}

uint32_t orc_weight(float s, float m, float kappa) {
  float x = s - m;
  float t = x * kappa;
  return weight_from_t(t);
}

void orc_weight_batch(const float *t, uint32_t *w, int64_t n) {
  for (int64_t i = 0; i < n; ++i) w[i] = weight_from_t(t[i]);
}

/* ------------------------------------------------------------------------------------
 * Calibrated Top-p (section 2.A, tier 2; section 2.B): keep the smallest set of
 * survivors, taken in order of decreasing weight (lower position first on
 * ties), whose mass reaches T = ceil(p_q W_U / 2^16), p_q = rne(p 2^16).
 * ---------------------------------------------------------------------------------- */
uint32_t orc_pq(double p) { return (uint32_t)rint(p * 65536.0); }

typedef struct {
  uint32_t w;
  int32_t idx;
  int64_t pos;
} wp_t;

static int cmp_wp(const void *pa, const void *pb) {
  const wp_t *a = (const wp_t *)pa, *b = (const wp_t *)pb;
  if (a->w != b->w) return a->w > b->w ? -1 : 1;
  if (a->pos != b->pos) return a->pos < b->pos ? -1 : 1;
  return 0;
}

int32_t orc_topp(const uint32_t *w, const int64_t *pos, int32_t n, uint32_t pq, uint8_t *selected,
                 uint64_t *thresh_out) {
  if (thresh_out) *thresh_out = 0;
  if (n <= 0) return 0;
  uint64_t wu = 0;
  for (int32_t i = 0; i < n; ++i) wu += w[i];
  uint64_t T = ((uint64_t)pq * wu + 65535u) / 65536u;
  if (thresh_out) *thresh_out = T;
  memset(selected, 0, (size_t)n);
  wp_t *arr = (wp_t *)malloc(sizeof(wp_t) * (size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    arr[i].w = w[i];
    arr[i].idx = i;
    arr[i].pos = pos[i];
  }
  qsort(arr, (size_t)n, sizeof(wp_t), cmp_wp);
  uint64_t acc = 0;
  int32_t k = 0;
  while (acc < T) {
    acc += arr[k].w;
    selected[arr[k].idx] = 1;
    ++k;
  }
  free(arr);
  return k;
}

/* ------------------------------------------------------------------------------------
 * Attention over a list of rows, binary64.  logit_i = (q . key_i) / sqrt(D) + bias_i,
 * out = sum softmax(logit)_i value_i.  Shared by the tiered attention and the
 * full-attention reference so that the two agree bit for bit on the same rows.
 * ---------------------------------------------------------------------------------- */
typedef void (*row_fn)(const void *ctx, int64_t i, double *key, double *val, double *bias,
                       int *has_bias);

static void attend_core(const double *qd, int D, int64_t n, row_fn get, const void *ctx,
                        double *out) {
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (n == 0) return;
  double *logit = (double *)malloc(sizeof(double) * (size_t)n);
  double *key = (double *)malloc(sizeof(double) * (size_t)D);
  double *val = (double *)malloc(sizeof(double) * (size_t)D);
  double sq = sqrt((double)D);
  double mx = -INFINITY;
  for (int64_t i = 0; i < n; ++i) {
    double bias = 0.0;
    int hb = 0;
    get(ctx, i, key, val, &bias, &hb);
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += qd[d] * key[d];
    double l = dot / sq;
    if (hb) l = l + bias;
    logit[i] = l;
    if (l > mx) mx = l;
  }
  double sum = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double bias = 0.0;
    int hb = 0;
    get(ctx, i, key, val, &bias, &hb);
    double e = exp(logit[i] - mx);
    sum += e;
    for (int d = 0; d < D; ++d) out[d] += e * val[d];
  }
  for (int d = 0; d < D; ++d) out[d] /= sum;
  free(logit);
  free(key);
  free(val);
}

typedef struct {
  const float *k, *v;
  int D;
} flat_ctx;

static void flat_row(const void *ctx, int64_t i, double *key, double *val, double *bias, int *hb) {
  const flat_ctx *c = (const flat_ctx *)ctx;
  for (int d = 0; d < c->D; ++d) {
    key[d] = (double)c->k[i * c->D + d];
    val[d] = (double)c->v[i * c->D + d];
  }
  *bias = 0.0;
  *hb = 0;
}

void orc_full_attention(const float *q, const float *k, const float *v, int32_t n, int32_t D,
                        double *out) {
  double qd[1024];
  for (int d = 0; d < D; ++d) qd[d] = (double)q[d];
  flat_ctx c = {k, v, D};
  attend_core(qd, D, n, flat_row, &c, out);
}

/* the tiers of one unit, in attention order: sink positions (p < min(S, t)), condensed
 * slots with n > 0, view rows r < k*, pool positions that arrived after the last
 * selection (steps without selection only), dense positions ascending (section 2.A:
 * condensed, sparse, dense tiers) */
typedef struct {
  const orc_cfg *cfg;
  const orc_state *st;
  int64_t u;
  int64_t n_sink, n_cond, n_view, n_tail, tail_lo, n_dense, dense_lo;
  const int64_t *kept_rows;  /* pool rows of the kept positions, ascending; NULL: the view */
  int32_t slot[4096];
} tier_ctx;

static void tier_row(const void *ctx, int64_t i, double *key, double *val, double *bias,
                     int *hb) {
  const tier_ctx *tc = (const tier_ctx *)ctx;
  const orc_cfg *cfg = tc->cfg;
  const orc_state *st = tc->st;
  int D = cfg->head_dim, eb = cfg->elem_bytes;
  if (i < tc->n_sink) {
    const int64_t row = tc->u * cfg->sink + i;
    for (int d = 0; d < D; ++d) {
      key[d] = (double)elem_get(st->sink_k, row * D + d, eb);
      val[d] = (double)elem_get(st->sink_v, row * D + d, eb);
    }
    *bias = 0.0;
    *hb = 0;
    return;
  }
  i -= tc->n_sink;
  if (i < tc->n_cond) {
    int64_t s = tc->u * cfg->condensed_slots + tc->slot[i];
    double om = st->cond_omega[s];
    for (int d = 0; d < D; ++d) {
      key[d] = st->cond_kn[s * D + d] / om;
      val[d] = st->cond_vn[s * D + d] / om;
    }
    *bias = log((double)st->cond_n[s]);
    *hb = cfg->merge_bias;
    return;
  }
  i -= tc->n_cond;
  int64_t row;
  const void *kb, *vb;
  if (i < tc->n_view && tc->kept_rows) {  /* Sparse Loading: the kept rows in the pool */
    row = tc->kept_rows[i];
    kb = st->pool_k;
    vb = st->pool_v;
  } else if (i < tc->n_view) {
    row = tc->u * cfg->view_cap + i;
    kb = st->view_k;
    vb = st->view_v;
  } else if (i < tc->n_view + tc->n_tail) {
    row = pool_row(cfg, tc->u, tc->tail_lo + (i - tc->n_view));
    kb = st->pool_k;
    vb = st->pool_v;
  } else {
    int64_t p = tc->dense_lo + (i - tc->n_view - tc->n_tail);
    row = tc->u * cfg->dense_window + p % cfg->dense_window;
    kb = st->dense_k;
    vb = st->dense_v;
  }
  for (int d = 0; d < D; ++d) {
    key[d] = (double)elem_get(kb, row * D + d, eb);
    val[d] = (double)elem_get(vb, row * D + d, eb);
  }
  *bias = 0.0;
  *hb = 0;
}

/* ------------------------------------------------------------------------------------
 * Prefill: the cascade cache of a context of L tokens with nothing condensed yet.
 * The last min(L, W) positions sit in the dense ring, [0, L - W) in the pool.
 * ---------------------------------------------------------------------------------- */
int32_t orc_prefill(const orc_cfg *cfg, orc_state *st, const void *k_ctx, const void *v_ctx,
                    const int64_t *ctx_len, int64_t max_len) {
  int B = cfg->batch, H = cfg->num_kv_heads, D = cfg->head_dim, eb = cfg->elem_bytes;
  int W = cfg->dense_window, C = cfg->condensed_slots;
  for (int b = 0; b < B; ++b) {
    int64_t L = ctx_len[b];
    if (L < 0 || L > max_len) return -1;
    if (L - W + 1 - cfg->sink > (int64_t)cfg->pool_blocks * BK) return -3;
  }
  st->error_word = 0;
  for (int b = 0; b < B; ++b) {
    int64_t L = ctx_len[b];
    st->seq_len[b] = L;
    for (int h = 0; h < H; ++h) {
      int64_t u = (int64_t)b * H + h;
      st->pool_head[u] = cfg->sink;
      st->pend_sel[u] = cfg->sink;  /* no selection yet: the whole pool is unselected */
      st->budget[u] = 0;
      if (st->regularized) st->regularized[u] = 0;
      st->cond_cursor[u] = 0;
      for (int s = 0; s < C; ++s) {
        int64_t si = u * C + s;
        st->cond_omega[si] = 0.0;
        st->cond_n[si] = 0;
        for (int d = 0; d < D; ++d) st->cond_kn[si * D + d] = st->cond_vn[si * D + d] = 0.0;
      }
      memset((char *)st->dense_k + u * W * D * eb, 0, (size_t)W * D * eb);
      memset((char *)st->dense_v + u * W * D * eb, 0, (size_t)W * D * eb);
      int64_t src0 = u * max_len;
      const int64_t S = cfg->sink;
      if (S > 0) {
        memset((char *)st->sink_k + u * S * D * eb, 0, (size_t)S * D * eb);
        memset((char *)st->sink_v + u * S * D * eb, 0, (size_t)S * D * eb);
      }
      for (int64_t p = 0; p < L && p < S; ++p) {
        row_copy(st->sink_k, u * S + p, k_ctx, src0 + p, D, eb);
        row_copy(st->sink_v, u * S + p, v_ctx, src0 + p, D, eb);
      }
      int64_t lo = dense_lo_of(cfg, L);
      for (int64_t p = lo; p < L; ++p) {
        row_copy(st->dense_k, u * W + p % W, k_ctx, src0 + p, D, eb);
        row_copy(st->dense_v, u * W + p % W, v_ctx, src0 + p, D, eb);
      }
      for (int64_t p = S; p < lo; ++p) {
        row_copy(st->pool_k, pool_row(cfg, u, p), k_ctx, src0 + p, D, eb);
        row_copy(st->pool_v, pool_row(cfg, u, p), v_ctx, src0 + p, D, eb);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------------------
 * One unit (sequence b, KV head h) of the step after the append.
 * ---------------------------------------------------------------------------------- */
/* ahead: a selection made ahead of its use (seq_len is the snapshot of the step it is made
 * for): plan, score, calibrate, top-p and regularize only; the planned condensation waits for
 * orc_condense_plan and there is no attention. */
static uint32_t unit_step(const orc_cfg *cfg, orc_state *st, int b, int h, const void *q,
                          double *out, int do_attend, int ahead) {
  const int H = cfg->num_kv_heads, Hq = cfg->num_q_heads, G = Hq / H, D = cfg->head_dim;
  const int eb = cfg->elem_bytes, P = cfg->pool_blocks;
  const int64_t u = (int64_t)b * H + h;
  uint32_t err = 0;

  const int64_t t = st->seq_len[b];
  const int64_t c = st->pool_head[u];
  const int64_t pend = pool_end_of(cfg, t);
  const int64_t N = pend - c;

  /* plan (section 2.A, tier 3): whole oldest blocks leave the pool once it holds
   * more than S_cap tokens */
  int64_t E = 0;
  if (cfg->cond_mode != ORC_COND_OFF && N > cfg->sparse_cap) E = (N - cfg->sparse_cap + BK - 1) / BK;
  const int64_t u0 = c + BK * E;

  /* queries of the group, widened */
  float *qg = (float *)malloc(sizeof(float) * (size_t)G * D);
  for (int g = 0; g < G; ++g)
    for (int d = 0; d < D; ++d) qg[g * D + d] = elem_get(q, ((int64_t)b * Hq + h * G + g) * D + d, eb);

  /* the rows still in play: all of them, or with destructive selection the rows the last
   * selection kept and the positions that arrived since it (read before this selection
   * replaces the mask) */
  const int64_t psel = st->pend_sel[u];
  uint8_t *live = (uint8_t *)malloc((size_t)(N > 0 ? N : 1));
  for (int64_t j = c; j < pend; ++j)
    live[j - c] = cfg->selection == 0 || j >= psel || ((st->mask[u * P + (j / BK) % P] >> (j % BK)) & 1u);

  /* score; the calibration's maximum is over the rows in play */
  float *krow = (float *)malloc(sizeof(float) * (size_t)D);
  float m = -INFINITY;
  for (int64_t j = c; j < pend; ++j) {
    int64_t r = pool_row(cfg, u, j);
    for (int d = 0; d < D; ++d) krow[d] = elem_get(st->pool_k, r * D + d, eb);
    float s = orc_score_row(qg, G, krow, D);
    if (!isfinite(s)) err |= ORC_ERR_NONFINITE;
    st->scores[r] = s;
    if (live[j - c] && s > m) m = s;
  }

  /* calibrate over the whole pool */
  float tau_u = cfg->tau[h];
  if (cfg->calibration == 1) {
    if (cfg->tau_unit) {
      tau_u = cfg->tau_unit[u];
    } else {
      /* every query's dot products over the pool, and the max-pooled scores in order */
      const int64_t n = pend - c;
      float *dd = (float *)malloc(sizeof(float) * (size_t)(G * (n > 0 ? n : 1)));
      float *ss = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
      for (int64_t j = c; j < pend; ++j) {
        int64_t r = pool_row(cfg, u, j);
        for (int d = 0; d < D; ++d) krow[d] = elem_get(st->pool_k, r * D + d, eb);
        for (int g = 0; g < G; ++g) dd[(int64_t)g * n + (j - c)] = orc_dot_pairwise(qg + (int64_t)g * D, krow, D);
        ss[j - c] = st->scores[r];
      }
      tau_u = orc_fit_tau(dd, G, ss, n, D, NULL);
      free(dd);
      free(ss);
    }
    if (st->tau_fit) st->tau_fit[u] = tau_u;
  }
  const float kappa = orc_kappa(D, tau_u);
  uint64_t w_all = 0, w_u = 0;
  for (int64_t j = c; j < pend; ++j) {
    int64_t r = pool_row(cfg, u, j);
    /* a dropped row weighs nothing: it is in no mass, never kept and never merged */
    uint32_t w = live[j - c] ? orc_weight(st->scores[r], m, kappa) : 0u;
    st->weights[r] = w;
    w_all += w;
    if (j >= u0) w_u += w;
  }

  /* top-p over the survivors U = [u0, pend) */
  const int32_t nU = (int32_t)(pend - u0);
  uint32_t *wU = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(nU > 0 ? nU : 1));
  int64_t *pU = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nU > 0 ? nU : 1));
  uint8_t *sel = (uint8_t *)malloc((size_t)(nU > 0 ? nU : 1));
  for (int32_t i = 0; i < nU; ++i) {
    pU[i] = u0 + i;
    wU[i] = st->weights[pool_row(cfg, u, u0 + i)];
  }
  uint64_t T = 0;
  const int32_t kstar = orc_topp(wU, pU, nU, orc_pq(cfg->top_p), sel, &T);

  for (int i = 0; i < P; ++i) st->mask[u * P + i] = 0;
  for (int32_t i = 0; i < nU; ++i)
    if (sel[i]) {
      int64_t j = u0 + i;
      st->mask[u * P + (j / BK) % P] |= (uint64_t)1 << (j % BK);
    }

  /* Index Regularization (section 2.C).  The regularize policy decides whether this
   * head's kept rows are rewritten (Rewrite Cache) or left in the pool for attention to
   * load through the mask (Sparse Loading): every head, none, the heads whose budget lies
   * in caller thresholds [L_lower, L_upper], or the memory-time controller above over the
   * nU survivors. */
  const int rw = head_rewritten(cfg, kstar, nU);
  if (st->regularized) st->regularized[u] = rw;
  /* with the packed (sum) layout the views are written after every unit's budget is
   * known (orc_step); attention reads the kept rows from the pool either way */
  const int packed = cfg->view_layout == 1;
  /* the pool rows of the kept positions, ascending (Sparse Loading reads these) */
  int64_t *kept = (int64_t *)malloc(sizeof(int64_t) * (size_t)(kstar > 0 ? kstar : 1));
  {
    int32_t r = 0;
    for (int32_t i = 0; i < nU; ++i)
      if (sel[i]) kept[r++] = pool_row(cfg, u, u0 + i);
  }
  /* Rewrite Cache with a max-length flat index: the selected rows, in ascending
   * position, become rows 0 .. k*-1 of the head's fixed-capacity view */
  if (rw && !packed) {
    int32_t r = 0;
    if (kstar > cfg->view_cap) err |= ORC_ERR_VIEW_OVERFLOW;
    for (int32_t i = 0; i < nU; ++i) {
      if (!sel[i]) continue;
      if (r < cfg->view_cap) {
        int64_t j = u0 + i;
        row_copy(st->view_k, u * cfg->view_cap + r, st->pool_k, pool_row(cfg, u, j), D, eb);
        row_copy(st->view_v, u * cfg->view_cap + r, st->pool_v, pool_row(cfg, u, j), D, eb);
        st->view_pos[u * cfg->view_cap + r] = (int32_t)j;
      }
      ++r;
    }
  }

  /* condense (section 2.A, tier 3): each of the E oldest blocks is dropped
   * (evict) or merged into the next condensed slot with weights w / W_all */
  if (cfg->cond_mode == ORC_COND_MERGE && !ahead) {
    const int C = cfg->condensed_slots;
    for (int64_t e = 0; e < E; ++e) {
      int32_t sigma = st->cond_cursor[u];
      st->cond_cursor[u] = (sigma + 1) % C;
      int64_t si = u * C + sigma;
      int32_t nlive = 0;  /* the block's rows still in play (all 64 unless dropped) */
      for (int64_t j = c + BK * e; j < c + BK * (e + 1); ++j) {
        int64_t rr = pool_row(cfg, u, j);
        if (st->weights[rr] == 0) continue;
        ++nlive;
        double om = (double)st->weights[rr] / (double)w_all;
        st->cond_omega[si] += om;
        for (int d = 0; d < D; ++d) {
          st->cond_kn[si * D + d] += om * (double)elem_get(st->pool_k, rr * D + d, eb);
          st->cond_vn[si * D + d] += om * (double)elem_get(st->pool_v, rr * D + d, eb);
        }
      }
      st->cond_n[si] += nlive;
    }
  }
  if (!ahead) st->pool_head[u] = c + BK * E;
  st->pend_sel[u] = pend;
  st->budget[u] = kstar;
  st->n_condense[u] = (int32_t)E;
  st->w_all[u] = w_all;
  st->w_u[u] = w_u;
  st->thresh[u] = T;

  /* attention over condensed, sparse (view) and dense tiers */
  if (do_attend && !ahead) {
    tier_ctx *tc = (tier_ctx *)malloc(sizeof(tier_ctx));
    tc->cfg = cfg;
    tc->st = st;
    tc->u = u;
    tc->n_cond = 0;
    for (int s = 0; s < cfg->condensed_slots && s < 4096; ++s)
      if (st->cond_n[u * cfg->condensed_slots + s] > 0) tc->slot[tc->n_cond++] = s;
    tc->kept_rows = (rw && !packed) ? NULL : kept;
    tc->n_view = (rw && !packed) ? (kstar < cfg->view_cap ? kstar : cfg->view_cap) : kstar;
    tc->n_tail = 0;
    tc->tail_lo = pend;
    tc->dense_lo = dense_lo_of(cfg, t);
    tc->n_dense = t - tc->dense_lo;
    tc->n_sink = t < cfg->sink ? t : cfg->sink;
    double qd[1024];
    for (int g = 0; g < G; ++g) {
      for (int d = 0; d < D; ++d) qd[d] = (double)qg[g * D + d];
      attend_core(qd, D, tc->n_sink + tc->n_cond + tc->n_view + tc->n_dense, tier_row, tc,
                  out + ((int64_t)b * Hq + h * G + g) * D);
    }
    free(tc);
  }
  free(qg);
  free(live);
  free(krow);
  free(wU);
  free(pU);
  free(sel);
  free(kept);
  return err;
}

/* ------------------------------------------------------------------------------------
 * The step: linear append to the dense tier (section 2.A, stage 1), then per
 * unit: plan, score, calibrate, top-p (stage 2), regularize (stage 3),
 * condense (stage 4), and attention.
 * ---------------------------------------------------------------------------------- */
/* stage 1, the linear append: the position leaving the dense window moves to the pool
 * tail (once past the sinks), the new token takes its dense slot (or its sink row) */
static uint32_t append_all(const orc_cfg *cfg, orc_state *st, const void *k_new, const void *v_new) {
  const int B = cfg->batch, H = cfg->num_kv_heads, D = cfg->head_dim, eb = cfg->elem_bytes;
  const int W = cfg->dense_window;
  uint32_t err = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t t = st->seq_len[b];
    for (int h = 0; h < H; ++h) {
      const int64_t u = (int64_t)b * H + h;
      const int64_t S = cfg->sink;
      if (t < S) { /* a sink position */
        row_copy(st->sink_k, u * S + t, k_new, u, D, eb);
        row_copy(st->sink_v, u * S + t, v_new, u, D, eb);
        continue;
      }
      if (t - W >= S) {
        const int64_t p = t - W; /* leaves the dense window, joins the pool tail */
        if (p + 1 - st->pool_head[u] > (int64_t)cfg->pool_blocks * BK) err |= ORC_ERR_POOL_OVERFLOW;
        row_copy(st->pool_k, pool_row(cfg, u, p), st->dense_k, u * W + p % W, D, eb);
        row_copy(st->pool_v, pool_row(cfg, u, p), st->dense_v, u * W + p % W, D, eb);
      }
      row_copy(st->dense_k, u * W + t % W, k_new, u, D, eb);
      row_copy(st->dense_v, u * W + t % W, v_new, u, D, eb);
    }
    st->seq_len[b] = t + 1;
  }
  return err;
}

int32_t orc_step(const orc_cfg *cfg, orc_state *st, const void *q, const void *k_new,
                 const void *v_new, double *out, int32_t do_attend, int32_t nthreads) {
  const int B = cfg->batch, H = cfg->num_kv_heads, D = cfg->head_dim, eb = cfg->elem_bytes;
  if (cfg->condensed_slots > 4096 || D > 1024) return -2;
  uint32_t err = append_all(cfg, st, k_new, v_new);
  const int64_t units = (int64_t)B * H;
#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt) reduction(| : err)
#endif
  for (int64_t i = 0; i < units; ++i) err |= unit_step(cfg, st, (int)(i / H), (int)(i % H), q, out, do_attend, 0);
  (void)nthreads;

  /* Flatten Index to the sum (section 2.C): the rewritten heads' kept rows, each head's in
   * ascending position, packed in unit order; head u starts at row view_off[u] */
  if (cfg->view_layout == 1) {
    const int P = cfg->pool_blocks;
    int64_t off = 0;
    for (int64_t u = 0; u < units; ++u) {
      const int32_t kstar = st->budget[u];
      const int64_t t = st->seq_len[u / H];
      const int64_t pend = pool_end_of(cfg, t);
      const int rw = head_rewritten(cfg, kstar, pend - st->pool_head[u]);  /* survivors */
      st->view_off[u] = (int32_t)off;
      if (!rw) continue;
      const int64_t c0 = st->pool_head[u] - (int64_t)BK * st->n_condense[u];
      int64_t r = 0;
      for (int64_t j = c0; j < pend; ++j) {
        if (!((st->mask[u * P + (j / BK) % P] >> (j % BK)) & 1u)) continue;
        if (off + r < cfg->view_total) {
          row_copy(st->view_k, off + r, st->pool_k, pool_row(cfg, u, j), D, eb);
          row_copy(st->view_v, off + r, st->pool_v, pool_row(cfg, u, j), D, eb);
          st->view_pos[off + r] = (int32_t)j;
        }
        ++r;
      }
      off += kstar;
    }
    st->view_off[units] = (int32_t)off;
    if (off > cfg->view_total) err |= ORC_ERR_VIEW_OVERFLOW;
  }
  st->error_word |= err;
  return 0;
}

/* ------------------------------------------------------------------------------------
 * A step that reuses the last selection (section 2.C: a rewritten cache stays in use for
 * later steps, its cost spread over them).  Reading: selection reruns when the caller
 * asks for it (a step with selection is orc_step); in between, each step appends, and
 * attention covers the sinks, the condensed slots, the rows the last selection kept (the
 * view of a rewritten head, else the pool rows its mask marks, which stay in place: nothing
 * is condensed without a selection), every pool position that arrived after that
 * selection, and the dense window.
 * ---------------------------------------------------------------------------------- */
static void unit_reuse(const orc_cfg *cfg, orc_state *st, int b, int h, const void *q, double *out) {
  const int H = cfg->num_kv_heads, Hq = cfg->num_q_heads, G = Hq / H, D = cfg->head_dim;
  const int eb = cfg->elem_bytes, P = cfg->pool_blocks;
  const int64_t u = (int64_t)b * H + h;
  const int64_t t = st->seq_len[b];
  const int64_t c = st->pool_head[u];
  const int64_t psel = st->pend_sel[u];
  const int64_t pend = pool_end_of(cfg, t);
  const int32_t kstar = st->budget[u];
  /* survivors of the last selection: [pool head, its pool end) (nothing condenses since) */
  const int rw = st->regularized ? st->regularized[u] : head_rewritten(cfg, kstar, psel - c);
  const int packed = cfg->view_layout == 1;
  int64_t *kept = (int64_t *)malloc(sizeof(int64_t) * (size_t)(kstar > 0 ? kstar : 1));
  int64_t nk = 0;
  for (int64_t j = c; j < psel && nk < kstar; ++j)
    if ((st->mask[u * P + (j / BK) % P] >> (j % BK)) & 1u) kept[nk++] = pool_row(cfg, u, j);
  tier_ctx *tc = (tier_ctx *)malloc(sizeof(tier_ctx));
  tc->cfg = cfg;
  tc->st = st;
  tc->u = u;
  tc->n_cond = 0;
  for (int s = 0; s < cfg->condensed_slots && s < 4096; ++s)
    if (st->cond_n[u * cfg->condensed_slots + s] > 0) tc->slot[tc->n_cond++] = s;
  tc->kept_rows = (rw && !packed) ? NULL : kept;
  tc->n_view = (rw && !packed) ? (kstar < cfg->view_cap ? kstar : cfg->view_cap) : nk;
  tc->tail_lo = psel;
  tc->n_tail = pend > psel ? pend - psel : 0;
  tc->dense_lo = dense_lo_of(cfg, t);
  tc->n_dense = t - tc->dense_lo;
  tc->n_sink = t < cfg->sink ? t : cfg->sink;
  double qd[1024];
  for (int g = 0; g < G; ++g) {
    for (int d = 0; d < D; ++d) qd[d] = (double)elem_get(q, ((int64_t)b * Hq + h * G + g) * D + d, eb);
    attend_core(qd, D, tc->n_sink + tc->n_cond + tc->n_view + tc->n_tail + tc->n_dense, tier_row, tc,
                out + ((int64_t)b * Hq + h * G + g) * D);
  }
  free(tc);
  free(kept);
}

int32_t orc_step_reuse(const orc_cfg *cfg, orc_state *st, const void *q, const void *k_new,
                       const void *v_new, double *out, int32_t nthreads) {
  const int B = cfg->batch, H = cfg->num_kv_heads, D = cfg->head_dim;
  if (cfg->condensed_slots > 4096 || D > 1024) return -2;
  uint32_t err = append_all(cfg, st, k_new, v_new);
  const int64_t units = (int64_t)B * H;
#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
  for (int64_t i = 0; i < units; ++i) unit_reuse(cfg, st, (int)(i / H), (int)(i % H), q, out);
  (void)nthreads;
  st->error_word |= err;
  return 0;
}

/* ------------------------------------------------------------------------------------
 * The asynchronous pipeline of the four stages (section 2.A names it; reading: with a
 * selection reused over later steps, the next one can be made on the side while decode
 * steps continue on the current one, and switched in at a later step).  A selection made
 * ahead runs plan, score, calibrate, top-p and regularize over the pool as it stood after
 * the append of step t_snap (seq_len holds that snapshot here; the pool head is the live
 * one, which only a condensation moves), into a state of its own that shares the pool,
 * the dense and sink rows and the condensed tier; its condensation is applied at the
 * switch, with its own weights and mass, by orc_condense_plan.
 * ---------------------------------------------------------------------------------- */
int32_t orc_select_ahead(const orc_cfg *cfg, orc_state *st, const void *q) {
  const int B = cfg->batch, H = cfg->num_kv_heads;
  uint32_t err = 0;
  if (cfg->view_layout == 1) return -2; /* packed views are written by orc_step only */
  if (cfg->selection != 0) return -2;   /* a selection ahead of its use keeps views only */
  for (int64_t i = 0; i < (int64_t)B * H; ++i) err |= unit_step(cfg, st, (int)(i / H), (int)(i % H), q, NULL, 0, 1);
  st->error_word |= err;
  return 0;
}

int32_t orc_condense_plan(const orc_cfg *cfg, orc_state *st) {
  const int B = cfg->batch, H = cfg->num_kv_heads, D = cfg->head_dim, eb = cfg->elem_bytes;
  const int C = cfg->condensed_slots;
  for (int64_t u = 0; u < (int64_t)B * H; ++u) {
    const int64_t c = st->pool_head[u], E = st->n_condense[u];
    const uint64_t w_all = st->w_all[u];
    if (cfg->cond_mode == ORC_COND_MERGE) {
      for (int64_t e = 0; e < E; ++e) {
        int32_t sigma = st->cond_cursor[u];
        st->cond_cursor[u] = (sigma + 1) % C;
        int64_t si = u * C + sigma;
        for (int64_t j = c + BK * e; j < c + BK * (e + 1); ++j) {
          int64_t rr = pool_row(cfg, u, j);
          double om = (double)st->weights[rr] / (double)w_all;
          st->cond_omega[si] += om;
          for (int d = 0; d < D; ++d) {
            st->cond_kn[si * D + d] += om * (double)elem_get(st->pool_k, rr * D + d, eb);
            st->cond_vn[si * D + d] += om * (double)elem_get(st->pool_v, rr * D + d, eb);
          }
        }
        st->cond_n[si] += BK;
      }
    }
    st->pool_head[u] = c + BK * E;
  }
  return 0;
}
