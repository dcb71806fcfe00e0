/* hardkv_oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU definition of one decode step of HARD-KV ("HARD-KV:
 * Head-Adaptive Regularization for Decoding-time KV Compression", technical
 * summary, section 2: Cascade Cache Hierarchy, Logits Calibration Mechanism,
 * System-Aware Index Regularization).  Only the tests, the smoke check and the
 * benchmark's CPU baseline may load this library; the product path never does.
 * It shares no source with the HIP library: its layouts follow the same
 * written specification, restated here independently.
 *
 * All buffers are host memory owned by the caller.
 *
 * Layouts (B batch, H KV heads, G = Hq/H, D head_dim, W dense window,
 * P pool ring blocks of 64 rows, V view capacity, C condensed slots):
 *   dense_k/v   [B][H][W][D]     storage elements; position p sits in slot p mod W
 *   pool_k/v    [B][H][P][64][D] position p sits in block (p/64) mod P, row p mod 64
 *   view_k/v    [B][H][V][D]     row r holds the r-th selected position (ascending)
 *   view_pos    int32 [B][H][V]
 *   cond_kn/vn  double [B][H][C][D]   weighted sums (numerators)
 *   cond_omega  double [B][H][C]      sum of merge weights
 *   cond_n      int32 [B][H][C]       tokens merged into the slot
 *   cond_cursor int32 [B][H]          next slot (ring)
 *   seq_len     int64 [B]             t, tokens so far
 *   pool_head   int64 [B][H]          c, oldest pool position (multiple of 64)
 *   scores      float [B][H][P*64]    indexed by pool ring row
 *   weights     uint32 [B][H][P*64]
 *   mask        uint64 [B][H][P]      word (p/64) mod P, bit p mod 64
 *   budget, n_condense int32 [B][H]
 *   w_all, w_u, thresh uint64 [B][H] (diagnostics: total mass, survivor mass, T)
 * q is [B][Hq][D], k_new/v_new are [B][H][D], all in the storage type.
 * out is double [B][Hq][D].
 */
#ifndef HARDKV_ORACLE_H
#define HARDKV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_COND_OFF = 0, ORC_COND_EVICT = 1, ORC_COND_MERGE = 2 };
enum { ORC_ERR_POOL_OVERFLOW = 1u, ORC_ERR_VIEW_OVERFLOW = 2u, ORC_ERR_NONFINITE = 4u };

typedef struct {
  int32_t batch, num_q_heads, num_kv_heads, head_dim;
  int32_t elem_bytes;        /* 2: bf16, 4: fp32 */
  int32_t dense_window, pool_blocks, sparse_cap, view_cap, condensed_slots, cond_mode;
  int32_t merge_bias;        /* 1: condensed slot logit gets + ln n (default), 0: none */
  double top_p;
  const float *tau;          /* [H] */
  int32_t regularize;        /* 0 rewrite every head, 1 none (Sparse Loading), 2 the heads with
                                mti_lower <= k* <= mti_upper, 3 the memory-time controller
                                (orc_mti_rewrite) */
  int32_t mti_lower, mti_upper;
  int32_t view_layout;       /* 0: every head owns view_cap rows; 1: packed in unit order (CSR) */
  int32_t view_total;        /* rows of the packed views (layout 1) */
  int32_t calibration;       /* 0: tau from tau[h]; 1: tau fitted per unit by entropy matching */
  const float *tau_unit;     /* [B*H] with calibration 1: use these instead of fitting (or NULL) */
  int32_t sink;              /* S: the first S positions form a sink tier (multiple of 64, or 0) */
  /* memory-time controller (regularize 3): H, the steps expected to reuse a selection, and
   * costs in femtoseconds per kept row (K and V) unless stated */
  int32_t mti_horizon;
  uint32_t mti_c_view;       /* a later step reading the row from a contiguous view */
  uint32_t mti_c_write;      /* writing the row into the view at the selection step */
  uint32_t mti_c_scan;       /* per survivor row, per step that gathers through the mask */
  uint32_t mti_c_hold;       /* holding the row in a view for one step (memory occupancy) */
  uint32_t mti_c_score;      /* per pool row scored at a selection (reselection period only) */
  uint32_t mti_c_gather[9];  /* a later step gathering the row from the pool, by the kept
                                eighth of the survivors: floor(8 k* / N_U) */
  int64_t mti_fixed;         /* per rewritten head and selection */
  int32_t selection;         /* 0: each selection picks a view of the whole pool; 1: destructive:
                                a selection drops for good the survivors it does not keep, so the
                                next one chooses among the rows it kept and the positions that
                                arrived since (the whole pool before the first) */
} orc_cfg;

typedef struct {
  void *dense_k, *dense_v, *pool_k, *pool_v, *view_k, *view_v;
  int32_t *view_pos;
  double *cond_kn, *cond_vn, *cond_omega;
  int32_t *cond_n, *cond_cursor;
  int64_t *seq_len, *pool_head;
  float *scores;
  uint32_t *weights;
  uint64_t *mask;
  int32_t *budget, *n_condense;
  uint64_t *w_all, *w_u, *thresh;
  int32_t *regularized;      /* [B*H] 1 if the head's view was rewritten this step (may be NULL) */
  int32_t *view_off;         /* [B*H + 1] row offsets of the packed views (layout 1) */
  float *tau_fit;            /* [B*H] the temperature used (calibration 1; may be NULL) */
  uint32_t error_word;
  void *sink_k, *sink_v;     /* [B*H][S][D]: position p < S in row p (S > 0) */
  int64_t *pend_sel;         /* [B*H] the pool end at the last selection (the pool head, S, after
                                a prefill): a step without selection attends the pool positions
                                from here on in full */
} orc_state;

/* building blocks, exported for the pin tests */
float    orc_dot_pairwise(const float *a, const float *b, int32_t n);
float    orc_score_row(const float *q, int32_t G, const float *k, int32_t D);
float    orc_kappa(int32_t D, float tau);
float    orc_poly_coeff(int32_t i);
float    orc_exp2_poly(float f);
void     orc_exp2_poly_batch(const float *f, float *y, int64_t n);
uint32_t orc_weight(float s, float m, float kappa);
void     orc_weight_batch(const float *t, uint32_t *w, int64_t n);
uint32_t orc_pq(double p);
int32_t  orc_topp(const uint32_t *w, const int64_t *pos, int32_t n, uint32_t pq,
                  uint8_t *selected, uint64_t *thresh_out);

/* the step */
int32_t orc_prefill(const orc_cfg *cfg, orc_state *st, const void *k_ctx, const void *v_ctx,
                    const int64_t *ctx_len, int64_t max_len);
int32_t orc_step(const orc_cfg *cfg, orc_state *st, const void *q, const void *k_new,
                 const void *v_new, double *out, int32_t do_attend, int32_t nthreads);
/* a step that reuses the last selection: the append, then attention over the sinks, the
 * condensed slots, the rows the last selection kept (its views, or the pool rows its mask
 * marks), the pool positions that arrived since it, and the dense window */
int32_t orc_step_reuse(const orc_cfg *cfg, orc_state *st, const void *q, const void *k_new,
                       const void *v_new, double *out, int32_t nthreads);
/* a selection made ahead of its use (the asynchronous pipeline): st's seq_len holds the
 * snapshot of the step it is made for, its pool, dense, sink and condensed buffers and pool
 * head are the live ones; plan, score, calibrate, top-p and regularize, no condensation and
 * no attention (max-length views only) */
int32_t orc_select_ahead(const orc_cfg *cfg, orc_state *st, const void *q);
/* the switch to a selection made ahead: its planned condensation (E blocks from the pool
 * head, its weights and mass), and the pool head moved past them */
int32_t orc_condense_plan(const orc_cfg *cfg, orc_state *st);
/* entropy-matched temperature: d are the G x n raw dot products (query-major), s the n
 * max-pooled scores; returns the fitted tau (fp32) and the target entropy in *h_target */
float   orc_fit_tau(const float *d, int32_t G, const float *s, int64_t n, int32_t D, double *h_target);
/* entropy (nats) of softmax(s / (sqrt(D) tau)) over n scores, binary64 */
double  orc_calibrated_entropy(const float *s, int64_t n, int32_t D, double tau);
/* memory-time controller: whether a head with k* kept rows out of n survivors is rewritten
 * (regularize 3); the smallest and largest budgets in [1, n] that are rewritten (lo = 0,
 * hi = -1 when none); and the steps per selection in [1, max_period] that minimise the memory
 * time per step of a head with n_pool pool rows, n survivors and k* kept rows */
int32_t orc_mti_rewrite(const orc_cfg *cfg, int64_t kstar, int64_t n);
void    orc_mti_thresholds(const orc_cfg *cfg, int64_t n, int64_t *lo, int64_t *hi);
int32_t orc_mti_period(const orc_cfg *cfg, int64_t n_pool, int64_t n, int64_t kstar, int32_t max_period);
/* full softmax attention over positions [0, t) of a flat cache, binary64 (pin I4) */
void    orc_full_attention(const float *q, const float *k, const float *v, int32_t n,
                           int32_t D, double *out);

#ifdef __cplusplus
}
#endif
#endif
