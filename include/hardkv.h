/* hardkv.h -- C ABI of the HARD-KV decode-time cascade-cache step on one AMD
 * Instinct MI355X (gfx950).
 *
 * HARD-KV ("HARD-KV: Head-Adaptive Regularization for Decoding-time KV
 * Compression", technical summary section 2) keeps each KV head's cache in
 * three tiers: a dense window of the most recent tokens, a sparse tier from
 * which a calibrated top-p selection keeps a head-adaptive set of tokens, and a
 * constant-size condensed tier into which the oldest blocks are evicted or
 * merged.  One decode step runs four stages (section 2.A): linear append to the
 * dense tier; logits calibration and top-p to build sparse masks; index
 * regularization that rewrites the selected tokens into contiguous blocks; and
 * eviction or weighted merging of the oldest blocks.  Decode attention then
 * reads the three tiers.
 *
 * Per (sequence b, KV head h) a step computes, with G = Hq / Hkv and query
 * heads h*G .. h*G+G-1 sharing KV head h:
 *   1. append: the new (k, v) goes to dense slot t mod W; position t - W, which
 *      leaves the window, is copied to the tail of the pool; t grows by one.
 *   2. plan: the pool holds positions [c, t - W); N = t - W - c.  When the mode is
 *      not OFF and N > S_cap, the E = ceil((N - S_cap) / 64) oldest blocks will be
 *      condensed; the survivors are U = [c + 64E, t - W).
 *   3. score: s_j = max over the group's queries of q . k_j, each dot product a
 *      pairwise tree of fp32 products with one rounding per operation (2.B,
 *      "max-pooled logits").
 *   4. calibrate: m = max s over the pool; w_j = max(1, floor(2^24 * 2^t_j)),
 *      t_j = (s_j - m) * kappa_h, kappa_h = log2(e) / (sqrt(D) tau_h) (2.B,
 *      temperature calibration into one softmax).
 *   5. top-p: T = ceil(p_q W_U / 2^16) with p_q = round(p * 2^16) and W_U the mass
 *      of U; the survivors in order of decreasing w (lower position first on
 *      ties) are kept until their mass reaches T.  k* tokens are kept (the
 *      head-adaptive budget of tier 2).
 *   6. regularize: the kept positions, in ascending order, are copied bit for bit
 *      into rows 0 .. k*-1 of the head's view (2.C, Rewrite Cache with a flat index
 *      to the maximum length, every head owning V_cap view rows, or to the sum, the
 *      views packed by the budgets), for the heads the regularize policy rewrites; the
 *      others are attended through the mask (Sparse Loading).
 *   7. condense: each of the E oldest blocks is dropped (EVICT) or merged into the
 *      next condensed slot (MERGE, a ring of C slots): Kn += sum w_j/W_all k_j,
 *      Vn += sum w_j/W_all v_j, Omega += sum w_j/W_all, n += 64.  c += 64 E.
 *   8. attend: softmax attention of each query over the condensed slots with
 *      n > 0 (key Kn/Omega, value Vn/Omega, logit bias ln n), the view rows
 *      r < k*, the dense window, and the sink rows.  Output in fp32.
 * Sink tier (optional, cfg->sink = S > 0; a reading of the dense tier's role of
 * preserving "attention sinks", 2.A): positions [0, S) are kept apart in the sink
 * rows, attended at every step and never scored, condensed or rewritten.  Then the
 * dense window holds [max(S, t - W), t), the pool [c, max(S, t - W)) with c starting
 * at S, and an append below S writes the sink row instead; with S = 0 every range
 * above is as written.
 * Steps 2-7 give bit-identical integer results (masks, budgets, indices, view
 * rows) to a plain CPU definition of the same step.
 *
 * Conventions
 *   - head_dim is 128; the block size is 64 tokens (one mask word).
 *   - Every device buffer is owned by the caller (for example allocated as
 *     tensors) on the current HIP device.  The library never allocates, frees,
 *     synchronizes, or reads device memory from the host.  Calls are
 *     asynchronous on `stream` (a hipStream_t; NULL is the default stream) and
 *     may be captured into a HIP graph.
 *   - Host-detectable errors (bad sizes, null or misaligned pointers, too small a
 *     workspace) return a negative status before anything is enqueued.
 *   - Runtime conditions set bits of *error_word on the device (the caller reads
 *     it after a synchronization of its choosing): HARDKV_ERR_POOL_OVERFLOW (a
 *     unit's pool ring overflowed, or the SHARED pool had no free block),
 *     HARDKV_ERR_VIEW_OVERFLOW,
 *     HARDKV_ERR_NONFINITE (a non-finite score; outputs are then undefined).
 *   - The workspace must be zero-filled once before first use; the kernels leave
 *     its counters at zero after each call.  It belongs to its state: besides
 *     per-call scratch it keeps, per (b, h), whether a key whose products with a
 *     query could round in fp32 (a nonzero 16-bit element of magnitude below 2^-63
 *     or from 2^65) has entered the pool since the prefill; hardkv_prefill and
 *     hardkv_append keep it, so a state's pool is filled only through them.
 *   - Calls on one state must not overlap (they share the workspace).
 */
#ifndef HARDKV_H
#define HARDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HARDKV_OK = 0,
  HARDKV_EINVAL = -1,      /* bad argument: null/misaligned pointer, inconsistent sizes */
  HARDKV_EUNSUPPORTED = -2,/* valid but not supported: head_dim != 128, G not in {1,2,4,8} */
  HARDKV_ECAPACITY = -3,   /* a capacity is too small for the requested contents */
  HARDKV_EHIP = -4,        /* a HIP launch failed */
  HARDKV_ESCRATCH = -5     /* hardkv_step_noalloc: the step needs more scratch than the
                              library's static array holds (HARDKV_STATIC_SCRATCH_BYTES) */
} hardkv_status;

typedef enum { HARDKV_BF16 = 0, HARDKV_F32 = 1 } hardkv_dtype;
typedef enum { HARDKV_COND_OFF = 0, HARDKV_COND_EVICT = 1, HARDKV_COND_MERGE = 2 } hardkv_cond_mode;

/* How the kept tokens reach attention (section 2.C names Rewrite Cache, which moves the
 * selected blocks into contiguous ranges, and Sparse Loading, which loads them through
 * hardware-friendly masks, with a memory-time trade-off between the two switched by
 * budget thresholds L_lower and L_upper; the pages give no formula, so the switch is a
 * stated rule):
 *   REWRITE  every head's kept rows are rewritten into its view (the default);
 *   SPARSE   no head is rewritten: attention gathers the kept rows from the pool ring
 *            through the mask words;
 *   MTI      head (b, h) is rewritten iff mti_lower <= k* <= mti_upper: below L_lower so
 *            few rows are kept that gathering them each step costs less than keeping a
 *            view; above L_upper the mask covers so much of the pool that masked loads
 *            are nearly contiguous and a rewrite would copy almost everything;
 *   MTI_AUTO the memory-time controller below decides per head from its k*, its survivor
 *            count and the reuse horizon.
 * The attention output, masks and budgets do not depend on the policy (the fused step
 * attends the kept rows from registers either way); only the views differ: a head that is
 * not rewritten leaves its view rows and view_pos untouched. */
typedef enum { HARDKV_REG_REWRITE = 0, HARDKV_REG_SPARSE = 1, HARDKV_REG_MTI = 2, HARDKV_REG_MTI_AUTO = 3 }
    hardkv_regularize_policy;

/* The memory-time controller (policy MTI_AUTO; a reading of section 2.C's memory-time integral
 * that weighs the one-off rewrite against the per-step gains).  For a head with k* kept rows
 * out of N_U survivors and a horizon of H later steps that reuse the selection
 * (cfg->mti_horizon, what the caller expects until it selects again), the memory time the
 * kept rows cost over the selection step and those H steps, in femtoseconds:
 *   Sparse Loading  (H + 1) (k* g[b] + N_U c_scan)
 *   Rewrite Cache   k* g[b] + N_U c_scan + k* c_write + H k* (c_view + c_hold) + F
 * with b = min(8, floor(8 k* / N_U)) the kept eighth of the survivors, g[b] a later step's
 * gather of one kept row through the mask, c_scan its walk over one survivor row's mask bit,
 * c_write the view write of one row at the selection, c_view a later step's read of one
 * view row, c_hold one view row held for one step, F a fixed cost per rewritten head.  The
 * head is rewritten iff the second is smaller, compared exactly in 64-bit integers (k* = 0 is
 * never rewritten; with H = 0 nothing is).  For a given N_U the rewritten budgets run from
 * L_lower to L_upper (hardkv_mti_thresholds) when g does not grow with b.  Costs are per row
 * of K and V in the layer's dtype; the defaults below were measured with this library's own
 * kernels on the 16k-context, batch-16 bf16 layer (per kept row: the view attention 97 ps, the
 * fused step's view stores 68 ps, the gathered attention 124 ps; the score 44 ps per pool
 * row), so on this part a rewrite pays from H = 3 reused steps on. */
#define HARDKV_MTI_C_VIEW 97000u
#define HARDKV_MTI_C_WRITE 68000u
#define HARDKV_MTI_C_GATHER 124000u
#define HARDKV_MTI_C_SCORE 44000u
#define HARDKV_MTI_MAX_HORIZON 65535
#define HARDKV_MTI_MAX_COST (1u << 24)     /* every cost below this, in fs */
#define HARDKV_MTI_MAX_FIXED (1ll << 40)

/* Flatten Index (section 2.C: indices regularized to the maximum length or to their sum):
 *   MAXLEN  every head owns view_cap rows: head u's row r is row u * view_cap + r (default);
 *   SUM     the rewritten heads' kept rows are packed in unit order (CSR): head u's row r is
 *           row view_off[u] + r, view_off the exclusive prefix sum over units of k* (0 for a
 *           head that is not rewritten), so view memory follows the sum of the budgets.
 *           The view arrays then hold view_total rows; rows past view_total are not
 *           written and set HARDKV_ERR_VIEW_OVERFLOW.  A head's view only lives until the
 *           next select (the offsets move with every step's budgets). */
typedef enum { HARDKV_VIEW_MAXLEN = 0, HARDKV_VIEW_SUM = 1 } hardkv_view_layout;
/* The pool's memory (section 2.C: a head-wise block manager allocates head-adaptively while
 * keeping static shapes and persistent pointers for graph capture):
 *   RING    every (b, h) owns a ring of pool_blocks blocks in pool_k/v (default);
 *   SHARED  one pool of pool_total_blocks physical blocks of 64 rows for all (b, h): ring
 *           block pb of unit u is physical block block_table[u][pb] (-1: none).  The prefill
 *           gives each unit the blocks its pool holds, in unit order, and leaves the others
 *           on the free list; an append takes a block from the free list when a position
 *           starts a new one; a condensation returns the blocks it condenses.  Memory then
 *           follows what the pools hold instead of B * Hkv worst-case rings; pool_blocks stays
 *           the per-unit ring (the table's length).  An append or prefill that finds the free
 *           list empty sets HARDKV_ERR_POOL_OVERFLOW and writes nothing.  The prefill writes
 *           the table and the free list (they need no initialisation); which free block an
 *           append takes depends on the order of the appends' atomics, every result does
 *           not.  hardkv_shared_pool_blocks sizes a pool that cannot overflow. */
typedef enum { HARDKV_POOL_RING = 0, HARDKV_POOL_SHARED = 1 } hardkv_pool_layout;
/* What a selection does to the survivors it does not keep (section 2.A: the sparse tier
 * retains the tokens the calibrated top-p selects; the pages leave open whether the others
 * are gone for good):
 *   VIEW         nothing: every selection chooses among the whole pool (default);
 *   DESTRUCTIVE  they are dropped for good: the next selection chooses among the rows the
 *                last one kept and the positions that arrived since it (the whole pool
 *                before the first selection after a prefill).  Dropped rows keep their pool
 *                rows but take no part: the calibration maximum is over the rows in play, a
 *                dropped row weighs 0 (weights[] holds 0; it is in no mass, never kept), and
 *                a condensation merges only the rows in play (a block adds their count to
 *                n; one with none adds nothing).  Selections run when the caller takes
 *                hardkv_step (hardkv_step_reuse between them keeps the last one), so with a
 *                selection every step the tier shrinks towards what top-p keeps of a few
 *                arrivals.  With p = 1 it is VIEW.  Needs the FIXED calibration, and is not
 *                taken by the pipeline calls or hardkv_step_noalloc (HARDKV_EUNSUPPORTED). */
typedef enum { HARDKV_SEL_VIEW = 0, HARDKV_SEL_DESTRUCTIVE = 1 } hardkv_selection_mode;

/* Logits Calibration temperature (section 2.B calibrates the scores by the temperature of
 * the attention scores without fixing how it is obtained):
 *   FIXED    tau_h from hardkv_config.tau (default);
 *   ENTROPY  tau fitted per (b, h) and step: the calibrated softmax of the max-pooled scores,
 *            softmax(s / (sqrt(D) tau)) over the pool, gets the mean entropy (in nats) of
 *            the group's raw attention softmax(q_g . k / sqrt(D)) over the pool.  tau is
 *            the midpoint of the bracket found by five rounds of a 17-point grid on
 *            log2 tau in [-12, 12] (entropy grows with tau), rounded to fp32; kappa then
 *            follows from it as for a fixed tau.  Written to hardkv_state.tau_fit. */
typedef enum { HARDKV_CAL_FIXED = 0, HARDKV_CAL_ENTROPY = 1 } hardkv_calibration;

/* (The fused step's attention reads the kept rows themselves, so it does not depend on
 * whether their view rows fit; hardkv_attend reads the views and sees only rows that fit.) */

#define HARDKV_BLOCK 64
#define HARDKV_HEAD_DIM 128
#define HARDKV_MAX_KV_HEADS 64
#define HARDKV_ERR_POOL_OVERFLOW 1u
#define HARDKV_ERR_VIEW_OVERFLOW 2u
#define HARDKV_ERR_NONFINITE 4u
#define HARDKV_MAX_SINK 8192
#define HARDKV_MAX_UNITS 65535     /* batch * num_kv_heads (one launch row per unit) */
#define HARDKV_MAX_POOL_BLOCKS 6144 /* pool ring blocks per unit the select can index */
#define HARDKV_STATIC_SCRATCH_BYTES (128u << 20) /* the no-alloc step's scratch per GPU */

/* Host-side description of one layer; passed by pointer to every call. */
typedef struct {
  int32_t batch;           /* B >= 1; B * Hkv <= HARDKV_MAX_UNITS (else HARDKV_EUNSUPPORTED) */
  int32_t num_q_heads;     /* Hq */
  int32_t num_kv_heads;    /* Hkv, 1..64; G = Hq / Hkv in {1, 2, 4, 8} */
  int32_t head_dim;        /* D, must be 128 */
  int32_t dtype;           /* storage and compute type of q, K, V: HARDKV_BF16 or HARDKV_F32 */
  int32_t dense_window;    /* W >= 1 */
  int32_t pool_blocks;     /* P: pool ring blocks of 64 rows per (b, h); P*64 >= sparse_cap + 64;
                              P <= HARDKV_MAX_POOL_BLOCKS (else HARDKV_EUNSUPPORTED) */
  int32_t sparse_cap;      /* S_cap: multiple of 64, >= 64 */
  int32_t view_cap;        /* V_cap >= sparse_cap (>= P*64 in mode OFF) */
  int32_t condensed_slots; /* C >= 1 */
  int32_t cond_mode;       /* hardkv_cond_mode */
  int32_t merge_bias;      /* 1: merged slots get logit bias ln n (default); 0: no bias */
  double top_p;            /* p in (0, 1]; p_q = round(p * 65536) must be >= 1 */
  const float *tau;        /* host array [num_kv_heads], calibration temperatures > 0 (+inf allowed) */
  int32_t regularize;      /* hardkv_regularize_policy (0: REWRITE) */
  int32_t mti_lower;       /* L_lower, tokens, >= 0 (policy MTI) */
  int32_t mti_upper;       /* L_upper, tokens, >= mti_lower (policy MTI) */
  int32_t view_layout;     /* hardkv_view_layout (0: MAXLEN) */
  int32_t view_total;      /* rows of the packed views (layout SUM), >= 0 */
  int32_t calibration;     /* hardkv_calibration (0: FIXED) */
  int32_t sink;            /* S: sink prefix tokens, a multiple of 64 in [0, HARDKV_MAX_SINK]
                              (0: none); see the sink tier above */
  /* the memory-time controller (policy MTI_AUTO; see above; femtoseconds per row of K and V) */
  int32_t mti_horizon;     /* H in [0, HARDKV_MTI_MAX_HORIZON] */
  uint32_t mti_c_view, mti_c_write, mti_c_scan, mti_c_hold;
  uint32_t mti_c_score;    /* per pool row scored at a selection (hardkv_mti_period only) */
  uint32_t mti_c_gather[9];/* by the kept eighth b of the survivors */
  int64_t mti_fixed;       /* F per rewritten head, in [0, HARDKV_MTI_MAX_FIXED] */
  int32_t pool_layout;     /* hardkv_pool_layout (0: RING) */
  int32_t pool_total_blocks; /* NB, physical blocks of the SHARED pool, in [1, 2^26) */
  int32_t selection;       /* hardkv_selection_mode (0: VIEW) */
} hardkv_config;

/* Device buffers of one layer.  All fixed capacity; 16-byte aligned.
 * Element types: "e" is bf16 (2 bytes) or fp32 (4 bytes) per cfg->dtype. */
typedef struct {
  void *dense_k, *dense_v;   /* e [B][Hkv][W][128]: position p in slot p mod W                    */
  void *pool_k, *pool_v;     /* e [B][Hkv][P][64][128] (RING): position p in block (p/64) mod P, row
                                p%64; e [NB][64][128] (SHARED): in physical block
                                block_table[b][h][(p/64) mod P], row p%64                         */
  void *view_k, *view_v;     /* e [B][Hkv][V_cap][128] (MAXLEN) or e [view_total][128] (SUM): the
                                head's row r = its r-th kept position (ascending)                */
  int32_t *view_pos;         /* [B][Hkv][V_cap] or [view_total]: position of each view row        */
  float *cond_kn, *cond_vn;  /* fp32 [B][Hkv][C][128]: merged numerators                          */
  float *cond_omega;         /* fp32 [B][Hkv][C]: merged weight                                   */
  int32_t *cond_n;           /* [B][Hkv][C]: tokens merged into the slot                          */
  int32_t *cond_cursor;      /* [B][Hkv]: next slot of the ring                                   */
  int64_t *seq_len;          /* [B]: t                                                            */
  int64_t *pool_head;        /* [B][Hkv]: c, a multiple of 64                                     */
  float *scores;             /* fp32 [B][Hkv][P*64]: s by pool ring row (rows outside the pool, and rows a
                                destructive selection dropped, unspecified) */
  uint32_t *weights;         /* [B][Hkv][P*64]: w by pool ring row                                */
  uint64_t *mask;            /* [B][Hkv][P]: word (p/64) mod P, bit p%64 set iff p is kept        */
  int32_t *budget;           /* [B][Hkv]: k*                                                      */
  int32_t *n_condense;       /* [B][Hkv]: E of the last select                                    */
  uint64_t *w_all;           /* [B][Hkv]: total pool mass                                         */
  uint64_t *w_u;             /* [B][Hkv]: survivor mass W_U                                       */
  uint64_t *thresh;          /* [B][Hkv]: T                                                       */
  int32_t *regularized;      /* [B][Hkv]: 1 if the head's view is rewritten this step, else 0
                                (may be NULL: not reported)                                       */
  int32_t *view_off;         /* [B*Hkv + 1]: CSR row offsets of the SUM layout, the last one the
                                total (written by select; may be NULL in the MAXLEN layout)       */
  float *tau_fit;            /* [B][Hkv]: the fitted temperature (calibration ENTROPY; may be NULL
                                otherwise)                                                        */
  void *sink_k, *sink_v;     /* e [B][Hkv][S][128]: sink position p in row p (may be NULL if S = 0) */
  uint32_t *error_word;      /* [1]: HARDKV_ERR_* bits, or-ed                                     */
  void *workspace;           /* hardkv_workspace_size() bytes, zero-filled before first use      */
  size_t workspace_bytes;
  int32_t *block_table;      /* SHARED pool: [B][Hkv][P] physical block of each ring block (-1: none) */
  int32_t *free_list;        /* SHARED pool: [pool_total_blocks] free physical blocks               */
  int32_t *free_top;         /* SHARED pool: [1] free blocks in free_list (written by the prefill)  */
} hardkv_state;

/* Bytes of workspace a state needs.  Returns HARDKV_EINVAL/EUNSUPPORTED on a bad config. */
int32_t hardkv_workspace_size(const hardkv_config *cfg, size_t *bytes);

/* Places a context: k_ctx/v_ctx are e [B][Hkv][max_len][128] (device), ctx_len_dev is
 * int64 [B] (device) with 0 <= L_b <= max_len.  Positions below S go to the sink rows,
 * [max(S, L_b - W), L_b) to the dense ring and the rest to the pool; t = L_b, c = S,
 * condensed tier emptied, cursor 0.
 * HARDKV_ECAPACITY if max_len - W + 1 - S > P*64 (the first append would not fit). */
int32_t hardkv_prefill(const hardkv_config *cfg, hardkv_state *st, const void *k_ctx,
                       const void *v_ctx, const int64_t *ctx_len_dev, int64_t max_len, void *stream);

/* Stage 1 (section 2.A): k_new, v_new are e [B][Hkv][128] (device). */
int32_t hardkv_append(const hardkv_config *cfg, hardkv_state *st, const void *k_new,
                      const void *v_new, void *stream);

/* Stage 2 (sections 2.A, 2.B): score, calibrate and top-p for every (b, h); writes scores,
 * weights, mask, budget, n_condense, w_all, w_u, thresh.  q is e [B][Hq][128] (device). */
int32_t hardkv_select(const hardkv_config *cfg, hardkv_state *st, const void *q, void *stream);

/* Stage 3 (section 2.C): copies the kept rows into the view and writes view_pos, for the
 * heads that the regularize policy rewrites (all of them under REWRITE). */
int32_t hardkv_regularize(const hardkv_config *cfg, hardkv_state *st, void *stream);

/* Stage 4 (section 2.A, tier 3): evicts or merges the E oldest blocks; advances c and
 * the slot cursor. */
int32_t hardkv_condense(const hardkv_config *cfg, hardkv_state *st, void *stream);

/* Decode attention over the three tiers (technical summary 2.A: the dense tier of recent
 * tokens, the sparse tier's kept tokens and the constant-size condensed tier together
 * stand for the whole context): each query's softmax over the condensed slots with n > 0,
 * the view rows r < k*, the dense window and the sink rows; out is fp32 [B][Hq][128]
 * (device).  Heads that the last select left to Sparse Loading are attended through the
 * pool and the mask instead of the view. */
int32_t hardkv_attend(const hardkv_config *cfg, hardkv_state *st, const void *q, float *out,
                      void *stream);

/* Sparse Loading (section 2.C): attention over the condensed tier, the kept rows gathered
 * from the pool ring through the mask of the last select (whatever the policy; no view is
 * read), and the dense tier.  Same arguments and output as hardkv_attend. */
int32_t hardkv_attend_sparse(const hardkv_config *cfg, hardkv_state *st, const void *q, float *out,
                             void *stream);

/* The whole step (technical summary 2.A: the four stages of a step -- linear append to
 * the dense tier, calibrated top-p masks, index regularization, eviction or weighted
 * merging of the oldest blocks -- followed by attention over the tiers; 2.C: static
 * shapes and persistent pointers so that the step can be captured into a graph): append,
 * select, regularize, condense, attend, in one stream-ordered, capturable sequence (the
 * view attention is fused into the rewrite, and when at most four blocks can condense per
 * step, P - S_cap/64 <= 4, the condensation into the select). */
int32_t hardkv_step(const hardkv_config *cfg, hardkv_state *st, const void *q, const void *k_new,
                    const void *v_new, float *out, void *stream);

/* A step that keeps the last selection (section 2.C: a rewritten cache is used for later
 * steps, spreading its cost over them; when to select again is the caller's choice, for
 * example every R steps): the append, then attention over the sinks, the condensed slots,
 * the rows the last selection kept (views of rewritten heads, pool rows through the mask
 * for the others), every pool position that arrived after that selection (the pool end at
 * its t up to the pool end now), and the dense window.  Nothing is scored, selected or
 * condensed, so the pool grows by one position per step: pool_blocks must hold S_cap
 * plus the positions of the steps between selections (HARDKV_ERR_POOL_OVERFLOW
 * otherwise), and the next hardkv_step condenses what has accumulated.  Before any
 * selection since the prefill, the whole pool counts as arrived after the last selection.
 * Same arguments as hardkv_step; capturable. */
int32_t hardkv_step_reuse(const hardkv_config *cfg, hardkv_state *st, const void *q, const void *k_new,
                          const void *v_new, float *out, void *stream);

/* hardkv_step for callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): the same kernels and results,
 * with the step's scratch (plan, per-block offsets, attention partials, select and fit
 * scratch) in a static device array of the library, HARDKV_STATIC_SCRATCH_BYTES on every
 * GPU it runs on, held from the first call on that GPU until the process ends, instead of
 * st->workspace (which may be NULL; workspace_bytes is ignored).  Allocates nothing.
 *   - HARDKV_ESCRATCH (before anything is enqueued) when hardkv_workspace_size(cfg) exceeds
 *     HARDKV_STATIC_SCRATCH_BYTES; the other checks and statuses are hardkv_step's.
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's contents:
 *     calls that overlap on one GPU (other streams, other threads) race, and their results
 *     are undefined.  Nothing in the array has to start at zero.
 *   - The first call on a GPU looks up the array's address on it (HARDKV_EHIP if that
 *     fails); make it outside graph capture.
 *   - The array keeps nothing of a state between calls, so the record of keys whose
 *     products with a query could round in fp32 (see the workspace above) is not kept:
 *     every head's scores take the plain pairwise tree, which gives the same bits.  A state
 *     stepped by this call lacks that record in its own workspace afterwards: keep stepping
 *     it with this call (or prefill it again) rather than with the calls that read the
 *     workspace (hardkv_step, hardkv_step_reuse, hardkv_regularize, hardkv_condense,
 *     hardkv_attend, hardkv_attend_sparse).
 *   - A DESTRUCTIVE selection reads the last selection's plan, which the array does not keep:
 *     HARDKV_EUNSUPPORTED. */
int32_t hardkv_step_noalloc(const hardkv_config *cfg, hardkv_state *st, const void *q, const void *k_new,
                            const void *v_new, float *out, void *stream);

/* The asynchronous pipeline (section 2.A: the four stages run as an asynchronous pipeline;
 * a reading with selections reused over later steps): the next selection is made on a second
 * stream while decode steps continue on the current one (hardkv_step_reuse), and switched in
 * at a later step.  It takes a second state, st_next, that shares the cache itself with the
 * current one (dense_k/v, pool_k/v, sink_k/v, cond_kn/vn/omega/n, cond_cursor, seq_len,
 * pool_head, and the SHARED pool's block_table, free_list and free_top: the same pointers)
 * and has its own selection buffers (scores, weights, mask,
 * budget, n_condense, w_all, w_u, thresh, view_k/v, view_pos, regularized, tau_fit) and its
 * own workspace; otherwise HARDKV_EINVAL.
 *   1. hardkv_select_fork(cfg, st_next, st_cur, s_main): on the main stream, right after the
 *      append of the step the selection is made for: records t of every sequence and the
 *      current state's key-magnitude record in st_next's workspace.
 *   2. hardkv_select_ahead(cfg, st_next, q, unit_begin, unit_count, stream): score, calibrate,
 *      top-p and Rewrite Cache (the views of the heads the policy rewrites) of units
 *      [unit_begin, unit_begin + unit_count) (unit b * Hkv + h) over the pool as it stood at
 *      the forked step, with that step's queries q (kept alive by the caller until the last
 *      part has run); the planned condensation is not applied.  Either all units at once on
 *      a second stream, after an event the caller records on s_main behind the fork, or in
 *      parts spread over the steps before the switch on any stream ordered after the fork.
 *      HARDKV_EINVAL for a range outside [0, B * Hkv]; the max-length view layout only
 *      (HARDKV_EUNSUPPORTED for SUM).
 *   3. Meanwhile s_main may take hardkv_step_reuse steps on st_cur (no selection, no
 *      condensation): they append and attend the current selection.  The pool ring must
 *      hold S_cap plus the positions of the steps until the switch.
 *   4. The switch, on s_main after the caller waits for the side stream: hardkv_condense(cfg,
 *      st_next) applies the planned condensation (the blocks and merge weights of the forked
 *      step), and from then on st_next is the current state (hardkv_step_reuse attends its
 *      kept rows and every position since the forked step).
 * Switched in at once (fork, ahead and condense before the next append), the selection is
 * the step's own: the same masks, budgets, views and condensed tier as hardkv_step. */
int32_t hardkv_select_fork(const hardkv_config *cfg, hardkv_state *st_next, const hardkv_state *st_cur,
                           void *stream);
int32_t hardkv_select_ahead(const hardkv_config *cfg, hardkv_state *st_next, const void *q, int32_t unit_begin,
                            int32_t unit_count, void *stream);

/* Launches only kernel `stage` of hardkv_step (0 append, 1 score, 2 select, 3 condense,
 * 4 rewrite with the view, condensed and dense attention, 5 combine), for timing one
 * kernel on its own; the condensation is always its own stage here.  Stages 1, 2, 4 and 5
 * only read what earlier stages wrote and may be repeated; 0 and 3 advance the state. */
int32_t hardkv_step_stage(const hardkv_config *cfg, hardkv_state *st, const void *q,
                          const void *k_new, const void *v_new, float *out, int32_t stage,
                          void *stream);

/* Number of kernels hardkv_step launches, and the name of kernel `stage`. */
int32_t hardkv_step_num_stages(void);
const char *hardkv_step_stage_name(int32_t stage);

/* Size of a SHARED pool (host only): *blocks is the number of physical blocks the units'
 * pools hold after a prefill of the lengths ctx_len[0 .. batch) (a host array) followed by
 * `steps` appends with no condensation: per unit, the blocks that cover its pool
 * [S, max(S, L + steps - W)), at most pool_blocks, summed over num_kv_heads heads per sequence.
 * A pool of that many blocks never overflows over those steps; a condensation only returns
 * blocks.  HARDKV_EINVAL on a bad config, a null pointer, or a length or step count outside
 * [0, 2^40]. */
int32_t hardkv_shared_pool_blocks(const hardkv_config *cfg, const int64_t *ctx_len, int64_t steps,
                                  int64_t *blocks);

/* The memory-time controller's thresholds (host only): *l_lower and *l_upper are the smallest
 * and the largest budget k* in [1, n_survivors] that policy MTI_AUTO rewrites for a head of
 * n_survivors survivors (0 and -1 when it rewrites none).  HARDKV_EINVAL on a bad config or
 * n_survivors outside [0, 2^20). */
int32_t hardkv_mti_thresholds(const hardkv_config *cfg, int64_t n_survivors, int32_t *l_lower,
                              int32_t *l_upper);

/* When to select again (host only; a reading by the same memory-time integral): the number of
 * steps R in [1, max_period] per selection that minimises the memory time per step of a head
 * with n_pool pool rows, n_survivors survivors and budget kstar, selecting every R steps: the
 * score of the pool (c_score per row), the cheaper of the two policies above for H = R - 1,
 * and, j steps after the selection, the j pool rows that arrived since (c_view each); the
 * smallest such R.  Nothing here bounds how stale a selection may grow: max_period does. */
int32_t hardkv_mti_period(const hardkv_config *cfg, int64_t n_pool, int64_t n_survivors, int64_t kstar,
                          int32_t max_period, int32_t *period);

/* Text for a status code. */
const char *hardkv_strerror(int32_t code);

#ifdef __cplusplus
}
#endif
#endif /* HARDKV_H */
