/*
 * spin.h -- C ABI of the SPIN decode-step library for AMD Instinct MI355X (gfx950).
 *
 * SPIN ("SPIN: Shadow Predictive Indexer for Sparse Attention", arXiv
 * 2610.09025) replaces the dense indexer scan of a DSA-style sparse-attention
 * layer with four stages per decode step:
 *   1. predict block importance from two EMA states (Sec. 3.2, Eq. 1, Eq. 2);
 *   2. fill the block budget with top-ranked blocks plus Philox-drawn
 *      exploration blocks (Algorithm 1 steps 4-5, Sec. 3.2.1);
 *   3. run the indexer z[i] = sum_h w_h ReLU(q_h . k_i) on the selected blocks
 *      only and apply top-K (Sec. 2, Algorithm 1 steps 6-7);
 *   4. update the EMAs, deferred to the prefix-valid verifier rows under
 *      speculative decoding (Algorithm 1 steps 8-10, Sec. 3.2.2).
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers unless marked "host".  The caller
 *     owns every buffer; the library never allocates, frees, or retains a
 *     pointer past the call.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns without synchronising the host.
 *   - Positions and lengths are in compressed KV slots.  A KV block is 64
 *     consecutive logical slots and equals one physical page of the key pool
 *     (Sec. 3.2 and Sec. 4.1: blocks of 64 slots matching the backend's page).
 *   - Row r (0 <= r < n_rows) of a request is the verifier query at position
 *     q_pos[req] + r; the EMA offset axis is D[q - i] with q - i >= 1.
 *   - The return status reports host-visible argument and launch errors only.
 *     Range errors that depend on device data (ctx_len, q_pos, page ids) set
 *     bits of the optional device word `spin_batch.err` (SPIN_DERR_*); the
 *     offending request is then skipped, never read or written out of bounds.
 *   - Results are deterministic: integer atomics only, fixed-order floating
 *     point.  Inputs must be finite (NaN/Inf behaviour is unspecified).
 */
#ifndef SPIN_H_
#define SPIN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spin_status {
  SPIN_OK = 0,
  SPIN_E_NULL = 1,         /* a required pointer is NULL                    */
  SPIN_E_SHAPE = 2,        /* a size or range argument is invalid           */
  SPIN_E_UNSUPPORTED = 3,  /* dtype / head shape combination not built      */
  SPIN_E_WORKSPACE = 4,    /* workspace missing or smaller than required    */
  SPIN_E_HIP = 5           /* the HIP runtime rejected a launch             */
} spin_status;

/* element types */
enum { SPIN_F32 = 0, SPIN_BF16 = 1, SPIN_FP8_E4M3 = 2 };
/* how V[i] and D[q-i] combine into a predicted slot score */
enum { SPIN_COMBINE_MAX = 0, /* Eq. 1 of the paper                       */
       SPIN_COMBINE_SUM = 1  /* one fp32 add, the "EMA_pos + EMA_off" form */ };
/* per-row block reason codes written by spin_select_blocks */
enum { SPIN_CODE_SKIP = 0, SPIN_CODE_FORCED = 1, SPIN_CODE_RANKED = 2,
       SPIN_CODE_EXPLORED = 3, SPIN_CODE_DENSE = 4 };
/* device error-word bits (OR-ed into spin_batch.err) */
enum { SPIN_DERR_CTX = 1,   /* ctx_len < 1, > 64*max_blocks or > v_ld        */
       SPIN_DERR_QPOS = 2,  /* q_pos < ctx_len or q_pos + n_rows - 1 >= d_ld */
       SPIN_DERR_PAGE = 4   /* a page-table entry outside [0, n_pages)       */ };

/* limits of this build */
#define SPIN_BLOCK 64
#define SPIN_MAX_BATCH 4096   /* requests per call */
#define SPIN_MAX_ROWS 4
#define SPIN_MAX_BLOCKS 8192  /* per request: up to 524,288 slots */
#define SPIN_MAX_TOPK 8192
#define SPIN_MAX_LAYERS 256  /* layers of one spin_stack */

/*
 * spin_config.flags: the design choices the paper ablates, as variants; 0
 * selects the paper's defaults throughout.
 *  - Block pooling of the predicted slot scores (Sec. 4.6, "Block reduction",
 *    variant A1), bits 0-1: SPIN_POOL_MAX (default): the largest; SPIN_POOL_TOP4:
 *    the mean of the up to four largest, summed largest first, divided by
 *    their count; SPIN_POOL_MEAN: the mean over the block's valid slots, the
 *    64 slot values (0 past the context) summed as a balanced pairwise tree
 *    ((s0 + s1) + (s2 + s3)) + ... in fp32, divided by the valid count.  The
 *    V block maxima (v_max) apply to SPIN_POOL_MAX only and are ignored
 *    otherwise.
 *  - SPIN_MTP_ROW0_MASK (Sec. 4.5, "Offline policy ablation", row-0 sharing):
 *    the scored union is row 0's mask alone, not the union of every row's.
 *  - SPIN_MTP_ROW0_UPDATE (same passage, row-0 update): the EMA takes row 0's
 *    scores only, whatever the acceptance outcome, instead of replaying the
 *    prefix-valid rows; q positions still advance by the accepted rows.
 *  - SPIN_EXPLORE_PER_ROW: each verifier row draws its own exploration
 *    priorities, with counter (j, step, layer + 65536 row, req_id) (layer
 *    < 65536), instead of sharing row 0's.
 *  - Exploration policy (Sec. 4.6, "Staleness mitigation"), bits 5-6; each
 *    picks the n_e explored blocks among those neither forced nor ranked
 *    (ties: lower block).  Random (0, default): the smallest Philox words.
 *    SPIN_EXPLORE_AGE: the least recently observed first, i.e. the smallest
 *    last_obs[j], the step at which block j was last in the scored union.
 *    SPIN_EXPLORE_STALENESS: predicted importance weighted by staleness
 *    first, the largest S[j] * (float)(step - last_obs[j]) (one fp32
 *    product).  Both need the last_obs array (below).
 *  - Block reduction (Sec. 4.6, "Block reduction"), bits 7-8.  A1 (0,
 *    default): pool the predicted slot scores into block scores.
 *    SPIN_REDUCE_A0: the K slots with the largest predicted slot score (K =
 *    topk; ties: lower slot) expanded to every block holding one (code
 *    RANKED), plus the forced blocks, plus floor(|mask| * explore_bp / 10000)
 *    explored blocks from the rest; sparsity_bp and the budget override do
 *    not apply (the realized sparsity follows from how the slots spread).  A0
 *    runs in spin_step / spin_step_plan only (it reads the slot-level state).
 *    SPIN_REDUCE_A2: block-level EMA states in the same V and D arrays, V[j]
 *    per block and D[floor(q / 64) - j] per block offset (floor(q / 64) <
 *    d_ld), updated from each scored block's pooled indexer score (the
 *    pooling flag's rule over its valid slots), three fp32 roundings per
 *    update, rows replayed in order; prediction S[j] = C(V[j], D[floor(q /
 *    64) - j]).  v_max does not apply.
 *  - SPIN_PREDICT_AHEAD (an execution choice; results are unchanged, bit for
 *    bit): the EMA update of a whole step (spin_step, spin_step_finish,
 *    spin_stack_step, spin_stack_commit) also computes, from the state it has
 *    just written, the block scores the next step's prediction (Eq. 1, Eq. 2)
 *    would, at that step's position q + A (A = the counter advance), into
 *    io->S, and records (step, q + A, ctx_len) per request in io->s_tag.  The
 *    next step's prediction then skips every request whose tag matches its
 *    step counter, q_pos and ctx_len, so the prediction reads no V or D of its
 *    own; any other request is predicted as usual.  One verifier row: with
 *    several the flag changes nothing (the EMA runs as without it and the
 *    next step predicts).  Requires block reduction A1 and io->s_tag.  Between such steps V, D, v_max and S must change only
 *    through these calls (or spin_reset_state, which zeroes the step counter
 *    and so invalidates every tag): a caller that edits them otherwise sets
 *    the affected tags to -1.  The step workspace grows by 4 R max_blocks
 *    bytes (spin_workspace_bytes).
 */
enum {
  SPIN_POOL_MAX = 0, SPIN_POOL_TOP4 = 1, SPIN_POOL_MEAN = 2, SPIN_POOL_MASK = 3,
  SPIN_MTP_ROW0_MASK = 4, SPIN_MTP_ROW0_UPDATE = 8, SPIN_EXPLORE_PER_ROW = 16,
  SPIN_EXPLORE_AGE = 32, SPIN_EXPLORE_STALENESS = 64, SPIN_EXPLORE_POLICY_MASK = 96,
  SPIN_REDUCE_A0 = 128, SPIN_REDUCE_A2 = 256, SPIN_REDUCE_MASK = 384,
  SPIN_PREDICT_AHEAD = 512,
  SPIN_FLAGS_ALL = 1023
};

/* Method parameters, passed by host pointer and copied by value. */
typedef struct spin_config {
  int32_t n_heads;      /* indexer heads n_h; this build: 64                       */
  int32_t head_dim;     /* indexer head dim d; this build: 128                     */
  int32_t block_size;   /* b; must be 64                                           */
  int32_t topk;         /* K of the post-indexer top-K, 1..SPIN_MAX_TOPK           */
  int32_t sparsity_bp;  /* target block sparsity rho in basis points, 0..10000     */
  int32_t explore_bp;   /* exploration share gamma in basis points, 0..10000       */
  float ema_alpha;      /* EMA decay alpha in [0,1]; beta = 1.0f - alpha in fp32   */
  int32_t combine;      /* SPIN_COMBINE_*                                          */
  int32_t key_dtype;    /* SPIN_F32 | SPIN_BF16 | SPIN_FP8_E4M3                    */
  int32_t q_dtype;      /* SPIN_F32 | SPIN_BF16                                    */
  int32_t layer;        /* layer id, part of the Philox counter                    */
  int32_t flags;        /* SPIN_POOL_* | SPIN_MTP_* | SPIN_EXPLORE_*; 0 = defaults  */
  uint64_t seed;        /* Philox4x32-10 key (lo, hi words)                        */
} spin_config;

/* One decode step of one layer for a batch of requests (host struct). */
typedef struct spin_batch {
  int32_t batch;           /* R requests, 0..SPIN_MAX_BATCH (0 = nothing to do)     */
  int32_t n_rows;          /* verifier queries per request, 1..SPIN_MAX_ROWS        */
  int32_t max_blocks;      /* capacity of per-request block arrays (>= ceil(N/64)) */
  int32_t n_pages;         /* pages in the key pool (page ids must be < n_pages)   */
  const int32_t* ctx_len;  /* [R] context length N in slots, 1..64*max_blocks      */
  const int32_t* q_pos;    /* [R] position of verifier row 0, >= N                 */
  const int32_t* step;     /* [R] decode steps since the last reset (0 = dense)    */
  const int32_t* req_id;   /* [R] stable request id (Philox counter word)          */
  int32_t* err;            /* optional device error word, OR of SPIN_DERR_*        */
} spin_batch;

/*
 * Stage 1 (Sec. 3.2, Eq. 1 and Eq. 2; Algorithm 1 steps 1-3).
 * S[r][row][j] = max over slots i in block j with i < N of C(V[i], D[q_row - i]),
 * C = max or fp32 sum (cfg->combine), q_row = q_pos[r] + row.
 *   V: f32 [R][v_ld] (v_ld >= N), D: f32 [R][d_ld] (d_ld > q_pos + n_rows - 1),
 *   v_max: optional f32 [R][max_blocks], the block maxima of V.  With C = max,
 *          max_i max(V[i], D[q - i]) = max(max_i V[i], max_i D[q - i]), so every
 *          block but the last one then reads v_max[r][j] instead of V.  Entry j
 *          must hold the max of V over all 64 slots of block j (slots >= N hold
 *          V = 0); spin_reset_state, spin_ema_update and spin_step keep it so
 *          when given it.  ctx_len must not shrink between resets.
 *   S: f32 [R][n_rows][max_blocks]; entries j >= ceil(N/64) are not written.
 * With SPIN_REDUCE_A2 the states are block-level (see spin_config.flags):
 * S[r][row][j] = C(V[j], D[floor(q_row / 64) - j]); v_max is ignored.
 */
spin_status spin_predict_blocks(const spin_config* cfg, const spin_batch* bt,
                                const float* V, int64_t v_ld, const float* D, int64_t d_ld,
                                const float* v_max, float* S, void* stream);

/*
 * Stage 2 (Algorithm 1 steps 4-5; the sink and newest blocks are always kept
 * and count toward the budget; Sec. 3.2.1 exploration share; Sec. 3.2.2 union).
 * Per row: m = min(B, max(ceil(K/64), ceil((10000 - rho_bp) B / 10000))), or
 * min(B, budget[r]) when budget != NULL and budget[r] > 0; forced = {0, B-1};
 * n_e = min(floor(m gamma_bp / 10000), m - n_f); ranked = the m - n_f - n_e
 * remaining blocks with the largest S (ties: lower block); explored = the n_e
 * blocks neither forced nor ranked with the smallest Philox4x32-10 word 0 of
 * counter (j, step, layer, req_id) under key (seed lo, seed hi) (ties: lower
 * block).  step == 0 selects every block (dense warm-up).
 *   budget:   optional i32 [R]
 *   last_obs: optional i32 [R][max_blocks], the step at which each block was
 *             last in the scored union (all 0 after a reset: the dense first
 *             step observes every block); required by the age and staleness
 *             exploration policies.  When given, every block of this step's
 *             union gets step[r].
 *   row_code: u8 [R][n_rows][max_blocks] (SPIN_CODE_*; entries j >= B not written)
 *   sel:      i32 [R][max_blocks] ascending union of the rows' masks, -1 padded
 *   n_sel:    i32 [R] union size
 * Block reduction A0 is refused here (SPIN_E_UNSUPPORTED): it runs in spin_step.
 */
spin_status spin_select_blocks(const spin_config* cfg, const spin_batch* bt, const float* S,
                               const int32_t* budget, int32_t* last_obs, uint8_t* row_code,
                               int32_t* sel, int32_t* n_sel, void* stream);

/*
 * Stage 3a (Sec. 2): z[r][row][64k + s] = sum_h w[r][row][h] ReLU(q[r][row][h] . key(i))
 * for slot i = 64 sel[r][k] + s, k < n_sel[r]; key(i) = k_pages[page_table[r][i/64]][i%64]
 * (times k_scale[page][i%64] for fp8 keys).  Slots i >= N get z = 0.
 *   q:          [R][n_rows][n_heads][head_dim] of cfg->q_dtype
 *   w:          f32 [R][n_rows][n_heads]
 *   k_pages:    [n_pages][64][head_dim] of cfg->key_dtype (fp8 = OCP E4M3 codes)
 *   k_scale:    f32 [n_pages][64], non-negative; required for fp8 keys, else ignored
 *   page_table: i32 [R][pt_ld], pt_ld >= max_blocks
 *   z:          f32 [R][n_rows][z_ld], z_ld >= 64 * max_blocks
 *   workspace:  optional, the layer's top-K workspace (spin_workspace_bytes()).
 *               With it the call runs the kernel spin_step runs, which also
 *               writes the slots at or above each row's top-K threshold hint
 *               into the workspace's candidate lists; z is the same either way.
 * Supported (key, q) dtypes: (f32, f32), (bf16, bf16), (fp8, bf16), (fp8, f32).
 */
spin_status spin_sparse_index_score(const spin_config* cfg, const spin_batch* bt, const void* q,
                                    const float* w, const void* k_pages, const float* k_scale,
                                    const int32_t* page_table, int64_t pt_ld, const int32_t* sel,
                                    const int32_t* n_sel, float* z, int64_t z_ld, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * Stage 3b (Algorithm 1 step 7): per row, the min(K, |dom|) slots of dom(z)
 * (selected slots < N) with the largest z (ties: lower slot), written in
 * ascending slot order and padded with -1.
 *   topk_idx: i32 [R][n_rows][K]
 *   workspace: device scratch of spin_workspace_bytes() bytes (may be NULL when
 *              that function returns 0)
 */
spin_status spin_topk(const spin_config* cfg, const spin_batch* bt, const float* z, int64_t z_ld,
                      const int32_t* sel, const int32_t* n_sel, int32_t* topk_idx,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Stage 4 (Algorithm 1 steps 8-10; Sec. 3.2.2 deferred in-order replay).
 * For rows r = 0 .. L-1 in order (L = n_valid[req], or n_rows when n_valid is
 * NULL) and every slot i of dom(z):
 *   V[i]         <- (alpha * V[i])         + (beta * z_r[i])
 *   D[q_r - i]   <- (alpha * D[q_r - i])   + (beta * z_r[i])
 * each product and the sum rounded to fp32 separately (no fused multiply-add),
 * beta = 1.0f - alpha rounded to fp32.
 *   n_valid: optional i32 [R], each in 1..n_rows
 *   v_max:   optional f32 [R][max_blocks]: the updated blocks' V maxima are
 *            refreshed (see spin_predict_blocks)
 * With SPIN_REDUCE_A2 the update is block-level: for each selected block j
 * and row r in order, with p the pooled z of its valid slots (the pooling
 * flag's rule), V[j] <- (alpha V[j]) + (beta p) and D[floor(q_r / 64) - j]
 * likewise.
 */
spin_status spin_ema_update(const spin_config* cfg, const spin_batch* bt, const float* z,
                            int64_t z_ld, const int32_t* sel, const int32_t* n_sel,
                            const int32_t* n_valid, float* V, int64_t v_ld, float* D, int64_t d_ld,
                            float* v_max, void* stream);

/*
 * Advance the per-request counters after a committed step:
 * q_pos[r] += n_valid ? n_valid[r] : n_rows; step[r] += 1.
 */
spin_status spin_advance(int32_t batch, int32_t n_rows, const int32_t* n_valid, int32_t* q_pos,
                         int32_t* step, void* stream);

/*
 * Reset after prefill or at a turn start (prose after Algorithm 1): V[r][0..v_ld),
 * D[r][0..d_ld) = 0, v_max[r][0..vmax_ld) = 0 (when v_max != NULL) and step[r] = 0
 * for every r < batch, so the next step is dense.
 * Uses fill kernels only (safe inside captured graphs).
 */
spin_status spin_reset_state(int32_t batch, float* V, int64_t v_ld, float* D, int64_t d_ld,
                             float* v_max, int64_t vmax_ld, int32_t* step, void* stream);

/* Buffers of one whole step (spin_step).  Pointer meanings as above. */
typedef struct spin_step_io {
  float* V; int64_t v_ld;               /* EMA state, updated in place        */
  float* D; int64_t d_ld;
  float* v_max;                         /* optional V block maxima [R][max_blocks] */
  const void* q; const float* w;        /* indexer queries and head weights   */
  const void* k_pages; const float* k_scale;
  const int32_t* page_table; int64_t pt_ld;
  const int32_t* budget;                /* optional per-request block budget  */
  const int32_t* n_valid;               /* optional accepted rows per request */
  float* S;                             /* f32 [R][n_rows][max_blocks]        */
  uint8_t* row_code;                    /* u8  [R][n_rows][max_blocks]        */
  int32_t* sel; int32_t* n_sel;         /* i32 [R][max_blocks], i32 [R]       */
  float* z; int64_t z_ld;               /* f32 [R][n_rows][z_ld]              */
  int32_t* topk_idx;                    /* i32 [R][n_rows][K]                 */
  int32_t* q_pos_mut;                   /* optional: advanced after the EMA   */
  int32_t* step_mut;                    /* optional: advanced after the EMA   */
  void* workspace; size_t workspace_bytes;
  int32_t* last_obs;                    /* optional i32 [R][max_blocks]: see
                                           spin_select_blocks                 */
  int32_t* s_tag;                       /* with SPIN_PREDICT_AHEAD: i32 [R][4],
                                           caller-owned, -1 before the first
                                           step (none predicted ahead)        */
} spin_step_io;

/*
 * One whole decode step on `stream`: predict, select (+union), score, top-K
 * and, unless defer_ema != 0, the EMA update followed by spin_advance on
 * q_pos_mut / step_mut when those are non-NULL (they normally alias
 * bt->q_pos / bt->step).  With defer_ema != 0 the caller runs
 * spin_ema_update with the acceptance outcome and then spin_advance.
 */
spin_status spin_step(const spin_config* cfg, const spin_batch* bt, const spin_step_io* io,
                      int32_t defer_ema, void* stream);

/*
 * spin_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same step, bit for bit, with io->workspace and io->workspace_bytes ignored.
 * Its workspace is a static device array of SPIN_NOALLOC_WORKSPACE_BYTES
 * inside the library, one per GPU, held until the process ends; the call
 * itself allocates and frees nothing.  Shapes whose spin_workspace_bytes()
 * exceeds that size return SPIN_E_WORKSPACE.  Every call on a GPU shares that
 * GPU's array and its contents carry over between calls (only top-K
 * threshold hints, which change speed, not results), so calls that may
 * overlap on one GPU -- on different streams, or from different threads --
 * race and must not be issued; issue them on one stream, or use spin_step
 * with a workspace per caller.
 */
#define SPIN_NOALLOC_WORKSPACE_BYTES (160u * 1024u * 1024u)
spin_status spin_step_noalloc(const spin_config* cfg, const spin_batch* bt,
                              const spin_step_io* io, int32_t defer_ema, void* stream);

/*
 * The two halves of spin_step, for callers that overlap them.  Block
 * prediction needs only the EMA state, not the current query, so it can be
 * scheduled off the critical path (paper Sec. 3.2, after Eq. 2; blog, "Score
 * only where history points").
 * spin_step_plan: predict and select (+ union) into io->S, row_code, sel,
 *   n_sel, and the step's q_pos snapshot in the workspace.  Reads V, D,
 *   v_max, budget and the bt counters; never q, w or the key pages.
 * spin_step_finish: score, top-K and (defer_ema == 0) the EMA update +
 *   counter advance, exactly as the rest of spin_step.  It must run after
 *   the same step's spin_step_plan (same io), ordered by stream or event.
 * spin_step_plan then spin_step_finish on one stream is spin_step.
 */
spin_status spin_step_plan(const spin_config* cfg, const spin_batch* bt, const spin_step_io* io,
                           void* stream);
spin_status spin_step_finish(const spin_config* cfg, const spin_batch* bt,
                             const spin_step_io* io, int32_t defer_ema, void* stream);

/*
 * Multi-layer decode step with the plan of every layer on a side stream,
 * overlapped with the scoring of other layers (paper Sec. 3.2, after Eq. 2:
 * prediction and EMA upkeep may run asynchronously beside the other layers'
 * forward pass).  A spin_stack holds a few host events; it is created once
 * per model and reused every decode step.
 * spin_stack_step(stack, n, cfgs, bts, ios, order_after_main, main, side)
 * runs one decode step of layers 0 .. n-1 (each with its own EMA state,
 * counters, buffers and workspace).  The layers form two groups, A = [0, h)
 * and B = [h, n) with h = ceil(n / 2):
 *   side: after the previous call's finishes of group A, the plans of A;
 *         after all of the previous call's finishes, the plans of B
 *   main: after the plans of A, the finishes of A (score, top-K, EMA);
 *         after the plans of B, the finishes of B
 * so group A's plans run beside the previous step's group-B scoring and
 * group B's beside this step's group-A scoring, with two cross-stream waits
 * on main per step.  With ema_stream != NULL the finishes on main are score +
 * top-K only, and each group's EMA updates + counter advances run on
 * ema_stream after the group's finishes; the plans then wait for the
 * previous call's EMA of their group instead of its finishes.  Every layer
 * sees the same results as n spin_step calls in layer order.  The plans also
 * read the caller's ctx_len, req_id and budget: when the caller has written
 * any of them on `main` since the previous call (or reset a layer there), it
 * passes order_after_main != 0, and the side stream first waits for all work
 * issued on `main` before this call.  The streams must differ and belong to
 * the stack's device; the call returns without waiting.  The caller's later
 * work on `main` is ordered after every layer's top-K; without ema_stream
 * also after every EMA update, with it the caller makes `main` wait for
 * ema_stream before it reads or writes a layer's EMA state or counters.
 * With defer_ema != 0 (speculative decoding, paper Sec. 3.2.2: the updates
 * wait for the verification outcome) the finishes are score + top-K only and
 * the caller then calls spin_stack_commit once the accepted rows are known
 * (ios[l].n_valid); the next spin_stack_step is refused until it has.  Not
 * with ema_stream.
 * With side_stream == NULL (and ema_stream == NULL) everything runs on `main`
 * in layer order, with no events: layer l + 1's plan runs inside layer l's
 * two launches -- its prediction in the last workgroups of the score launch,
 * which start as the scoring workgroups leave their CUs, its selection in
 * the last workgroups of the top-K + EMA launch -- when layer l's keys are
 * fp8 or bf16 (its score kernel filters the top-K candidates) and layer l + 1
 * has one verifier row; otherwise layer l + 1's plan is issued on its own
 * before its finish.  Layer 0's plan always is.  order_after_main is then
 * moot.  A stack may alternate between the forms from call to call (a
 * one-stream call after one with an EMA stream first waits for those EMA
 * updates).  The one-stream form issues kernels only (no events), so a
 * caller may capture it in a HIP graph.
 * Errors: SPIN_E_SHAPE when n is < 1 or exceeds the stack's layers, two
 * streams are the same, or ema_stream is given without side_stream; each
 * layer's arguments are validated as for spin_step before anything is
 * issued.
 */
typedef struct spin_stack spin_stack;
spin_status spin_stack_create(int32_t n_layers, spin_stack** out);
void spin_stack_destroy(spin_stack* stack);
spin_status spin_stack_step(spin_stack* stack, int32_t n_layers, const spin_config* cfgs,
                            const spin_batch* bts, const spin_step_io* ios,
                            int32_t order_after_main, int32_t defer_ema, void* main_stream,
                            void* side_stream, void* ema_stream);
/*
 * The deferred EMA updates of the last spin_stack_step (defer_ema != 0), on
 * main_stream, in layer order: each layer replays its rows 0 .. n_valid - 1
 * in row order (ios[l].n_valid, or every row when NULL) and advances its
 * counters, exactly as spin_ema_update + spin_advance after that layer's
 * deferred spin_step (paper Sec. 3.2.2).  n_layers and the ios must be the
 * step's (the q positions come from the step's snapshot in each workspace).
 * Errors: SPIN_E_SHAPE when the last step did not defer, or n_layers differs.
 */
spin_status spin_stack_commit(spin_stack* stack, int32_t n_layers, const spin_config* cfgs,
                              const spin_batch* bts, const spin_step_io* ios,
                              void* main_stream);

/*
 * Per-layer block budgets (blog "Sparse Attention Still Has a Dense Problem",
 * section "Per-layer block budgets": every P steps a dense probe step measures
 * each layer's miss curve -- the share of the dense top-K slots that fall in
 * skipped blocks, at each budget -- and the budgets are re-sized per layer at
 * a fixed total, minimising the worst layer's miss rate, into a device-side
 * table).  A budget is a level g in 0 .. levels (levels divides 10000): the
 * blocks the selection keeps at target sparsity 10000 - (10000/levels) g bp,
 * at least ceil(K/64) and at most B.
 *
 * spin_miss_curve: after a dense step (every block selected, e.g. budget B),
 *   from that step's predicted scores S (f32 [R][n_rows][max_blocks], as the
 *   plan left them) and dense top-K (i32 [R][n_rows][K], -1 padded):
 *   covered[r][row][g] = top-K slots inside the blocks kept at level g
 *   without exploration (the forced blocks and the first m - n_f - n_e
 *   others by S desc, lower block first), g = 0 .. levels;
 *   kprime[r][row] = valid top-K slots.  Device buffers; max_blocks <= 8192.
 * spin_budget_fill: budget[r] (i32 [R], the selection's budget override) =
 *   the blocks of level level_table[0] (device i32) for request r.  Reading
 *   the level on the device keeps the table usable from captured graphs.
 * spin_budget_allocate (host only, no device work): per-layer levels from
 *   covered / total (i64 [L][levels + 1] and [L], summed over a layer's
 *   requests and rows) with sum_l level_l = L * target_level:
 *   SPIN_BUDGET_MINIMAX raises, one level at a time, the layer with the
 *   largest miss rate (1 - covered/total at its level; ties: lower layer)
 *   from all-zero levels; SPIN_BUDGET_PROPORTIONAL shares the levels in
 *   proportion to running_miss[l] + 1e-3 (f64 [L]), clamped to [0, levels],
 *   integer parts plus one level to the largest fractional parts (ties: lower
 *   layer).  covered/total may be NULL for the proportional rule,
 *   running_miss for minimax.
 */
enum { SPIN_BUDGET_MINIMAX = 0, SPIN_BUDGET_PROPORTIONAL = 1 };
spin_status spin_miss_curve(const spin_config* cfg, const spin_batch* bt, const float* S,
                            const int32_t* topk_idx, int32_t levels, int32_t* covered,
                            int32_t* kprime, void* stream);
spin_status spin_budget_fill(const spin_config* cfg, const spin_batch* bt,
                             const int32_t* level_table, int32_t levels, int32_t* budget,
                             void* stream);
spin_status spin_budget_allocate(int32_t policy, int32_t n_layers, int32_t levels,
                                 int32_t target_level, const int64_t* covered,
                                 const int64_t* total, const double* running_miss,
                                 int32_t* level_out);

/*
 * The per-layer budget policy run by a spin_stack itself (blog, "Per-layer
 * block budgets": a dense probe every P steps measures each layer's miss
 * curve, and the budgets are re-sized at a fixed total and published to a
 * device-side table whenever the curves drift).  With a policy set, spin_stack_step
 *   - counts its calls since spin_stack_reset_budgets; call t = P, 2P, ... is
 *     a probe: every layer selects every block (probe_budget);
 *   - otherwise layer l selects with budget[l] (its level in level_table[l],
 *     filled by spin_budget_fill); the ios' own budget pointers are ignored;
 *   - after a probe call's finishes, on the main stream: each layer's miss
 *     curve (spin_miss_curve into covered / kprime), then one device kernel
 *     that sums the curves over requests and rows, updates the running miss
 *     rates (state) and, unless drift_bp > 0 and no layer's miss rate at any
 *     level moved by more than drift_bp / 10000 since the curves of the last
 *     publication (the first probe always publishes), writes the new levels
 *     into level_table -- the same arithmetic as spin_budget_allocate -- then
 *     each layer's budget fill.
 *     The next call selects with them; nothing waits for the host.
 * Every layer of the stack takes part (n_layers of the stack), with the same
 * batch and n_rows; defer_ema is not available with a policy.  Buffers are
 * device memory owned by the caller:
 *   level_table i32 [n_layers]; budget i32 [n_layers][batch];
 *   probe_budget i32 [batch]; covered i32 [n_layers][batch][n_rows][levels + 1];
 *   kprime i32 [n_layers][batch][n_rows]; state: spin_budget_state_bytes().
 * spin_stack_set_budget_policy copies the struct (NULL: no policy).
 * spin_stack_reset_budgets (with the layers' reset, and after their contexts
 * change) sets every level to target_level, clears the probe history and
 * fills the budgets, on main_stream.
 */
typedef struct spin_budget_policy {
  int32_t policy;        /* SPIN_BUDGET_MINIMAX | SPIN_BUDGET_PROPORTIONAL          */
  int32_t probe_period;  /* P >= 1                                                  */
  int32_t levels;        /* divides 10000                                           */
  int32_t target_level;  /* 0 .. levels; the level sum is n_layers * target_level  */
  int32_t drift_bp;      /* 0 .. 10000: publish only past this drift (0: always)    */
  int32_t* level_table;
  int32_t* budget;
  int32_t* probe_budget;
  int32_t* covered;
  int32_t* kprime;
  void* state;
} spin_budget_policy;
size_t spin_budget_state_bytes(int32_t n_layers, int32_t levels);
/*
 * The device step of the policy on its own, for callers with their own
 * schedule: from the curves of one probe (covered i32 [n_layers][rows_total]
 * [levels + 1], kprime i32 [n_layers][rows_total], rows_total = batch x
 * n_rows), on `stream`: per layer the sums over its rows, then
 *   SPIN_BUDGET_MINIMAX: the greedy minimax allocation of spin_budget_allocate;
 *   SPIN_BUDGET_PROPORTIONAL: each layer's miss rate at its current level
 *     (level_table on entry) added to its running sum in `state`, the probe
 *     count incremented, and the proportional allocation of the running means;
 * new levels into level_table, which is left as it is when drift_bp > 0 and
 * no miss rate of any layer at any level moved by more than drift_bp / 10000
 * from the curves of the last call that wrote it (the first call always
 * writes; the running miss rates advance either way).  state
 * (spin_budget_state_bytes()) must be zero before the first probe.  No host
 * synchronisation.  drift_bp outside [0, 10000]: SPIN_E_SHAPE.
 */
spin_status spin_budget_update(int32_t policy, int32_t n_layers, int32_t levels,
                               int32_t target_level, int32_t drift_bp, int32_t rows_total,
                               const int32_t* covered, const int32_t* kprime, void* state,
                               int32_t* level_table, void* stream);
spin_status spin_stack_set_budget_policy(spin_stack* stack, const spin_budget_policy* policy);
spin_status spin_stack_reset_budgets(spin_stack* stack, int32_t n_layers, const spin_config* cfgs,
                                     const spin_batch* bts, void* main_stream);

/*
 * Device workspace bytes spin_topk / spin_step need for this shape.  The
 * buffer holds the top-K threshold hints and candidate lists (any initial
 * contents are valid: a hint only changes speed) followed, for spin_step, by
 * the step's q_pos snapshot that lets one kernel run the EMA update and the
 * counter advance together.  One workspace per layer; calls that share a
 * workspace must not overlap.
 */
size_t spin_workspace_bytes(const spin_config* cfg, int32_t batch, int32_t n_rows,
                            int32_t max_blocks);

/* Message for the last non-OK status returned on the calling thread (host string). */
const char* spin_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SPIN_H_ */
