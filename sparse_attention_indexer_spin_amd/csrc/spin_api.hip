// C ABI of the SPIN decode-step library: argument validation, error
// reporting, and stream-ordered launches of the stage kernels.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <memory>
#include <mutex>
#include <utility>
#include <vector>

#include "spin_launch.h"
#include "spin_probe.h"

namespace {

thread_local char g_err[512] = "";

spin_status fail(spin_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

spin_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SPIN_OK;
  return fail(SPIN_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define SPIN_REQUIRE(ptr)                                                 \
  do {                                                                    \
    if (!(ptr)) return fail(SPIN_E_NULL, "%s: %s is NULL", fn, #ptr);     \
  } while (0)

spin_status check_config(const char* fn, const spin_config* c) {
  if (!c) return fail(SPIN_E_NULL, "%s: cfg is NULL", fn);
  if (c->block_size != SPIN_BLOCK)
    return fail(SPIN_E_UNSUPPORTED, "%s: block_size %d (only 64 is supported)", fn, c->block_size);
  if (c->n_heads != 64 || c->head_dim != 128)
    return fail(SPIN_E_UNSUPPORTED, "%s: n_heads=%d head_dim=%d (this build: 64 x 128)", fn,
                c->n_heads, c->head_dim);
  if (c->topk < 1 || c->topk > SPIN_MAX_TOPK)
    return fail(SPIN_E_SHAPE, "%s: topk %d outside [1, %d]", fn, c->topk, SPIN_MAX_TOPK);
  if (c->sparsity_bp < 0 || c->sparsity_bp > 10000 || c->explore_bp < 0 || c->explore_bp > 10000)
    return fail(SPIN_E_SHAPE, "%s: sparsity_bp/explore_bp outside [0, 10000]", fn);
  if (!(c->ema_alpha >= 0.0f && c->ema_alpha <= 1.0f))
    return fail(SPIN_E_SHAPE, "%s: ema_alpha outside [0, 1]", fn);
  if (c->combine != SPIN_COMBINE_MAX && c->combine != SPIN_COMBINE_SUM)
    return fail(SPIN_E_SHAPE, "%s: unknown combine %d", fn, c->combine);
  if (c->key_dtype < SPIN_F32 || c->key_dtype > SPIN_FP8_E4M3 || c->q_dtype < SPIN_F32 ||
      c->q_dtype > SPIN_BF16)
    return fail(SPIN_E_UNSUPPORTED, "%s: unknown dtype", fn);
  if ((c->flags & ~SPIN_FLAGS_ALL) != 0 || (c->flags & SPIN_POOL_MASK) == SPIN_POOL_MASK ||
      (c->flags & SPIN_EXPLORE_POLICY_MASK) == SPIN_EXPLORE_POLICY_MASK ||
      (c->flags & SPIN_REDUCE_MASK) == SPIN_REDUCE_MASK)
    return fail(SPIN_E_SHAPE, "%s: unknown flags 0x%x", fn, c->flags);
  if ((c->flags & SPIN_EXPLORE_PER_ROW) && (c->layer < 0 || c->layer >= 65536))
    return fail(SPIN_E_SHAPE, "%s: per-row exploration needs 0 <= layer < 65536", fn);
  if ((c->flags & SPIN_PREDICT_AHEAD) && (c->flags & SPIN_REDUCE_MASK) != 0)
    return fail(SPIN_E_SHAPE, "%s: SPIN_PREDICT_AHEAD needs block reduction A1", fn);
  return SPIN_OK;
}

spin_status check_batch(const char* fn, const spin_batch* b) {
  if (!b) return fail(SPIN_E_NULL, "%s: batch is NULL", fn);
  if (b->batch < 0 || b->batch > SPIN_MAX_BATCH)
    return fail(SPIN_E_SHAPE, "%s: batch %d outside [0, %d]", fn, b->batch, SPIN_MAX_BATCH);
  if (b->n_rows < 1 || b->n_rows > SPIN_MAX_ROWS)
    return fail(SPIN_E_SHAPE, "%s: n_rows %d outside [1, %d]", fn, b->n_rows, SPIN_MAX_ROWS);
  if (b->max_blocks < 1 || b->max_blocks > SPIN_MAX_BLOCKS)
    return fail(SPIN_E_SHAPE, "%s: max_blocks %d outside [1, %d]", fn, b->max_blocks,
                SPIN_MAX_BLOCKS);
  if (b->batch > 0) {
    SPIN_REQUIRE(b->ctx_len);
    SPIN_REQUIRE(b->q_pos);
    SPIN_REQUIRE(b->step);
    SPIN_REQUIRE(b->req_id);
  }
  return SPIN_OK;
}

#define SPIN_CHECK(expr)                 \
  do {                                   \
    spin_status _s = (expr);             \
    if (_s != SPIN_OK) return _s;        \
  } while (0)

spin_status check_state(const char* fn, const spin_batch* b, const float* V, int64_t v_ld,
                        const float* D, int64_t d_ld) {
  SPIN_REQUIRE(V);
  SPIN_REQUIRE(D);
  if (v_ld < 1 || d_ld < 2) return fail(SPIN_E_SHAPE, "%s: v_ld/d_ld too small", fn);
  (void)b;
  return SPIN_OK;
}

spin_status check_z(const char* fn, const spin_batch* b, const float* z, int64_t z_ld) {
  SPIN_REQUIRE(z);
  if (z_ld < (int64_t)SPIN_BLOCK * b->max_blocks || (z_ld & 3))
    return fail(SPIN_E_SHAPE, "%s: z_ld %lld must be >= 64*max_blocks and a multiple of 4", fn,
                (long long)z_ld);
  return SPIN_OK;
}

bool reduce_a0(const spin_config& c) { return (c.flags & SPIN_REDUCE_MASK) == SPIN_REDUCE_A0; }
bool reduce_a2(const spin_config& c) { return (c.flags & SPIN_REDUCE_MASK) == SPIN_REDUCE_A2; }
bool explore_needs_obs(const spin_config& c) {
  return (c.flags & SPIN_EXPLORE_POLICY_MASK) != 0;
}

}  // namespace

namespace spin {

int resident_workgroups(const void* kernel, int threads, size_t dyn_lds) {
  static std::mutex mu;
  static std::map<std::pair<std::pair<int, const void*>, size_t>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_pair(std::make_pair(dev, kernel), dyn_lds);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, dyn_lds) != hipSuccess ||
      per < 1)
    per = 1;
  const int g = per * cus;
  cache[key] = g;
  return g;
}

bool lds_fits(const void* kernel, size_t dyn_lds) {
  static std::mutex mu;
  static std::map<std::pair<std::pair<int, const void*>, size_t>, bool> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_pair(std::make_pair(dev, kernel), dyn_lds);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int max_lds = 0;
  hipFuncAttributes fa{};
  const bool ok =
      hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) ==
          hipSuccess &&
      hipFuncGetAttributes(&fa, kernel) == hipSuccess &&
      dyn_lds + fa.sharedSizeBytes <= (size_t)max_lds &&
      (fa.maxDynamicSharedSizeBytes <= 0 || dyn_lds <= (size_t)fa.maxDynamicSharedSizeBytes);
  cache[key] = ok;
  return ok;
}

}  // namespace spin

extern "C" {

const char* spin_last_error(void) { return g_err; }

spin_status spin_read_pages(const void* k_pages, int64_t n_pages, const int32_t* page_ids,
                            int32_t n_ids, uint32_t* sink, void* stream) {
  const char* fn = "spin_read_pages";
  if (!k_pages || !page_ids || !sink) return fail(SPIN_E_NULL, "%s: NULL buffer", fn);
  if (n_ids < 0 || n_pages < 1)
    return fail(SPIN_E_SHAPE, "%s: n_ids %d, n_pages %lld", fn, n_ids, (long long)n_pages);
  if (n_ids == 0) return SPIN_OK;
  return hip_status(spin::launch_read_pages(k_pages, n_pages, page_ids, n_ids, sink,
                                            (hipStream_t)stream), fn);
}

size_t spin_workspace_bytes(const spin_config* cfg, int32_t batch, int32_t n_rows,
                            int32_t max_blocks) {
  if (!cfg) return 0;
  return spin::step_workspace_bytes(*cfg, batch, n_rows, max_blocks);
}

spin_status spin_predict_blocks(const spin_config* cfg, const spin_batch* bt, const float* V,
                                int64_t v_ld, const float* D, int64_t d_ld, const float* v_max,
                                float* S, void* stream) {
  const char* fn = "spin_predict_blocks";
  SPIN_CHECK(check_config(fn, cfg));
  SPIN_CHECK(check_batch(fn, bt));
  SPIN_CHECK(check_state(fn, bt, V, v_ld, D, d_ld));
  SPIN_REQUIRE(S);
  if (bt->batch == 0) return SPIN_OK;
  if (reduce_a2(*cfg))
    return hip_status(spin::launch_predict_a2(*cfg, *bt, V, v_ld, D, d_ld, S,
                                              (hipStream_t)stream), fn);
  return hip_status(spin::launch_predict(*cfg, *bt, V, v_ld, D, d_ld, v_max, S, (hipStream_t)stream),
                    fn);
}

spin_status spin_select_blocks(const spin_config* cfg, const spin_batch* bt, const float* S,
                               const int32_t* budget, int32_t* last_obs, uint8_t* row_code,
                               int32_t* sel, int32_t* n_sel, void* stream) {
  const char* fn = "spin_select_blocks";
  SPIN_CHECK(check_config(fn, cfg));
  SPIN_CHECK(check_batch(fn, bt));
  SPIN_REQUIRE(S);
  SPIN_REQUIRE(row_code);
  SPIN_REQUIRE(sel);
  SPIN_REQUIRE(n_sel);
  if (reduce_a0(*cfg))
    return fail(SPIN_E_UNSUPPORTED, "%s: block reduction A0 selects from predicted slot scores; "
                "it runs in spin_step / spin_step_plan", fn);
  if (explore_needs_obs(*cfg)) SPIN_REQUIRE(last_obs);
  if (bt->batch == 0) return SPIN_OK;
  return hip_status(spin::launch_select(*cfg, *bt, S, budget, row_code, sel, n_sel, last_obs,
                                        (hipStream_t)stream), fn);
}

static spin_status check_score_args(const char* fn, const spin_config* cfg, const spin_batch* bt,
                                    const void* q, const float* w, const void* k_pages,
                                    const float* k_scale, const int32_t* page_table,
                                    int64_t pt_ld, const int32_t* sel, const int32_t* n_sel,
                                    const float* z, int64_t z_ld) {
  SPIN_REQUIRE(q);
  SPIN_REQUIRE(w);
  SPIN_REQUIRE(k_pages);
  SPIN_REQUIRE(page_table);
  SPIN_REQUIRE(sel);
  SPIN_REQUIRE(n_sel);
  SPIN_CHECK(check_z(fn, bt, z, z_ld));
  if (pt_ld < bt->max_blocks) return fail(SPIN_E_SHAPE, "%s: pt_ld < max_blocks", fn);
  if (bt->n_pages < 1) return fail(SPIN_E_SHAPE, "%s: n_pages < 1", fn);
  const int kd = cfg->key_dtype, qd = cfg->q_dtype;
  const bool ok = (kd == SPIN_F32 && qd == SPIN_F32) || (kd == SPIN_BF16 && qd == SPIN_BF16) ||
                  (kd == SPIN_FP8_E4M3 && (qd == SPIN_BF16 || qd == SPIN_F32));
  if (!ok) return fail(SPIN_E_UNSUPPORTED, "%s: key/query dtype pair (%d, %d) not built", fn, kd, qd);
  if (kd == SPIN_FP8_E4M3) SPIN_REQUIRE(k_scale);
  return SPIN_OK;
}

spin_status spin_sparse_index_score(const spin_config* cfg, const spin_batch* bt, const void* q,
                                    const float* w, const void* k_pages, const float* k_scale,
                                    const int32_t* page_table, int64_t pt_ld, const int32_t* sel,
                                    const int32_t* n_sel, float* z, int64_t z_ld, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  const char* fn = "spin_sparse_index_score";
  SPIN_CHECK(check_config(fn, cfg));
  SPIN_CHECK(check_batch(fn, bt));
  SPIN_CHECK(check_score_args(fn, cfg, bt, q, w, k_pages, k_scale, page_table, pt_ld, sel, n_sel,
                              z, z_ld));
  if (workspace) {
    const size_t need = spin::topk_workspace_bytes(*cfg, bt->batch, bt->n_rows, bt->max_blocks);
    if (workspace_bytes < need)
      return fail(SPIN_E_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  }
  if (bt->batch == 0) return SPIN_OK;
  // with a workspace: the kernel spin_step runs, which also filters the
  // top-K candidates into it
  const spin::CandSink sink =
      workspace ? spin::topk_sink(workspace, bt->batch, bt->n_rows, bt->max_blocks)
                : spin::CandSink{};
  return hip_status(spin::launch_score(*cfg, *bt, q, w, k_pages, k_scale, page_table, pt_ld, sel,
                                       n_sel, z, z_ld, (hipStream_t)stream,
                                       workspace ? &sink : nullptr),
                    fn);
}

spin_status spin_topk(const spin_config* cfg, const spin_batch* bt, const float* z, int64_t z_ld,
                      const int32_t* sel, const int32_t* n_sel, int32_t* topk_idx,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "spin_topk";
  SPIN_CHECK(check_config(fn, cfg));
  SPIN_CHECK(check_batch(fn, bt));
  SPIN_CHECK(check_z(fn, bt, z, z_ld));
  SPIN_REQUIRE(sel);
  SPIN_REQUIRE(n_sel);
  SPIN_REQUIRE(topk_idx);
  const size_t need = spin::topk_workspace_bytes(*cfg, bt->batch, bt->n_rows, bt->max_blocks);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(SPIN_E_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  if (bt->batch == 0) return SPIN_OK;
  return hip_status(spin::launch_topk(*cfg, *bt, z, z_ld, sel, n_sel, topk_idx, workspace,
                                      workspace_bytes, (hipStream_t)stream), fn);
}

spin_status spin_ema_update(const spin_config* cfg, const spin_batch* bt, const float* z,
                            int64_t z_ld, const int32_t* sel, const int32_t* n_sel,
                            const int32_t* n_valid, float* V, int64_t v_ld, float* D, int64_t d_ld,
                            float* v_max, void* stream) {
  const char* fn = "spin_ema_update";
  SPIN_CHECK(check_config(fn, cfg));
  SPIN_CHECK(check_batch(fn, bt));
  SPIN_CHECK(check_z(fn, bt, z, z_ld));
  SPIN_CHECK(check_state(fn, bt, V, v_ld, D, d_ld));
  SPIN_REQUIRE(sel);
  SPIN_REQUIRE(n_sel);
  if (bt->batch == 0) return SPIN_OK;
  if (reduce_a2(*cfg))
    return hip_status(spin::launch_ema_a2(*cfg, *bt, z, z_ld, sel, n_sel, n_valid, V, v_ld, D,
                                          d_ld, (hipStream_t)stream), fn);
  return hip_status(spin::launch_ema(*cfg, *bt, z, z_ld, sel, n_sel, n_valid, V, v_ld, D, d_ld,
                                     v_max, (hipStream_t)stream), fn);
}

spin_status spin_advance(int32_t batch, int32_t n_rows, const int32_t* n_valid, int32_t* q_pos,
                         int32_t* step, void* stream) {
  const char* fn = "spin_advance";
  if (batch < 0 || n_rows < 1 || n_rows > SPIN_MAX_ROWS)
    return fail(SPIN_E_SHAPE, "%s: batch %d / n_rows %d invalid", fn, batch, n_rows);
  if (batch == 0 || (!q_pos && !step)) return SPIN_OK;
  return hip_status(spin::launch_advance(batch, n_rows, n_valid, q_pos, step, (hipStream_t)stream),
                    fn);
}

spin_status spin_reset_state(int32_t batch, float* V, int64_t v_ld, float* D, int64_t d_ld,
                             float* v_max, int64_t vmax_ld, int32_t* step, void* stream) {
  const char* fn = "spin_reset_state";
  if (batch < 0 || v_ld < 0 || d_ld < 0 || vmax_ld < 0)
    return fail(SPIN_E_SHAPE, "%s: negative size", fn);
  if (batch == 0) return SPIN_OK;
  if ((v_ld > 0 && !V) || (d_ld > 0 && !D)) return fail(SPIN_E_NULL, "%s: V or D is NULL", fn);
  return hip_status(spin::launch_reset(batch, V, v_ld, D, d_ld, v_max ? vmax_ld : 0, v_max, step,
                                       (hipStream_t)stream), fn);
}

}  // extern "C"

namespace {

spin_status check_step(const char* fn, const spin_config* cfg, const spin_batch* bt,
                       const spin_step_io* io) {
  SPIN_CHECK(check_config(fn, cfg));
  SPIN_CHECK(check_batch(fn, bt));
  SPIN_REQUIRE(io);
  SPIN_CHECK(check_state(fn, bt, io->V, io->v_ld, io->D, io->d_ld));
  SPIN_REQUIRE(io->S);
  SPIN_REQUIRE(io->row_code);
  SPIN_REQUIRE(io->topk_idx);
  SPIN_CHECK(check_score_args(fn, cfg, bt, io->q, io->w, io->k_pages, io->k_scale, io->page_table,
                              io->pt_ld, io->sel, io->n_sel, io->z, io->z_ld));
  const size_t need = spin::step_workspace_bytes(*cfg, bt->batch, bt->n_rows, bt->max_blocks);
  if (!io->workspace || io->workspace_bytes < need)
    return fail(SPIN_E_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  if (explore_needs_obs(*cfg)) SPIN_REQUIRE(io->last_obs);
  if (cfg->flags & SPIN_PREDICT_AHEAD) SPIN_REQUIRE(io->s_tag);
  return SPIN_OK;
}

// The step's q_pos snapshot: after the top-K region of the workspace (256-B aligned).
int32_t* step_qsnap(const spin_config& c, const spin_batch& b, const spin_step_io& io) {
  const size_t topk_bytes = spin::topk_workspace_bytes(c, b.batch, b.n_rows, b.max_blocks);
  return reinterpret_cast<int32_t*>(static_cast<char*>(io.workspace) +
                                    ((topk_bytes + 255) & ~size_t(255)));
}

bool ahead_on(const spin_config& c) { return (c.flags & SPIN_PREDICT_AHEAD) != 0; }

// With SPIN_PREDICT_AHEAD: each block's position in sel, written by the
// step's selection for its EMA, after the snapshot (256-B aligned).
int32_t* step_inv(const spin_config& c, const spin_batch& b, const spin_step_io& io) {
  if (!ahead_on(c)) return nullptr;
  const size_t snap = (size_t)4 * b.batch;
  return reinterpret_cast<int32_t*>(reinterpret_cast<char*>(step_qsnap(c, b, io)) +
                                    ((snap + 255) & ~size_t(255)));
}

const int32_t* step_tag(const spin_config& c, const spin_step_io& io) {
  return ahead_on(c) ? io.s_tag : nullptr;
}

// The step's EMA also predicts the next step's block scores (one verifier
// row), or nullptr.
const spin::Ahead* step_ahead(const spin_config& c, const spin_batch& b, const spin_step_io& io,
                              spin::Ahead& buf) {
  if (!ahead_on(c) || b.n_rows != 1) return nullptr;
  buf = spin::Ahead{step_inv(c, b, io), io.S, io.s_tag};
  return &buf;
}

// Predict + select (+ union), arguments already checked.
spin_status issue_plan(const spin_config& c, const spin_batch& b, const spin_step_io& io,
                       hipStream_t st) {
  if (reduce_a2(c)) {
    SPIN_CHECK(hip_status(spin::launch_predict_a2(c, b, io.V, io.v_ld, io.D, io.d_ld, io.S, st,
                                                  step_qsnap(c, b, io)),
                          "spin_step/predict(A2)"));
  } else {
    SPIN_CHECK(hip_status(spin::launch_predict(c, b, io.V, io.v_ld, io.D, io.d_ld, io.v_max,
                                               io.S, st, step_qsnap(c, b, io), step_tag(c, io)),
                          "spin_step/predict"));
  }
  if (reduce_a0(c)) {
    // A0: every slot's predicted score into z (all blocks listed), each
    // row's top-K of it into topk_idx, then the blocks holding them
    SPIN_CHECK(hip_status(spin::launch_predict_slots(c, b, io.V, io.v_ld, io.D, io.d_ld, io.z,
                                                     io.z_ld, io.sel, io.n_sel, st),
                          "spin_step/predict slots(A0)"));
    SPIN_CHECK(hip_status(spin::launch_topk(c, b, io.z, io.z_ld, io.sel, io.n_sel, io.topk_idx,
                                            io.workspace, io.workspace_bytes, st, false),
                          "spin_step/slot top-K(A0)"));
    return hip_status(spin::launch_a0_select(c, b, io.S, io.topk_idx, io.row_code, io.sel,
                                             io.n_sel, io.last_obs, st),
                      "spin_step/select(A0)");
  }
  return hip_status(spin::launch_select(c, b, io.S, io.budget, io.row_code, io.sel, io.n_sel,
                                        io.last_obs, st, step_inv(c, b, io)),
                    "spin_step/select");
}

// Score, top-K and (unless deferred) the EMA update + counter advance.
spin_status issue_finish(const spin_config& c, const spin_batch& b, const spin_step_io& io,
                         int32_t defer_ema, hipStream_t st) {
  int32_t* qsnap = step_qsnap(c, b, io);
  // where the score kernel can, it also applies the top-K threshold filter
  const bool prefilter = spin::score_filters(c, b);
  const spin::CandSink sink = spin::topk_sink(io.workspace, b.batch, b.n_rows, b.max_blocks);
  SPIN_CHECK(hip_status(spin::launch_score(c, b, io.q, io.w, io.k_pages, io.k_scale,
                                           io.page_table, io.pt_ld, io.sel, io.n_sel, io.z,
                                           io.z_ld, st, prefilter ? &sink : nullptr),
                        "spin_step/score"));
  if (reduce_a2(c)) {  // top-K, then the block-level EMA update + counter advance
    SPIN_CHECK(hip_status(spin::launch_topk(c, b, io.z, io.z_ld, io.sel, io.n_sel, io.topk_idx,
                                            io.workspace, io.workspace_bytes, st, prefilter),
                          "spin_step/topk"));
    if (defer_ema) return SPIN_OK;
    return hip_status(spin::launch_ema_a2(c, b, io.z, io.z_ld, io.sel, io.n_sel, io.n_valid, io.V,
                                          io.v_ld, io.D, io.d_ld, st, qsnap, io.q_pos_mut,
                                          io.step_mut),
                      "spin_step/ema+advance(A2)");
  }
  spin::Ahead abuf;
  const spin::Ahead* ahead = step_ahead(c, b, io, abuf);
  if (prefilter && !defer_ema)  // top-K beside the EMA update, one launch
    return hip_status(spin::launch_topk_ema(c, b, io.z, io.z_ld, io.sel, io.n_sel, io.topk_idx,
                                            io.workspace, io.n_valid, io.V, io.v_ld, io.D,
                                            io.d_ld, io.v_max, qsnap, io.q_pos_mut, io.step_mut,
                                            st, nullptr, true, ahead),
                      "spin_step/topk+ema");
  SPIN_CHECK(hip_status(spin::launch_topk(c, b, io.z, io.z_ld, io.sel, io.n_sel, io.topk_idx,
                                          io.workspace, io.workspace_bytes, st, prefilter),
                        "spin_step/topk"));
  if (defer_ema) return SPIN_OK;
  // EMA and counter advance in one kernel: it reads q positions from the
  // snapshot, so advancing q_pos_mut (normally the same array as b.q_pos)
  // cannot race with its reads
  return hip_status(spin::launch_ema(c, b, io.z, io.z_ld, io.sel, io.n_sel, io.n_valid, io.V,
                                     io.v_ld, io.D, io.d_ld, io.v_max, st, qsnap, io.q_pos_mut,
                                     io.step_mut, ahead),
                    "spin_step/ema+advance");
}

// Score, top-K and the EMA update + counter advance of one layer (its
// score kernel filters the top-K candidates), with the plan of layer `n`
// (one verifier row) run inside the same two launches: its prediction by the
// score launch's last workgroups, its selection by the top-K + EMA launch's.
// The two layers share no data.
spin_status issue_finish_with_plan(const spin_config& c, const spin_batch& b,
                                   const spin_step_io& io, const spin_config& nc,
                                   const spin_batch& nb, const spin_step_io& nio,
                                   int32_t defer_ema, hipStream_t st) {
  const spin::CandSink sink = spin::topk_sink(io.workspace, b.batch, b.n_rows, b.max_blocks);
  const spin::PredictPlan pp =
      spin::predict_plan(nc, nb, nio.V, nio.v_ld, nio.D, nio.d_ld, nio.v_max, nio.S,
                         step_qsnap(nc, nb, nio), step_tag(nc, nio));
  const spin::SelectPlan sp = spin::select_plan(nc, nb, nio.S, nio.budget, nio.row_code,
                                                nio.sel, nio.n_sel, nio.last_obs,
                                                step_inv(nc, nb, nio));
  spin::Ahead abuf;
  const spin::Ahead* ahead = step_ahead(c, b, io, abuf);
  SPIN_CHECK(hip_status(spin::launch_score(c, b, io.q, io.w, io.k_pages, io.k_scale,
                                           io.page_table, io.pt_ld, io.sel, io.n_sel, io.z,
                                           io.z_ld, st, &sink, &pp),
                        "spin_stack_step/score+predict"));
  return hip_status(spin::launch_topk_ema(c, b, io.z, io.z_ld, io.sel, io.n_sel, io.topk_idx,
                                          io.workspace, io.n_valid, io.V, io.v_ld, io.D,
                                          io.d_ld, io.v_max, step_qsnap(c, b, io),
                                          io.q_pos_mut, io.step_mut, st, &sp, !defer_ema, ahead),
                    "spin_stack_step/topk+ema+select");
}

// The EMA update + counter advance of a finished step (after a finish with
// defer_ema): q positions from the step's snapshot.
spin_status issue_ema(const spin_config& c, const spin_batch& b, const spin_step_io& io,
                      hipStream_t st) {
  if (reduce_a2(c))
    return hip_status(spin::launch_ema_a2(c, b, io.z, io.z_ld, io.sel, io.n_sel, io.n_valid, io.V,
                                          io.v_ld, io.D, io.d_ld, st, step_qsnap(c, b, io),
                                          io.q_pos_mut, io.step_mut),
                      "spin_stack_step/ema+advance(A2)");
  spin::Ahead abuf;
  return hip_status(spin::launch_ema(c, b, io.z, io.z_ld, io.sel, io.n_sel, io.n_valid, io.V,
                                     io.v_ld, io.D, io.d_ld, io.v_max, st, step_qsnap(c, b, io),
                                     io.q_pos_mut, io.step_mut, step_ahead(c, b, io, abuf)),
                    "spin_stack_step/ema+advance");
}

}  // namespace

// Host-side scheduler state of a multi-layer step.  The layers split into
// two groups, A = [0, h) and B = [h, n), h = ceil(n / 2); per group, the
// event of its last plans (side stream) and of its last finishes (main).
// Each cross-stream wait costs the waiting queue several microseconds even
// when the event has long completed, so main waits twice per step, not once
// per layer.
struct spin_stack {
  int32_t n_layers = 0;
  int device = 0;
  int32_t prev_h = 0;            // group split of the previous call
  bool one_stream_last = false;  // the previous call ran on one stream
  bool ema_stream_last = false;  // the previous call ran the EMA updates on an EMA stream
  bool commit_pending = false;   // the previous call deferred its EMA updates
  int32_t committed_layers = 0;  // layers of the previous call
  // per-layer budgets run by the stack (spin_stack_set_budget_policy)
  bool has_policy = false;
  spin_budget_policy policy{};
  int64_t budget_t = 0;          // calls since spin_stack_reset_budgets
  bool order_side = false;       // the last call wrote budgets on main after its finishes
  hipEvent_t plan_done[2] = {nullptr, nullptr};
  hipEvent_t finish_done[2] = {nullptr, nullptr};
  hipEvent_t ema_done[2] = {nullptr, nullptr};   // with an EMA stream
  hipEvent_t entry = nullptr;    // main at the call, for order_after_main
};

extern "C" {

static spin_status check_levels(const char* fn, int32_t levels) {
  if (levels < 1 || levels > 10000 || 10000 % levels != 0)
    return fail(SPIN_E_SHAPE, "%s: levels %d must divide 10000", fn, levels);
  return SPIN_OK;
}

spin_status spin_miss_curve(const spin_config* cfg, const spin_batch* bt, const float* S,
                            const int32_t* topk_idx, int32_t levels, int32_t* covered,
                            int32_t* kprime, void* stream) {
  const char* fn = "spin_miss_curve";
  SPIN_CHECK(check_config(fn, cfg));
  SPIN_CHECK(check_batch(fn, bt));
  SPIN_CHECK(check_levels(fn, levels));
  SPIN_REQUIRE(S);
  SPIN_REQUIRE(topk_idx);
  SPIN_REQUIRE(covered);
  SPIN_REQUIRE(kprime);
  if (bt->batch == 0) return SPIN_OK;
  return hip_status(spin::launch_miss_curve(*cfg, *bt, S, topk_idx, levels, covered, kprime,
                                            (hipStream_t)stream), fn);
}

spin_status spin_budget_fill(const spin_config* cfg, const spin_batch* bt,
                             const int32_t* level_table, int32_t levels, int32_t* budget,
                             void* stream) {
  const char* fn = "spin_budget_fill";
  SPIN_CHECK(check_config(fn, cfg));
  SPIN_CHECK(check_batch(fn, bt));
  SPIN_CHECK(check_levels(fn, levels));
  SPIN_REQUIRE(level_table);
  SPIN_REQUIRE(budget);
  if (bt->batch == 0) return SPIN_OK;
  return hip_status(spin::launch_budget_fill(*cfg, *bt, level_table, levels, budget,
                                             (hipStream_t)stream), fn);
}

spin_status spin_budget_allocate(int32_t policy, int32_t n_layers, int32_t levels,
                                 int32_t target_level, const int64_t* covered,
                                 const int64_t* total, const double* running_miss,
                                 int32_t* level_out) {
  const char* fn = "spin_budget_allocate";
  SPIN_CHECK(check_levels(fn, levels));
  if (n_layers < 1 || n_layers > SPIN_MAX_LAYERS)
    return fail(SPIN_E_SHAPE, "%s: n_layers %d outside [1, %d]", fn, n_layers, SPIN_MAX_LAYERS);
  if (target_level < 0 || target_level > levels)
    return fail(SPIN_E_SHAPE, "%s: target_level %d outside [0, %d]", fn, target_level, levels);
  SPIN_REQUIRE(level_out);
  if (policy == SPIN_BUDGET_MINIMAX) {
    SPIN_REQUIRE(covered);
    SPIN_REQUIRE(total);
    for (int l = 0; l < n_layers; ++l) {
      if (total[l] < 0) return fail(SPIN_E_SHAPE, "%s: total[%d] < 0", fn, l);
      for (int g = 0; g <= levels; ++g) {
        const int64_t c = covered[(int64_t)l * (levels + 1) + g];
        if (c < 0 || c > total[l])
          return fail(SPIN_E_SHAPE, "%s: covered[%d][%d] outside [0, total]", fn, l, g);
      }
    }
    spin::allocate_minimax(n_layers, levels, target_level, covered, total, level_out);
    return SPIN_OK;
  }
  if (policy == SPIN_BUDGET_PROPORTIONAL) {
    SPIN_REQUIRE(running_miss);
    for (int l = 0; l < n_layers; ++l)
      if (!(running_miss[l] >= 0.0 && running_miss[l] <= 1.0))
        return fail(SPIN_E_SHAPE, "%s: running_miss[%d] outside [0, 1]", fn, l);
    spin::allocate_proportional(n_layers, levels, target_level, running_miss, level_out);
    return SPIN_OK;
  }
  return fail(SPIN_E_SHAPE, "%s: unknown policy %d", fn, policy);
}

spin_status spin_step(const spin_config* cfg, const spin_batch* bt, const spin_step_io* io,
                      int32_t defer_ema, void* stream) {
  SPIN_CHECK(check_step("spin_step", cfg, bt, io));
  if (bt->batch == 0) return SPIN_OK;
  SPIN_CHECK(issue_plan(*cfg, *bt, *io, (hipStream_t)stream));
  return issue_finish(*cfg, *bt, *io, defer_ema, (hipStream_t)stream);
}

}  // extern "C"

// Device scratch of spin_step_noalloc: the workspace of a whole step for
// callers that cannot allocate device memory.  One copy per GPU, held until
// the process ends; host code uses only the address hipGetSymbolAddress
// returns for the current device, never this name.
static __device__ __align__(256) unsigned char scratch[SPIN_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices] = {};
hipError_t g_scratch_err[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device (with
// that device current) on the first call made on it.
spin_status scratch_of_current_device(const char* fn, void** out) {
  int dev = -1;
  SPIN_CHECK(hip_status(hipGetDevice(&dev), fn));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SPIN_E_UNSUPPORTED, "%s: device %d beyond the %d this build tracks", fn, dev,
                kMaxDevices);
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess) return hip_status(g_scratch_err[dev], fn);
  if (!g_scratch_ptr[dev]) return fail(SPIN_E_HIP, "%s: no scratch address on device %d", fn, dev);
  *out = g_scratch_ptr[dev];
  return SPIN_OK;
}

}  // namespace

extern "C" {

spin_status spin_step_noalloc(const spin_config* cfg, const spin_batch* bt,
                              const spin_step_io* io, int32_t defer_ema, void* stream) {
  const char* fn = "spin_step_noalloc";
  SPIN_CHECK(check_config(fn, cfg));
  SPIN_CHECK(check_batch(fn, bt));
  SPIN_REQUIRE(io);
  const size_t need = spin::step_workspace_bytes(*cfg, bt->batch, bt->n_rows, bt->max_blocks);
  if (need > (size_t)SPIN_NOALLOC_WORKSPACE_BYTES)
    return fail(SPIN_E_WORKSPACE,
                "%s: this shape needs %zu bytes of workspace, above the %zu bytes of the "
                "library's static scratch (use spin_step with a caller workspace)",
                fn, need, (size_t)SPIN_NOALLOC_WORKSPACE_BYTES);
  void* ws = nullptr;
  SPIN_CHECK(scratch_of_current_device(fn, &ws));
  spin_step_io own = *io;
  own.workspace = ws;
  own.workspace_bytes = SPIN_NOALLOC_WORKSPACE_BYTES;
  SPIN_CHECK(check_step(fn, cfg, bt, &own));
  if (bt->batch == 0) return SPIN_OK;
  SPIN_CHECK(issue_plan(*cfg, *bt, own, (hipStream_t)stream));
  return issue_finish(*cfg, *bt, own, defer_ema, (hipStream_t)stream);
}

spin_status spin_step_plan(const spin_config* cfg, const spin_batch* bt, const spin_step_io* io,
                           void* stream) {
  SPIN_CHECK(check_step("spin_step_plan", cfg, bt, io));
  if (bt->batch == 0) return SPIN_OK;
  return issue_plan(*cfg, *bt, *io, (hipStream_t)stream);
}

spin_status spin_step_finish(const spin_config* cfg, const spin_batch* bt,
                             const spin_step_io* io, int32_t defer_ema, void* stream) {
  SPIN_CHECK(check_step("spin_step_finish", cfg, bt, io));
  if (bt->batch == 0) return SPIN_OK;
  return issue_finish(*cfg, *bt, *io, defer_ema, (hipStream_t)stream);
}

spin_status spin_stack_create(int32_t n_layers, spin_stack** out) {
  const char* fn = "spin_stack_create";
  if (!out) return fail(SPIN_E_NULL, "%s: out is NULL", fn);
  *out = nullptr;
  if (n_layers < 1 || n_layers > SPIN_MAX_LAYERS)
    return fail(SPIN_E_SHAPE, "%s: n_layers %d outside [1, %d]", fn, n_layers, SPIN_MAX_LAYERS);
  std::unique_ptr<spin_stack> st(new spin_stack);
  st->n_layers = n_layers;
  SPIN_CHECK(hip_status(hipGetDevice(&st->device), fn));
  hipEvent_t* evs[7] = {&st->plan_done[0], &st->plan_done[1], &st->finish_done[0],
                        &st->finish_done[1], &st->ema_done[0], &st->ema_done[1],
                        &st->entry};
  for (hipEvent_t* e : evs) {
    const hipError_t r = hipEventCreateWithFlags(e, hipEventDisableTiming);
    if (r != hipSuccess) {
      spin_stack_destroy(st.release());
      return hip_status(r, fn);
    }
  }
  *out = st.release();
  return SPIN_OK;
}

void spin_stack_destroy(spin_stack* stack) {
  if (!stack) return;
  for (hipEvent_t e : {stack->plan_done[0], stack->plan_done[1], stack->finish_done[0],
                       stack->finish_done[1], stack->ema_done[0], stack->ema_done[1],
                       stack->entry})
    if (e) (void)hipEventDestroy(e);
  delete stack;
}

static spin_status stack_step_impl(spin_stack* stack, int32_t n_layers, const spin_config* cfgs,
                                   const spin_batch* bts, const spin_step_io* ios,
                                   int32_t order_after_main, int32_t defer_ema,
                                   void* main_stream, void* side_stream, void* ema_stream);

spin_status spin_stack_step(spin_stack* stack, int32_t n_layers, const spin_config* cfgs,
                            const spin_batch* bts, const spin_step_io* ios,
                            int32_t order_after_main, int32_t defer_ema, void* main_stream,
                            void* side_stream, void* ema_stream) {
  const char* fn = "spin_stack_step";
  if (!stack || !cfgs || !bts || !ios) return fail(SPIN_E_NULL, "%s: NULL argument", fn);
  if (!stack->has_policy)
    return stack_step_impl(stack, n_layers, cfgs, bts, ios, order_after_main, defer_ema,
                           main_stream, side_stream, ema_stream);
  const spin_budget_policy& P = stack->policy;
  if (n_layers != stack->n_layers)
    return fail(SPIN_E_SHAPE, "%s: with a budget policy every layer (%d) takes part", fn,
                stack->n_layers);
  if (defer_ema)
    return fail(SPIN_E_SHAPE, "%s: deferred EMA updates are not available with a budget policy",
                fn);
  for (int l = 1; l < n_layers; ++l)
    if (bts[l].batch != bts[0].batch || bts[l].n_rows != bts[0].n_rows)
      return fail(SPIN_E_SHAPE, "%s: a budget policy needs the same batch and rows in every "
                  "layer", fn);
  const int R = bts[0].batch, rows = bts[0].n_rows, W = P.levels + 1;
  const bool probe = stack->budget_t > 0 && stack->budget_t % P.probe_period == 0;
  std::vector<spin_step_io> own(ios, ios + n_layers);
  for (int l = 0; l < n_layers; ++l)
    own[l].budget = probe ? P.probe_budget : P.budget + (int64_t)l * R;
  // the miss curves read the probe's own block scores: its EMA must not
  // replace them with the next step's (SPIN_PREDICT_AHEAD), so the probe runs
  // without the flag (its layers' next step then predicts as usual)
  std::vector<spin_config> pc(cfgs, cfgs + n_layers);
  if (probe)
    for (auto& c : pc) c.flags &= ~SPIN_PREDICT_AHEAD;
  cfgs = pc.data();
  SPIN_CHECK(stack_step_impl(stack, n_layers, cfgs, bts, own.data(),
                             order_after_main || stack->order_side, 0, main_stream, side_stream,
                             ema_stream));
  stack->order_side = false;
  ++stack->budget_t;
  if (!probe || R == 0) return SPIN_OK;
  // the probe's curves, the allocation and the new budgets, on main after
  // every layer's finish (the next call's plans are ordered after them)
  hipStream_t mst = (hipStream_t)main_stream;
  for (int l = 0; l < n_layers; ++l)
    SPIN_CHECK(hip_status(spin::launch_miss_curve(cfgs[l], bts[l], own[l].S, own[l].topk_idx,
                                                  P.levels,
                                                  P.covered + (int64_t)l * R * rows * W,
                                                  P.kprime + (int64_t)l * R * rows, mst),
                          "spin_stack_step/miss curve"));
  SPIN_CHECK(spin_budget_update(P.policy, n_layers, P.levels, P.target_level, P.drift_bp,
                                R * rows, P.covered, P.kprime, P.state, P.level_table, mst));
  for (int l = 0; l < n_layers; ++l)
    SPIN_CHECK(hip_status(spin::launch_budget_fill(cfgs[l], bts[l], P.level_table + l, P.levels,
                                                   P.budget + (int64_t)l * R, mst),
                          "spin_stack_step/budget fill"));
  stack->order_side = true;
  return SPIN_OK;
}

spin_status spin_budget_update(int32_t policy, int32_t n_layers, int32_t levels,
                               int32_t target_level, int32_t drift_bp, int32_t rows_total,
                               const int32_t* covered, const int32_t* kprime, void* state,
                               int32_t* level_table, void* stream) {
  const char* fn = "spin_budget_update";
  SPIN_CHECK(check_levels(fn, levels));
  if (policy != SPIN_BUDGET_MINIMAX && policy != SPIN_BUDGET_PROPORTIONAL)
    return fail(SPIN_E_SHAPE, "%s: unknown policy %d", fn, policy);
  if (n_layers < 1 || n_layers > SPIN_MAX_LAYERS)
    return fail(SPIN_E_SHAPE, "%s: n_layers %d outside [1, %d]", fn, n_layers, SPIN_MAX_LAYERS);
  if (target_level < 0 || target_level > levels)
    return fail(SPIN_E_SHAPE, "%s: target_level %d outside [0, %d]", fn, target_level, levels);
  if (drift_bp < 0 || drift_bp > 10000)
    return fail(SPIN_E_SHAPE, "%s: drift_bp %d outside [0, 10000]", fn, drift_bp);
  if (rows_total < 0 || rows_total > SPIN_MAX_BATCH * SPIN_MAX_ROWS)
    return fail(SPIN_E_SHAPE, "%s: rows_total %d", fn, rows_total);
  SPIN_REQUIRE(covered);
  SPIN_REQUIRE(kprime);
  SPIN_REQUIRE(state);
  SPIN_REQUIRE(level_table);
  return hip_status(spin::launch_budget_update(policy, n_layers, levels, target_level, drift_bp,
                                               rows_total, covered, kprime, state, level_table,
                                               (hipStream_t)stream), fn);
}

size_t spin_budget_state_bytes(int32_t n_layers, int32_t levels) {
  if (n_layers < 1 || levels < 1) return 0;
  return spin::budget_state_bytes(n_layers, levels);
}

spin_status spin_stack_set_budget_policy(spin_stack* stack, const spin_budget_policy* policy) {
  const char* fn = "spin_stack_set_budget_policy";
  if (!stack) return fail(SPIN_E_NULL, "%s: stack is NULL", fn);
  if (!policy) {
    stack->has_policy = false;
    return SPIN_OK;
  }
  const spin_budget_policy& P = *policy;
  if (P.policy != SPIN_BUDGET_MINIMAX && P.policy != SPIN_BUDGET_PROPORTIONAL)
    return fail(SPIN_E_SHAPE, "%s: unknown policy %d", fn, P.policy);
  SPIN_CHECK(check_levels(fn, P.levels));
  if (P.probe_period < 1) return fail(SPIN_E_SHAPE, "%s: probe_period < 1", fn);
  if (P.target_level < 0 || P.target_level > P.levels)
    return fail(SPIN_E_SHAPE, "%s: target_level outside [0, levels]", fn);
  if (P.drift_bp < 0 || P.drift_bp > 10000)
    return fail(SPIN_E_SHAPE, "%s: drift_bp outside [0, 10000]", fn);
  if (!P.level_table || !P.budget || !P.probe_budget || !P.covered || !P.kprime || !P.state)
    return fail(SPIN_E_NULL, "%s: a policy buffer is NULL", fn);
  stack->policy = P;
  stack->has_policy = true;
  stack->budget_t = 0;
  return SPIN_OK;
}

spin_status spin_stack_reset_budgets(spin_stack* stack, int32_t n_layers, const spin_config* cfgs,
                                     const spin_batch* bts, void* main_stream) {
  const char* fn = "spin_stack_reset_budgets";
  if (!stack || !cfgs || !bts) return fail(SPIN_E_NULL, "%s: NULL argument", fn);
  if (!stack->has_policy) return fail(SPIN_E_SHAPE, "%s: no budget policy set", fn);
  if (n_layers != stack->n_layers)
    return fail(SPIN_E_SHAPE, "%s: n_layers %d, the stack has %d", fn, n_layers, stack->n_layers);
  for (int l = 0; l < n_layers; ++l) {
    SPIN_CHECK(check_config(fn, &cfgs[l]));
    SPIN_CHECK(check_batch(fn, &bts[l]));
  }
  const spin_budget_policy& P = stack->policy;
  hipStream_t mst = (hipStream_t)main_stream;
  const int R = bts[0].batch;
  SPIN_CHECK(hip_status(spin::launch_budget_reset(n_layers, P.levels, P.target_level, R, P.state,
                                                  P.level_table, P.probe_budget, mst), fn));
  for (int l = 0; l < n_layers; ++l)
    if (bts[l].batch > 0)
      SPIN_CHECK(hip_status(spin::launch_budget_fill(cfgs[l], bts[l], P.level_table + l,
                                                     P.levels, P.budget + (int64_t)l * R, mst),
                            fn));
  stack->budget_t = 0;
  stack->order_side = true;
  return SPIN_OK;
}

static spin_status stack_step_impl(spin_stack* stack, int32_t n_layers, const spin_config* cfgs,
                                   const spin_batch* bts, const spin_step_io* ios,
                                   int32_t order_after_main, int32_t defer_ema,
                                   void* main_stream, void* side_stream, void* ema_stream) {
  const char* fn = "spin_stack_step";
  if (!stack || !cfgs || !bts || !ios) return fail(SPIN_E_NULL, "%s: NULL argument", fn);
  if (n_layers < 1 || n_layers > stack->n_layers)
    return fail(SPIN_E_SHAPE, "%s: n_layers %d outside [1, %d]", fn, n_layers, stack->n_layers);
  if (!side_stream && ema_stream)
    return fail(SPIN_E_SHAPE, "%s: an EMA stream needs a side stream", fn);
  if (defer_ema && ema_stream)
    return fail(SPIN_E_SHAPE, "%s: a deferred EMA update runs in spin_stack_commit, not on an "
                "EMA stream", fn);
  if (stack->commit_pending)
    return fail(SPIN_E_SHAPE, "%s: the previous step deferred its EMA updates; call "
                "spin_stack_commit first", fn);
  if (side_stream && (main_stream == side_stream ||
                      (ema_stream && (ema_stream == main_stream || ema_stream == side_stream))))
    return fail(SPIN_E_SHAPE, "%s: main, side and ema must be different streams", fn);
  int dev = -1;
  SPIN_CHECK(hip_status(hipGetDevice(&dev), fn));
  if (dev != stack->device)
    return fail(SPIN_E_SHAPE, "%s: stack created on device %d, current device %d", fn,
                stack->device, dev);
  for (int l = 0; l < n_layers; ++l) {
    char lfn[64];
    std::snprintf(lfn, sizeof(lfn), "%s[layer %d]", fn, l);
    SPIN_CHECK(check_step(lfn, &cfgs[l], &bts[l], &ios[l]));
  }
  hipStream_t mst = (hipStream_t)main_stream, sst = (hipStream_t)side_stream;
  if (!sst) {
    // the previous call's EMA updates may still run on its EMA stream: main
    // waits for them before any plan reads the EMA state
    if (stack->ema_stream_last) {
      SPIN_CHECK(hip_status(hipStreamWaitEvent(mst, stack->ema_done[0], 0), fn));
      SPIN_CHECK(hip_status(hipStreamWaitEvent(mst, stack->ema_done[1], 0), fn));
    }
    // one stream: layer l + 1's plan inside layer l's score and top-K + EMA
    // launches where both allow it (layer l's score kernel filters, layer
    // l + 1 has one verifier row), else on its own before its finish
    bool planned = false;  // this layer's plan was issued inside the previous launches
    for (int l = 0; l < n_layers; ++l) {
      if (bts[l].batch <= 0) {
        planned = false;
        continue;
      }
      if (!planned) SPIN_CHECK(issue_plan(cfgs[l], bts[l], ios[l], mst));
      const int m = l + 1;
      // (the fused launches run the method's block reduction, A1)
      const bool fuse = m < n_layers && bts[m].batch > 0 && bts[m].n_rows == 1 &&
                        spin::score_filters(cfgs[l], bts[l]) &&
                        (cfgs[l].flags & SPIN_REDUCE_MASK) == 0 &&
                        (cfgs[m].flags & SPIN_REDUCE_MASK) == 0;
      if (fuse)
        SPIN_CHECK(issue_finish_with_plan(cfgs[l], bts[l], ios[l], cfgs[m], bts[m], ios[m],
                                          defer_ema, mst));
      else
        SPIN_CHECK(issue_finish(cfgs[l], bts[l], ios[l], defer_ema, mst));
      planned = fuse;
    }
    stack->one_stream_last = true;
    stack->ema_stream_last = false;
    stack->commit_pending = defer_ema != 0;
    stack->committed_layers = n_layers;
    return SPIN_OK;
  }
  auto wait = [&](hipStream_t st, hipEvent_t e) {
    return hip_status(hipStreamWaitEvent(st, e, 0), fn);
  };
  auto record = [&](hipEvent_t e, hipStream_t st) { return hip_status(hipEventRecord(e, st), fn); };
  // after a one-stream call the stack's events describe an older call: the
  // side stream then starts after everything issued on main
  if (order_after_main || stack->one_stream_last) {  // or plan inputs the caller wrote on main
    SPIN_CHECK(record(stack->entry, mst));
    SPIN_CHECK(wait(sst, stack->entry));
  }
  const int h = (n_layers + 1) / 2;
  const int lo[2] = {0, h}, hi[2] = {h, n_layers};
  hipStream_t est = (hipStream_t)ema_stream;
  // side: every plan(l) after the previous call's update of layer l (its
  // finish, or with an EMA stream its EMA).  Group A's were recorded as a
  // group when the split was the same or wider; otherwise the previous
  // call's last record covers every layer.
  hipEvent_t* prev_done = est ? stack->ema_done : stack->finish_done;
  for (int g = 0; g < 2; ++g) {
    if (lo[g] == hi[g]) continue;
    const bool a_covers = g == 0 && h <= stack->prev_h;
    SPIN_CHECK(wait(sst, prev_done[a_covers ? 0 : 1]));
    for (int l = lo[g]; l < hi[g]; ++l)
      if (bts[l].batch > 0) SPIN_CHECK(issue_plan(cfgs[l], bts[l], ios[l], sst));
    SPIN_CHECK(record(stack->plan_done[g], sst));
  }
  // main: each group's finishes after the group's plans; with an EMA stream
  // the finishes are score + top-K and the group's EMA updates + counter
  // advances follow there
  for (int g = 0; g < 2; ++g) {
    if (lo[g] == hi[g]) continue;
    SPIN_CHECK(wait(mst, stack->plan_done[g]));
    for (int l = lo[g]; l < hi[g]; ++l)
      if (bts[l].batch > 0)
        SPIN_CHECK(issue_finish(cfgs[l], bts[l], ios[l], (est || defer_ema) ? 1 : 0, mst));
    SPIN_CHECK(record(stack->finish_done[g], mst));
    if (est) {
      SPIN_CHECK(wait(est, stack->finish_done[g]));
      for (int l = lo[g]; l < hi[g]; ++l)
        if (bts[l].batch > 0) SPIN_CHECK(issue_ema(cfgs[l], bts[l], ios[l], est));
      SPIN_CHECK(record(stack->ema_done[g], est));
    }
  }
  // with a single group, the [1] records (what the next call's group-A plans
  // may wait for when the split widens) must also cover this call
  if (lo[1] == hi[1]) {
    SPIN_CHECK(record(stack->finish_done[1], mst));
    if (est) SPIN_CHECK(record(stack->ema_done[1], est));
  }
  stack->prev_h = h;
  stack->one_stream_last = false;
  stack->ema_stream_last = est != nullptr;
  stack->commit_pending = defer_ema != 0;
  stack->committed_layers = n_layers;
  return SPIN_OK;
}

spin_status spin_stack_commit(spin_stack* stack, int32_t n_layers, const spin_config* cfgs,
                              const spin_batch* bts, const spin_step_io* ios,
                              void* main_stream) {
  const char* fn = "spin_stack_commit";
  if (!stack || !cfgs || !bts || !ios) return fail(SPIN_E_NULL, "%s: NULL argument", fn);
  if (!stack->commit_pending)
    return fail(SPIN_E_SHAPE, "%s: the previous step did not defer its EMA updates", fn);
  if (n_layers != stack->committed_layers)
    return fail(SPIN_E_SHAPE, "%s: n_layers %d, but the deferred step ran %d", fn, n_layers,
                stack->committed_layers);
  int dev = -1;
  SPIN_CHECK(hip_status(hipGetDevice(&dev), fn));
  if (dev != stack->device)
    return fail(SPIN_E_SHAPE, "%s: stack created on device %d, current device %d", fn,
                stack->device, dev);
  for (int l = 0; l < n_layers; ++l) {
    char lfn[64];
    std::snprintf(lfn, sizeof(lfn), "%s[layer %d]", fn, l);
    SPIN_CHECK(check_step(lfn, &cfgs[l], &bts[l], &ios[l]));
  }
  hipStream_t mst = (hipStream_t)main_stream;
  // in layer order, each layer's replay of its prefix-valid rows (io.n_valid)
  // and counter advance, q positions from the step's snapshot
  for (int l = 0; l < n_layers; ++l)
    if (bts[l].batch > 0) SPIN_CHECK(issue_ema(cfgs[l], bts[l], ios[l], mst));
  // the next two-stream call's plans wait for these updates
  if (!stack->one_stream_last) {
    SPIN_CHECK(hip_status(hipEventRecord(stack->finish_done[0], mst), fn));
    SPIN_CHECK(hip_status(hipEventRecord(stack->finish_done[1], mst), fn));
  }
  stack->commit_pending = false;
  return SPIN_OK;
}

}  // extern "C"
