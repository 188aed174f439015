// Host-side launchers of the SPIN kernels (internal).
#pragma once
#include <hip/hip_runtime.h>

#include "spin.h"
#include "plan_dev.h"
#include "ema_dev.h"

namespace spin {

// Where a score kernel that also filters for the top-K writes its candidates:
// the slots whose z key is >= the row's hint, as (key, slot) pairs in slot
// order.  A worker appends the candidates of its run of consecutive selected
// blocks k0 .. k1 of a row at cand[row * cand_ld + 64 k0 ..] and writes their
// count to pcnt[row * pcnt_ld + k0], and 0 for the run's other blocks: for
// every k, pcnt[k] candidates sit at cand[64 k ..].
struct CandSink {
  const uint32_t* hint;  // [rows_total]
  uint2* cand;
  int32_t* pcnt;
  int64_t cand_ld;
  int pcnt_ld;
};

// vmax (optional, [R][max_blocks]): the V block maxima (max combine only).
// qpos_snap (optional, [R]): predict records the step's q_pos there; the
// fused EMA + advance of a whole step reads it instead of q_pos.  tag
// (optional, [R][4]): requests whose scores the last EMA predicted ahead are
// skipped (their snapshot is still recorded).
hipError_t launch_predict(const spin_config& c, const spin_batch& b, const float* V, int64_t v_ld,
                          const float* D, int64_t d_ld, const float* vmax, float* S,
                          hipStream_t st, int32_t* qpos_snap = nullptr,
                          const int32_t* tag = nullptr);
// A layer's plan (one verifier row) run inside another layer's launches:
// its prediction by the last workgroups of a score launch, its selection by
// the last workgroups of a top-K + EMA launch.
struct PredictPlan {
  PredictArgs args;
  int wgs;
};
struct SelectPlan {
  SelectArgs args;
  SelectInputs in;
  int requests, ept;
};
// tag (optional): skip the requests whose scores were predicted ahead.
PredictPlan predict_plan(const spin_config& c, const spin_batch& b, const float* V, int64_t v_ld,
                         const float* D, int64_t d_ld, const float* vmax, float* S,
                         int32_t* qpos_snap, const int32_t* tag = nullptr);
// last_obs (optional, [R][max_blocks]): the step of each block's last
// observation, read by the age / staleness exploration policies and set to
// the step for every block of the union.
// inv (optional, [R][max_blocks]): each block's position in sel, -1 if not
// selected (what the predict-ahead EMA reads).
SelectPlan select_plan(const spin_config& c, const spin_batch& b, const float* S,
                       const int32_t* budget, uint8_t* code, int32_t* sel, int32_t* n_sel,
                       int32_t* last_obs, int32_t* inv = nullptr);
hipError_t launch_select(const spin_config& c, const spin_batch& b, const float* S,
                         const int32_t* budget, uint8_t* code, int32_t* sel, int32_t* n_sel,
                         int32_t* last_obs, hipStream_t st, int32_t* inv = nullptr);
// Block reduction A2: block scores from block-level states.
hipError_t launch_predict_a2(const spin_config& c, const spin_batch& b, const float* V,
                             int64_t v_ld, const float* D, int64_t d_ld, float* S,
                             hipStream_t st, int32_t* qpos_snap = nullptr);
// Block reduction A0: every slot's predicted score into z (all blocks listed
// in sel), then, from the rows' top-K of it, the masks.
hipError_t launch_predict_slots(const spin_config& c, const spin_batch& b, const float* V,
                                int64_t v_ld, const float* D, int64_t d_ld, float* z,
                                int64_t z_ld, int32_t* sel, int32_t* n_sel, hipStream_t st);
hipError_t launch_a0_select(const spin_config& c, const spin_batch& b, const float* S,
                            const int32_t* topk, uint8_t* code, int32_t* sel, int32_t* n_sel,
                            int32_t* last_obs, hipStream_t st);
// Block reduction A2's EMA update (+ counter advance with qpos_snap, as launch_ema).
hipError_t launch_ema_a2(const spin_config& c, const spin_batch& b, const float* z, int64_t z_ld,
                         const int32_t* sel, const int32_t* n_sel, const int32_t* n_valid,
                         float* V, int64_t v_ld, float* D, int64_t d_ld, hipStream_t st,
                         const int32_t* qpos_snap = nullptr, int32_t* qpos_out = nullptr,
                         int32_t* step_out = nullptr);
// With a non-null `sink`, kernels that can (score_filters()) also write the
// top-K candidates; the caller then runs launch_topk with `prefiltered`.
hipError_t launch_score(const spin_config& c, const spin_batch& b, const void* q, const float* w,
                        const void* kp, const float* ks, const int32_t* pt, int64_t pt_ld,
                        const int32_t* sel, const int32_t* n_sel, float* z, int64_t z_ld,
                        hipStream_t st, const CandSink* sink = nullptr,
                        const PredictPlan* plan = nullptr);
bool score_filters(const spin_config& c, const spin_batch& b);
hipError_t launch_topk(const spin_config& c, const spin_batch& b, const float* z, int64_t z_ld,
                       const int32_t* sel, const int32_t* n_sel, int32_t* out, void* ws,
                       size_t ws_bytes, hipStream_t st, bool prefiltered = false);
// After a filtering score kernel, the top-K and the EMA update + counter
// advance of a whole step in one launch (they share no outputs).  Both read
// q positions from the step's snapshot.  ema == false (deferred update; only
// with `next`): the top-K and the next layer's selection alone.
hipError_t launch_topk_ema(const spin_config& c, const spin_batch& b, const float* z,
                           int64_t z_ld, const int32_t* sel, const int32_t* n_sel, int32_t* out,
                           void* ws, const int32_t* n_valid, float* V, int64_t v_ld, float* D,
                           int64_t d_ld, float* vmax, const int32_t* qpos_snap,
                           int32_t* qpos_out, int32_t* step_out, hipStream_t st,
                           const SelectPlan* next = nullptr, bool ema = true,
                           const Ahead* ahead = nullptr);
// The candidate sink inside a top-K workspace.
CandSink topk_sink(void* ws, int R, int rows, int max_blocks);
size_t topk_workspace_bytes(const spin_config& c, int R, int rows, int max_blocks);
// A whole step's workspace: the top-K region, then the step's q_pos snapshot.
size_t step_workspace_bytes(const spin_config& c, int R, int rows, int max_blocks);
// With qpos_snap, q positions come from the snapshot and the kernel also
// advances qpos_out / step_out (each optional) like launch_advance.  With
// `ahead` (A1), every block's EMA update and the next step's block scores
// (SPIN_PREDICT_AHEAD).
hipError_t launch_ema(const spin_config& c, const spin_batch& b, const float* z, int64_t z_ld,
                      const int32_t* sel, const int32_t* n_sel, const int32_t* n_valid, float* V,
                      int64_t v_ld, float* D, int64_t d_ld, float* vmax, hipStream_t st,
                      const int32_t* qpos_snap = nullptr, int32_t* qpos_out = nullptr,
                      int32_t* step_out = nullptr, const Ahead* ahead = nullptr);
hipError_t launch_advance(int R, int rows, const int32_t* n_valid, int32_t* qpos, int32_t* step,
                          hipStream_t st);
hipError_t launch_reset(int R, float* V, int64_t v_ld, float* D, int64_t d_ld, int64_t vmax_ld,
                        float* vmax, int32_t* step, hipStream_t st);

// Per-layer budgets: the miss curve of a dense probe step, the budget table
// fill, and the host allocation between layers.
hipError_t launch_miss_curve(const spin_config& c, const spin_batch& b, const float* S,
                             const int32_t* topk, int levels, int32_t* covered, int32_t* kprime,
                             hipStream_t st);
hipError_t launch_budget_fill(const spin_config& c, const spin_batch& b, const int32_t* level,
                              int levels, int32_t* budget, hipStream_t st);
// After a probe step: the layers' curves summed, the running miss rates and
// the new levels (published when the curves drifted by more than drift_bp,
// always with drift_bp 0), all on the device (state: budget_state_bytes()).
hipError_t launch_budget_update(int policy, int L, int levels, int target, int drift_bp, int RR,
                                const int32_t* covered, const int32_t* kprime, void* state,
                                int32_t* level_table, hipStream_t st);
hipError_t launch_budget_reset(int L, int levels, int target, int R, void* state,
                               int32_t* level_table, int32_t* probe_budget, hipStream_t st);
size_t budget_state_bytes(int L, int levels);
void allocate_minimax(int L, int levels, int target, const int64_t* covered,
                      const int64_t* total, int32_t* out);
void allocate_proportional(int L, int levels, int target, const double* miss, int32_t* out);

// The HBM read probe of include/spin_probe.h.
hipError_t launch_read_pages(const void* kp, int64_t n_pages, const int32_t* ids, int n,
                             uint32_t* sink, hipStream_t st);

// Number of workgroups of `threads` threads of `kernel` resident at once on
// the current device (occupancy x compute units), cached per kernel.
int resident_workgroups(const void* kernel, int threads, size_t dyn_lds = 0);
// Whether `kernel` may be launched with dyn_lds bytes of dynamic LDS on the
// current device.
bool lds_fits(const void* kernel, size_t dyn_lds);

}  // namespace spin
