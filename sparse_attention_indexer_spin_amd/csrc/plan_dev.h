// Device code of a step's plan (block prediction and selection), shared by
// the plan kernels and the kernels that run a layer's plan beside another
// layer's scoring or top-K + EMA.
//
// Paper: "SPIN: Shadow Predictive Indexer for Sparse Attention", Sec. 3.2
// (Eq. 1, Eq. 2, Algorithm 1 steps 1-5 and the prose after it), Sec. 3.2.1
// (exploration inside the budget).
#pragma once
#include "spin_dev.h"

namespace spin {

// ---------------------------------------------------------------------------
// Stage 1: S[r][row][j] = max_{i in block j, i < N} C(V[i], D[q_row - i]).
// One wave per 8 consecutive blocks, lane = slot within the block; all 16
// loads of a lane are issued before the first reduction so each wave keeps
// 4 KB in flight.  V rows are read ascending, D rows descending (both as
// coalesced 256-B wave accesses).
// ---------------------------------------------------------------------------
// Exploration key of block j: the complement of Philox4x32-10 word 0 of
// counter (j, t, layer, req_id) under key (seed lo, seed hi), so that the
// smallest priority is the largest key (Sec. 3.2.1).
__device__ __forceinline__ uint32_t explore_key(int j, int t, int layer, int req_id,
                                                uint32_t seed_lo, uint32_t seed_hi) {
  return ~philox_word0((uint32_t)j, (uint32_t)t, (uint32_t)layer, (uint32_t)req_id, seed_lo,
                       seed_hi);
}

constexpr int kPredBlocksPerWave = 8;

// Pool block j's predicted slot scores, one per lane (`valid`: the slot lies
// in the context, n_valid of them), per spin_config.flags: the max (Eq. 2),
// the mean of the up to four largest (largest first), or the mean over the
// valid slots with the 64 values (0 past the context) summed as a balanced
// pairwise tree -- the xor butterfly below adds lane pairs, then pairs of
// pairs, in exactly that order, and fp32 addition is commutative.
__device__ __forceinline__ float pool_block_wave(float zhat, bool valid, int n_valid,
                                                 int pooling) {
  if (pooling == SPIN_POOL_MEAN) {
    float v = valid ? zhat : 0.0f;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v = v + __shfl_xor(v, m);
    return v / (float)n_valid;
  }
  float v = valid ? zhat : -INFINITY;
  if (pooling != SPIN_POOL_TOP4) return wave_max_f32(v);
  const int cnt = min(4, n_valid);
  float s = 0.0f;
  for (int it = 0; it < cnt; ++it) {
    const float m = wave_max_f32(v);
    s = it == 0 ? m : s + m;
    const uint64_t at = __ballot(v == m);  // one lane holding the max leaves the set
    if ((int)(threadIdx.x & 63) == __builtin_ctzll(at)) v = -INFINITY;
  }
  return s / (float)cnt;
}

// Prediction of NB blocks j0 .. j0 + NB - 1 (j0 < B) of one (request, row)
// by one wave, lane = slot: predict_load issues the loads, predict_reduce
// pools and stores the block scores.
template <int NB>
__device__ __forceinline__ void predict_load(int N, int B, int q, int j0,
                                             const float* __restrict__ Vr,
                                             const float* __restrict__ Dr,
                                             const float* __restrict__ vmax_r, float (&vv)[NB],
                                             float (&dd)[NB], float& vm) {
  static_assert(NB <= 64, "one V max per lane");
  const int lane = threadIdx.x & 63;
  // with the V block maxima (max combine), every block but the last reads
  // its V max (lane b holds block j0 + b's) instead of its 64 V values
  vm = vmax_r && lane < NB && j0 + lane < B - 1 ? vmax_r[j0 + lane] : -INFINITY;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int i = (j0 + b) * SPIN_BLOCK + lane;
    const bool ok = i < N;
    const bool cached = vmax_r && j0 + b < B - 1;
    vv[b] = ok && !cached ? Vr[i] : -INFINITY;
    dd[b] = ok ? Dr[q - i] : 0.0f;
  }
}

template <int NB>
__device__ __forceinline__ void predict_reduce(int combine, int pooling, int N, int B, int j0,
                                               const float (&vv)[NB], const float (&dd)[NB],
                                               float vm, float* __restrict__ Srow) {
  const int lane = threadIdx.x & 63;
  if (pooling == SPIN_POOL_MAX && (NB & (NB - 1)) == 0) {
    // all NB block maxima at once (wave_max_scatter), lane l holding block
    // j0 + (l >> (6 - log2 NB)); its V max comes from the lane that loaded it
    constexpr int LG = NB == 1 ? 0 : NB == 2 ? 1 : NB == 4 ? 2 : NB == 8 ? 3 : NB == 16 ? 4 : 5;
    float x[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int i = (j0 + b) * SPIN_BLOCK + lane;
      const float zhat =
          combine == SPIN_COMBINE_SUM ? __fadd_rn(vv[b], dd[b]) : fmaxf(vv[b], dd[b]);
      x[b] = i < N ? zhat : -INFINITY;
    }
    const int b = lane >> (6 - LG), j = j0 + b;
    const float m = fmaxf(wave_max_scatter<NB>(x), __shfl(vm, b, 64));
    if ((lane & ((1 << (6 - LG)) - 1)) == 0 && j < B) Srow[j] = m + 0.0f;
    return;
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int j = j0 + b;
    const int i = j * SPIN_BLOCK + lane;
    const float zhat =
        combine == SPIN_COMBINE_SUM ? __fadd_rn(vv[b], dd[b]) : fmaxf(vv[b], dd[b]);
    const float m =
        pooling == SPIN_POOL_MAX
            ? fmaxf(wave_max_f32(i < N ? zhat : -INFINITY),
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vm), b)))
            : pool_block_wave(zhat, i < N, min(SPIN_BLOCK, N - j * SPIN_BLOCK), pooling);
    if (lane == 0 && j < B) Srow[j] = m + 0.0f;
  }
}

// One wave's NB blocks j0 .. j0 + NB - 1 (j0 < B) of one (request, row),
// every load in flight before the reductions.
template <int NB = kPredBlocksPerWave>
__device__ __forceinline__ void predict_wave(int combine, int pooling, int N, int B, int q,
                                             int j0, const float* __restrict__ Vr,
                                             const float* __restrict__ Dr,
                                             const float* __restrict__ vmax_r,
                                             float* __restrict__ Srow) {
  float vv[NB], dd[NB], vm;
  predict_load<NB>(N, B, q, j0, Vr, Dr, vmax_r, vv, dd, vm);
  predict_reduce<NB>(combine, pooling, N, B, j0, vv, dd, vm, Srow);
}

// ---------------------------------------------------------------------------
// Stage 2: one workgroup per (request, verifier row); kSelectThreads threads,
// EPT blocks per thread.  The selection is a chain of block-wide radix steps
// whose wave scans run on DPP moves, so wide workgroups (few keys per thread
// per histogram pass) beat narrow ones despite their larger barriers.
// ---------------------------------------------------------------------------
constexpr int kSelectThreads = 1024;

enum { kExploreRandom = 0, kExploreAge = 1, kExploreStaleness = 2 };

struct SelectArgs {
  int K, sparsity_bp, explore_bp, layer, per_row;  // per_row: SPIN_EXPLORE_PER_ROW
  uint32_t seed_lo, seed_hi;
  int rows, max_blocks;
  uint8_t* code;   // [R][rows][max_blocks]
  int32_t* sel;    // [R][max_blocks]
  int32_t* n_sel;  // [R]
  int policy;          // kExplore*
  int32_t* last_obs;   // optional [R][max_blocks]: step of each block's last observation
  int32_t* inv;        // optional [R][max_blocks]: each block's position in sel, -1 if none
};

// Exploration key of block j (larger = taken first; ties: lower block) under
// the row's policy (Sec. 3.2.1; Sec. 4.6, "Staleness mitigation").
__device__ __forceinline__ uint32_t policy_key(const SelectArgs& a, int j, int t, int row,
                                               int rid, float s, int obs) {
  if (a.policy == kExploreAge) return ~(uint32_t)obs;  // smallest last_obs first
  if (a.policy == kExploreStaleness) return float_key(s * (float)(t - obs));
  return explore_key(j, t, a.layer + (a.per_row ? 65536 * row : 0), rid, a.seed_lo, a.seed_hi);
}

// Record step t for the chosen blocks of this thread (the union of a step).
template <int EPT>
__device__ __forceinline__ void record_observed(int32_t* last_obs_r, int j0, int B,
                                                uint32_t chosen, int t) {
  if (!last_obs_r) return;
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if ((chosen >> e & 1u) && j0 + e < B) last_obs_r[j0 + e] = t;
}

struct SelectLds {
  int hist[kRadixHist];
  int sh[32];
  uint32_t tmpu[32];
};

// The row's budget m (Algorithm 1 step 4; the forced blocks count toward it,
// Sec. 3.2.1 caps the exploration share by what is left).
struct RowBudget {
  int n_f, n_e, n_r;
};
__device__ __forceinline__ RowBudget row_budget(const SelectArgs& a, int B, int bud) {
  const int kb = (a.K + SPIN_BLOCK - 1) / SPIN_BLOCK;
  const int keep = (int)(((int64_t)(10000 - a.sparsity_bp) * B + 9999) / 10000);
  int m = bud > 0 ? min(B, bud) : min(B, max(kb, keep));
  const int n_f = B > 1 ? 2 : 1;
  m = max(m, n_f);
  const int n_e = min((int)((int64_t)m * a.explore_bp / 10000), m - n_f);
  return RowBudget{n_f, n_e, m - n_f - n_e};
}

// Block budget, forced / ranked / explored blocks and (compact) the block
// list of request r, row `row`: B blocks (0 when the request is invalid), t
// steps since reset, rid the request id, bud a budget override (<= 0: none).
// Every thread of the workgroup calls it.
template <int EPT>
__device__ __forceinline__ void select_row(const SelectArgs& a, int r, int row, int B, int t,
                                           int rid, int bud, const float* __restrict__ Srow,
                                           bool compact, SelectLds& L) {
  const int j0 = threadIdx.x * EPT;
  uint8_t* crow = a.code + ((int64_t)r * a.rows + row) * a.max_blocks;
  uint32_t chosen = 0u;
  uint8_t c[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) c[e] = SPIN_CODE_SKIP;

  if (B > 0 && t == 0) {
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (j0 + e < B) { c[e] = SPIN_CODE_DENSE; chosen |= 1u << e; }
  } else if (B > 0) {
    const RowBudget rb = row_budget(a, B, bud);
    const int n_e = rb.n_e, n_r = rb.n_r;
    float sv[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) sv[e] = j0 + e < B ? Srow[j0 + e] : 0.0f;
    uint32_t key[EPT];
    uint32_t elig = 0u;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int j = j0 + e;
      key[e] = 0u;
      if (j < B) {
        if (j == 0 || j == B - 1) { c[e] = SPIN_CODE_FORCED; chosen |= 1u << e; }
        else { key[e] = float_key(sv[e]); elig |= 1u << e; }
      }
    }
    const uint32_t ranked =
        block_select_top<EPT, kSelectThreads>(key, elig, n_r, L.hist, L.sh, L.tmpu);
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (ranked >> e & 1u) c[e] = SPIN_CODE_RANKED;
    chosen |= ranked;
    elig &= ~ranked;
    if (n_e > 0) {
      // exploration keys in registers; random priorities are shared by the
      // rows (the counter carries no row) unless each row draws its own
      const int32_t* orow = a.last_obs ? a.last_obs + (int64_t)r * a.max_blocks : nullptr;
      uint32_t pk[EPT];
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int obs = a.policy != kExploreRandom && orow && j0 + e < B ? orow[j0 + e] : 0;
        pk[e] = policy_key(a, j0 + e, t, row, rid, sv[e], obs);
      }
      const uint32_t expl =
          block_select_top<EPT, kSelectThreads>(pk, elig, n_e, L.hist, L.sh, L.tmpu);
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        if (expl >> e & 1u) c[e] = SPIN_CODE_EXPLORED;
      chosen |= expl;
    }
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if (j0 + e < B) crow[j0 + e] = c[e];
  if (compact) {
    compact_blocks<EPT, kSelectThreads>(chosen, a.max_blocks, a.sel + (int64_t)r * a.max_blocks,
                                        a.n_sel + r, L.sh,
                                        a.inv ? a.inv + (int64_t)r * a.max_blocks : nullptr);
    // the union is this row's mask: its blocks are observed at step t
    record_observed<EPT>(a.last_obs ? a.last_obs + (int64_t)r * a.max_blocks : nullptr, j0, B,
                         chosen, t);
  }
}

// ---------------------------------------------------------------------------
// A layer's plan run by workgroups of another kernel (a layer's score or
// top-K + EMA launch), one verifier row.
// ---------------------------------------------------------------------------
// Prediction: workgroup w of n covers request w / per_req, blocks
// [64 (w % per_req), + 64): 16 per wave.  These workgroups run as the scoring
// workgroups leave their CUs, two per CU (the kernel's registers), so the
// tail is bound by how fast a workgroup turns its loads into block scores:
// with one wave reduction per block most of it went into the reductions
// (workgroup timestamps: ~10 us of tail after the last scoring workgroup);
// the reduce-scatter over all of a wave's blocks (wave_max_scatter) took the
// one-stream stack from 93.3 to 89.5 us per layer-step, and 16 blocks per
// wave instead of 8 another ~0.6 us (32: no further gain).
constexpr int kTailPredBlocksPerWave = 16;
constexpr int kPredBlocksPerWg = 4 * kTailPredBlocksPerWave;

struct PredictArgs {
  int combine, pooling, max_blocks, per_req;  // per_req: workgroups per request
  const int32_t* ctx;
  const int32_t* qpos;
  const float* V;
  int64_t v_ld;
  const float* D;
  int64_t d_ld;
  const float* vmax;   // optional V block maxima
  float* S;            // [R][max_blocks]
  int32_t* err;
  int32_t* qpos_snap;  // optional: the step's q positions
  const int32_t* step;  // with tag: the step counters
  const int32_t* tag;   // optional [R][4]: scores already predicted (predicted_ahead)
};

// Request r's block scores for (step[r], q, N) already sit in S: the last
// EMA update predicted them (SPIN_PREDICT_AHEAD) and wrote the tag.
__device__ __forceinline__ bool predicted_ahead(const int32_t* tag, const int32_t* step, int r,
                                                int q, int N) {
  if (!tag || !step) return false;
  const int32_t* t = tag + 4 * (int64_t)r;
  return t[0] >= 0 && t[0] == step[r] && t[1] == q && t[2] == N;
}

__device__ __forceinline__ void predict_wg(const PredictArgs& a, int w) {
  const int r = w / a.per_req, bx = w % a.per_req;
  const int N = a.ctx[r], q0 = a.qpos[r];
  if (a.qpos_snap && bx == 0 && threadIdx.x == 0) a.qpos_snap[r] = q0;
  const int e = request_error(N, q0, 1, a.max_blocks, a.v_ld, a.d_ld);
  if (e) {
    if (bx == 0 && threadIdx.x == 0) raise_error(a.err, e);
    return;
  }
  if (predicted_ahead(a.tag, a.step, r, q0, N)) return;
  const int B = (N + SPIN_BLOCK - 1) / SPIN_BLOCK;
  const int wave = threadIdx.x >> 6;
  const int j0 = (bx * 4 + wave) * kTailPredBlocksPerWave;
  if (j0 >= B) return;
  predict_wave<kTailPredBlocksPerWave>(a.combine, a.pooling, N, B, q0, j0,
                                       a.V + (int64_t)r * a.v_ld, a.D + (int64_t)r * a.d_ld,
                                       a.vmax ? a.vmax + (int64_t)r * a.max_blocks : nullptr,
                                       a.S + (int64_t)r * a.max_blocks);
}

// Selection of request r (one row, compacted): the whole workgroup of
// kSelectThreads threads calls it.
struct SelectInputs {
  const int32_t* ctx;
  const int32_t* qpos;
  const int32_t* step;
  const int32_t* req_id;
  const float* S;
  const int32_t* budget;  // optional
};

template <int EPT>
__device__ __forceinline__ void select_request(const SelectArgs& a, const SelectInputs& in,
                                               int r, SelectLds& L) {
  const int N = in.ctx[r];
  const bool bad = request_error(N, in.qpos[r], 1, a.max_blocks, 0, 0) != 0;
  const int B = bad ? 0 : (N + SPIN_BLOCK - 1) / SPIN_BLOCK;
  select_row<EPT>(a, r, 0, B, in.step[r], in.req_id[r], in.budget ? in.budget[r] : 0,
                  in.S + (int64_t)r * a.max_blocks, true, L);
}

}  // namespace spin
