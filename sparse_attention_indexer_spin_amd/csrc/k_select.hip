// Stages 1-2 of the SPIN decode step: predicted block scores, block budget,
// ranked + Philox-explored block selection, verifier-row union; plus the
// per-request counter advance and the state reset.
//
// Paper: "SPIN: Shadow Predictive Indexer for Sparse Attention", Sec. 3.2
// (Eq. 1 predicted slot score, Eq. 2 block max pooling, Algorithm 1 steps
// 1-5 and the reset / dense first step / always-kept sink and newest block
// described after it), Sec. 3.2.1 (exploration inside the budget) and
// Sec. 3.2.2 (union of the verifier rows' masks).
#include "plan_dev.h"
#include "spin_launch.h"

namespace spin {

// Several verifier rows: one wave computes every row of its 8 blocks from
// one load of V and D.  Row r needs D[q0 + r - i] = the value row 0 loads
// for slot i - r, so lane l takes it from lane l - r of the same block's
// vector, or of the previous block's for l < r (the wave's first block
// loads the few previous offsets it needs, q0 + 1 .. q0 + rows - 1 at most).
template <int ROWS>
__device__ __forceinline__ void predict_wave_rows(int combine, int pooling, int N, int B, int q0,
                                                  int j0,
                                                  const float* __restrict__ Vr,
                                                  const float* __restrict__ Dr,
                                                  const float* __restrict__ vmax_r,
                                                  float* __restrict__ S0, int max_blocks) {
  const int lane = threadIdx.x & 63;
  const float vm = vmax_r && lane < kPredBlocksPerWave && j0 + lane < B - 1 ? vmax_r[j0 + lane]
                                                                             : -INFINITY;
  float vv[kPredBlocksPerWave], dd[kPredBlocksPerWave];
  // slot 64 j0 - 64 + lane: only lanes >= 64 - (ROWS - 1) are read by the shifts
  const int ip = j0 * SPIN_BLOCK - SPIN_BLOCK + lane;
  const float dprev = lane >= SPIN_BLOCK - (ROWS - 1) && ip < N ? Dr[q0 - ip] : 0.0f;
#pragma unroll
  for (int b = 0; b < kPredBlocksPerWave; ++b) {
    const int i = (j0 + b) * SPIN_BLOCK + lane;
    const bool ok = i < N;
    const bool cached = vmax_r && j0 + b < B - 1;
    vv[b] = ok && !cached ? Vr[i] : -INFINITY;
    dd[b] = ok ? Dr[q0 - i] : 0.0f;
  }
  if (pooling == SPIN_POOL_MAX) {
    // every (row, block) maximum at once: a reduce-scatter over the wave
    // instead of ROWS x 8 wave reductions (the kernel is bound by VALU issue)
    constexpr int NV = ROWS * kPredBlocksPerWave <= 16 ? 16 : 32;
    constexpr int SH = NV == 16 ? 2 : 1;  // lane l holds value l >> SH
    float x[NV];
#pragma unroll
    for (int b = 0; b < kPredBlocksPerWave; ++b) {
      const int i = (j0 + b) * SPIN_BLOCK + lane;
      const float before = b == 0 ? dprev : dd[b > 0 ? b - 1 : 0];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        float d = dd[b];
        if (r > 0) {
          const int src = (lane - r) & 63;
          const float xs = __shfl(dd[b], src), ys = __shfl(before, src);
          d = lane >= r ? xs : ys;
        }
        const float zhat = combine == SPIN_COMBINE_SUM ? __fadd_rn(vv[b], d) : fmaxf(vv[b], d);
        x[r * kPredBlocksPerWave + b] = i < N ? zhat : -INFINITY;
      }
    }
#pragma unroll
    for (int k = ROWS * kPredBlocksPerWave; k < NV; ++k) x[k] = -INFINITY;
    float m = wave_max_scatter<NV>(x);
    const int idx = lane >> SH, r = idx / kPredBlocksPerWave, j = j0 + idx % kPredBlocksPerWave;
    if (vmax_r && j < B - 1) m = fmaxf(m, vmax_r[j]);
    if ((lane & ((1 << SH) - 1)) == 0 && r < ROWS && j < B)
      S0[(int64_t)r * max_blocks + j] = m + 0.0f;
    return;
  }
#pragma unroll
  for (int b = 0; b < kPredBlocksPerWave; ++b) {
    const int j = j0 + b;
    const int i = j * SPIN_BLOCK + lane;
    const float before = b == 0 ? dprev : dd[b > 0 ? b - 1 : 0];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      float d = dd[b];
      if (r > 0) {
        const int src = (lane - r) & 63;
        const float x = __shfl(dd[b], src), y = __shfl(before, src);
        d = lane >= r ? x : y;
      }
      const float zhat = combine == SPIN_COMBINE_SUM ? __fadd_rn(vv[b], d) : fmaxf(vv[b], d);
      const float m =
          pooling == SPIN_POOL_MAX
              ? fmaxf(wave_max_f32(i < N ? zhat : -INFINITY),
                      __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vm), b)))
              : pool_block_wave(zhat, i < N, min(SPIN_BLOCK, N - j * SPIN_BLOCK), pooling);
      if (lane == 0 && j < B) S0[(int64_t)r * max_blocks + j] = m + 0.0f;
    }
  }
}

template <int ROWS>
__global__ __launch_bounds__(256) void k_predict_rows(int combine, int pooling, int max_blocks,
                                                      const int32_t* __restrict__ ctx,
                                                      const int32_t* __restrict__ qpos,
                                                      const float* __restrict__ V, int64_t v_ld,
                                                      const float* __restrict__ D, int64_t d_ld,
                                                      const float* __restrict__ vmax,
                                                      float* __restrict__ S, int32_t* err,
                                                      int32_t* __restrict__ qpos_snap,
                                                      const int32_t* __restrict__ step,
                                                      const int32_t* __restrict__ tag) {
  const int r = blockIdx.z;
  const int N = ctx[r], q0 = qpos[r];
  if (qpos_snap && blockIdx.x == 0 && threadIdx.x == 0) qpos_snap[r] = q0;
  const int e = request_error(N, q0, ROWS, max_blocks, v_ld, d_ld);
  if (e) {
    if (blockIdx.x == 0 && threadIdx.x == 0) raise_error(err, e);
    return;
  }
  if (predicted_ahead(tag, step, r, q0, N)) return;
  const int B = (N + SPIN_BLOCK - 1) / SPIN_BLOCK;
  const int j0 = (blockIdx.x * 4 + (int)(threadIdx.x >> 6)) * kPredBlocksPerWave;
  if (j0 >= B) return;
  predict_wave_rows<ROWS>(combine, pooling, N, B, q0, j0, V + (int64_t)r * v_ld,
                          D + (int64_t)r * d_ld,
                          vmax ? vmax + (int64_t)r * max_blocks : nullptr,
                          S + (int64_t)r * ROWS * max_blocks, max_blocks);
}

__global__ __launch_bounds__(256) void k_predict(int combine, int pooling, int rows,
                                                 int max_blocks,
                                                 const int32_t* __restrict__ ctx,
                                                 const int32_t* __restrict__ qpos,
                                                 const float* __restrict__ V, int64_t v_ld,
                                                 const float* __restrict__ D, int64_t d_ld,
                                                 const float* __restrict__ vmax,
                                                 float* __restrict__ S, int32_t* err,
                                                 int32_t* __restrict__ qpos_snap,
                                                 const int32_t* __restrict__ step,
                                                 const int32_t* __restrict__ tag) {
  const int r = blockIdx.z, row = blockIdx.y;
  const int N = ctx[r], q0 = qpos[r];
  // a whole step keeps the step's query position here for the fused EMA +
  // counter advance, which then never reads the array it advances
  if (qpos_snap && blockIdx.x == 0 && row == 0 && threadIdx.x == 0) qpos_snap[r] = q0;
  const int e = request_error(N, q0, rows, max_blocks, v_ld, d_ld);
  if (e) {
    if (row == 0 && blockIdx.x == 0 && threadIdx.x == 0) raise_error(err, e);
    return;
  }
  if (predicted_ahead(tag, step, r, q0, N)) return;
  const int B = (N + SPIN_BLOCK - 1) / SPIN_BLOCK;
  const int j0 = (blockIdx.x * 4 + (int)(threadIdx.x >> 6)) * kPredBlocksPerWave;
  if (j0 >= B) return;
  predict_wave(combine, pooling, N, B, q0 + row, j0, V + (int64_t)r * v_ld,
               D + (int64_t)r * d_ld,
               vmax ? vmax + (int64_t)r * max_blocks : nullptr,
               S + ((int64_t)r * rows + row) * max_blocks);
}

// Union of request r's row masks (Sec. 3.2.2), compacted to its block list.
template <int EPT>
__device__ __forceinline__ void union_row(int rows, int n_use, int max_blocks, int r, int B,
                                          const uint8_t* __restrict__ code,
                                          int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
                                          int* sh, int32_t* last_obs, int t, int32_t* inv) {
  const int j0 = threadIdx.x * EPT;
  uint32_t any = 0u;
  for (int row = 0; row < n_use; ++row) {  // the first n_use rows' masks
    const uint8_t* crow = code + ((int64_t)r * rows + row) * max_blocks;
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (j0 + e < B && crow[j0 + e] != SPIN_CODE_SKIP) any |= 1u << e;
  }
  compact_blocks<EPT>(any, max_blocks, sel + (int64_t)r * max_blocks, n_sel + r, sh,
                      inv ? inv + (int64_t)r * max_blocks : nullptr);
  record_observed<EPT>(last_obs ? last_obs + (int64_t)r * max_blocks : nullptr, j0, B, any, t);
}

template <int EPT>
__global__ __launch_bounds__(kSelectThreads) void k_select(
    SelectArgs a, const int32_t* __restrict__ ctx, const int32_t* __restrict__ qpos,
    const int32_t* __restrict__ step, const int32_t* __restrict__ req_id,
    const float* __restrict__ S, const int32_t* __restrict__ budget, int compact) {
  __shared__ SelectLds L;
  const int row = blockIdx.x, r = blockIdx.y;
  const int N = ctx[r];
  const bool bad = request_error(N, qpos[r], a.rows, a.max_blocks, 0, 0) != 0;
  const int B = bad ? 0 : (N + SPIN_BLOCK - 1) / SPIN_BLOCK;
  select_row<EPT>(a, r, row, B, step[r], req_id[r], budget ? budget[r] : 0,
                  S + ((int64_t)r * a.rows + row) * a.max_blocks, compact != 0, L);
}

// Union of the verifier rows' masks (Sec. 3.2.2), one workgroup per request.
template <int EPT>
__global__ __launch_bounds__(kSelThreads) void k_union(int rows, int n_use, int max_blocks,
                                                       const int32_t* __restrict__ ctx,
                                                       const int32_t* __restrict__ qpos,
                                                       const int32_t* __restrict__ step,
                                                       const uint8_t* __restrict__ code,
                                                       int32_t* __restrict__ sel,
                                                       int32_t* __restrict__ n_sel,
                                                       int32_t* last_obs, int32_t* inv) {
  __shared__ int sh[32];
  const int r = blockIdx.x;
  const int N = ctx[r];
  const bool bad = request_error(N, qpos[r], rows, max_blocks, 0, 0) != 0;
  const int B = bad ? 0 : (N + SPIN_BLOCK - 1) / SPIN_BLOCK;
  union_row<EPT>(rows, n_use, max_blocks, r, B, code, sel, n_sel, sh, last_obs, step[r], inv);
}

// ---------------------------------------------------------------------------
// Block reduction A2 (Sec. 4.6): block scores straight from block-level
// states, S[r][row][j] = C(V[j], D[floor(q_row / 64) - j]).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_predict_a2(int combine, int rows, int max_blocks,
                                                    const int32_t* __restrict__ ctx,
                                                    const int32_t* __restrict__ qpos,
                                                    const float* __restrict__ V, int64_t v_ld,
                                                    const float* __restrict__ D, int64_t d_ld,
                                                    float* __restrict__ S, int32_t* err,
                                                    int32_t* __restrict__ qpos_snap) {
  const int r = blockIdx.z, row = blockIdx.y;
  const int N = ctx[r], q0 = qpos[r];
  if (qpos_snap && blockIdx.x == 0 && row == 0 && threadIdx.x == 0) qpos_snap[r] = q0;
  const int e = request_error(N, q0, rows, max_blocks, v_ld, d_ld);
  if (e) {
    if (row == 0 && blockIdx.x == 0 && threadIdx.x == 0) raise_error(err, e);
    return;
  }
  const int B = (N + SPIN_BLOCK - 1) / SPIN_BLOCK;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= B) return;
  const int bq = (q0 + row) / SPIN_BLOCK;
  const float v = V[(int64_t)r * v_ld + j], d = D[(int64_t)r * d_ld + (bq - j)];
  const float m = combine == SPIN_COMBINE_SUM ? __fadd_rn(v, d) : fmaxf(v, d);
  S[((int64_t)r * rows + row) * max_blocks + j] = m + 0.0f;
}

// ---------------------------------------------------------------------------
// Block reduction A0 (Sec. 4.6): the predicted slot scores of every slot,
// C(V[i], D[q_row - i]), written where the indexer scores go (z, block j at
// [64 j, 64 j + 64)) with every block listed in sel, so the top-K kernels
// can pick each row's K largest; then the blocks holding them.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_predict_slots(int combine, int rows, int max_blocks,
                                                       const int32_t* __restrict__ ctx,
                                                       const int32_t* __restrict__ qpos,
                                                       const float* __restrict__ V, int64_t v_ld,
                                                       const float* __restrict__ D, int64_t d_ld,
                                                       float* __restrict__ z, int64_t z_ld,
                                                       int32_t* __restrict__ sel,
                                                       int32_t* __restrict__ n_sel) {
  const int r = blockIdx.z, row = blockIdx.y;
  const int N = ctx[r], q0 = qpos[r];
  const bool bad = request_error(N, q0, rows, max_blocks, v_ld, d_ld) != 0;
  const int B = bad ? 0 : (N + SPIN_BLOCK - 1) / SPIN_BLOCK;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (row == 0 && i == 0) n_sel[r] = B;
  if (row == 0 && i < max_blocks) sel[(int64_t)r * max_blocks + i] = i < B ? i : -1;
  if (i >= SPIN_BLOCK * B) return;
  const int q = q0 + row;
  float zhat = 0.0f;
  if (i < N) {
    const float v = V[(int64_t)r * v_ld + i], d = D[(int64_t)r * d_ld + (q - i)];
    zhat = combine == SPIN_COMBINE_SUM ? __fadd_rn(v, d) : fmaxf(v, d);
  }
  z[((int64_t)r * rows + row) * z_ld + i] = zhat + 0.0f;
}

// The row's A0 mask from its top-K predicted slots (topk: ascending slot ids,
// -1 padded): every block holding one, the forced blocks, then
// floor(|mask| gamma) explored blocks from the rest under the policy.
template <int EPT>
__global__ __launch_bounds__(kSelectThreads) void k_a0_select(
    SelectArgs a, const int32_t* __restrict__ ctx, const int32_t* __restrict__ qpos,
    const int32_t* __restrict__ step, const int32_t* __restrict__ req_id,
    const float* __restrict__ S, const int32_t* __restrict__ topk, int compact) {
  __shared__ SelectLds L;
  __shared__ uint8_t hit[SPIN_MAX_BLOCKS];
  const int row = blockIdx.x, r = blockIdx.y;
  const int N = ctx[r];
  const bool bad = request_error(N, qpos[r], a.rows, a.max_blocks, 0, 0) != 0;
  const int B = bad ? 0 : (N + SPIN_BLOCK - 1) / SPIN_BLOCK;
  const int t = step[r];
  const int j0 = threadIdx.x * EPT;
  for (int j = threadIdx.x; j < a.max_blocks; j += kSelectThreads) hit[j] = 0;
  __syncthreads();
  if (B > 0 && t > 0) {
    const int32_t* trow = topk + ((int64_t)r * a.rows + row) * a.K;
    for (int k = threadIdx.x; k < a.K; k += kSelectThreads) {
      const int s = trow[k];
      if (s >= 0 && s < N) hit[s >> 6] = 1;
    }
  }
  __syncthreads();
  uint8_t* crow = a.code + ((int64_t)r * a.rows + row) * a.max_blocks;
  uint8_t c[EPT];
  uint32_t chosen = 0u, elig = 0u;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int j = j0 + e;
    c[e] = SPIN_CODE_SKIP;
    if (j >= B) continue;
    if (t == 0) c[e] = SPIN_CODE_DENSE;
    else if (j == 0 || j == B - 1) c[e] = SPIN_CODE_FORCED;
    else if (hit[j]) c[e] = SPIN_CODE_RANKED;
    if (c[e] != SPIN_CODE_SKIP) chosen |= 1u << e;
    else elig |= 1u << e;
  }
  const int m = block_sum_i32<kSelectThreads>(__popc(chosen), L.sh);
  // at most the blocks left outside the mask
  const int n_e = t > 0 ? min((int)((int64_t)m * a.explore_bp / 10000), B - m) : 0;
  if (n_e > 0) {
    const int32_t* orow = a.last_obs ? a.last_obs + (int64_t)r * a.max_blocks : nullptr;
    const float* Srow = S + ((int64_t)r * a.rows + row) * a.max_blocks;
    uint32_t pk[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int j = j0 + e;
      const bool in = j < B;
      const int obs = a.policy != kExploreRandom && orow && in ? orow[j] : 0;
      const float sv = a.policy == kExploreStaleness && in ? Srow[j] : 0.0f;
      pk[e] = policy_key(a, j, t, row, req_id[r], sv, obs);
    }
    const uint32_t expl = block_select_top<EPT, kSelectThreads>(pk, elig, n_e, L.hist, L.sh,
                                                                L.tmpu);
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (expl >> e & 1u) c[e] = SPIN_CODE_EXPLORED;
    chosen |= expl;
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if (j0 + e < B) crow[j0 + e] = c[e];
  if (compact) {
    compact_blocks<EPT, kSelectThreads>(chosen, a.max_blocks, a.sel + (int64_t)r * a.max_blocks,
                                        a.n_sel + r, L.sh);
    record_observed<EPT>(a.last_obs ? a.last_obs + (int64_t)r * a.max_blocks : nullptr, j0, B,
                         chosen, t);
  }
}

__global__ void k_advance(int R, int rows, const int32_t* __restrict__ n_valid,
                          int32_t* __restrict__ qpos, int32_t* __restrict__ step) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  if (qpos) qpos[r] += n_valid ? n_valid[r] : rows;
  if (step) step[r] += 1;
}

__global__ void k_fill_zero(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}
__global__ void k_zero_i32(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
// The V block maxima stand in for V only under the max combine and max pooling.
static bool vmax_usable(const spin_config& c) {
  return c.combine == SPIN_COMBINE_MAX && (c.flags & SPIN_POOL_MASK) == SPIN_POOL_MAX;
}

template <int ROWS>
static void predict_rows_t(const spin_config& c, const spin_batch& b, const float* V,
                           int64_t v_ld, const float* D, int64_t d_ld, const float* vmax,
                           float* S, hipStream_t st, int32_t* qpos_snap, const int32_t* tag) {
  dim3 grid((b.max_blocks + 4 * kPredBlocksPerWave - 1) / (4 * kPredBlocksPerWave), 1, b.batch);
  const int pooling = c.flags & SPIN_POOL_MASK;
  hipLaunchKernelGGL(k_predict_rows<ROWS>, grid, dim3(256), 0, st, c.combine, pooling,
                     b.max_blocks, b.ctx_len, b.q_pos, V, v_ld, D, d_ld,
                     vmax_usable(c) ? vmax : nullptr, S, b.err, qpos_snap, b.step, tag);
}

hipError_t launch_predict(const spin_config& c, const spin_batch& b, const float* V, int64_t v_ld,
                          const float* D, int64_t d_ld, const float* vmax, float* S,
                          hipStream_t st, int32_t* qpos_snap, const int32_t* tag) {
  if (b.n_rows > 1) {  // every row from one load of V and D
    switch (b.n_rows) {
      case 2: predict_rows_t<2>(c, b, V, v_ld, D, d_ld, vmax, S, st, qpos_snap, tag); break;
      case 3: predict_rows_t<3>(c, b, V, v_ld, D, d_ld, vmax, S, st, qpos_snap, tag); break;
      default: predict_rows_t<4>(c, b, V, v_ld, D, d_ld, vmax, S, st, qpos_snap, tag); break;
    }
    return hipGetLastError();
  }
  dim3 grid((b.max_blocks + 4 * kPredBlocksPerWave - 1) / (4 * kPredBlocksPerWave), b.n_rows,
            b.batch);
  hipLaunchKernelGGL(k_predict, grid, dim3(256), 0, st, c.combine, c.flags & SPIN_POOL_MASK,
                     b.n_rows, b.max_blocks, b.ctx_len, b.q_pos, V, v_ld, D, d_ld,
                     vmax_usable(c) ? vmax : nullptr, S, b.err, qpos_snap, b.step, tag);
  return hipGetLastError();
}

static SelectArgs select_args(const spin_config& c, const spin_batch& b, uint8_t* code,
                              int32_t* sel, int32_t* n_sel, int32_t* last_obs,
                              int32_t* inv = nullptr) {
  const int pol = c.flags & SPIN_EXPLORE_POLICY_MASK;
  return SelectArgs{c.topk, c.sparsity_bp, c.explore_bp, c.layer,
                    (c.flags & SPIN_EXPLORE_PER_ROW) != 0,
                    (uint32_t)(c.seed & 0xFFFFFFFFu), (uint32_t)(c.seed >> 32), b.n_rows,
                    b.max_blocks, code, sel, n_sel,
                    pol == SPIN_EXPLORE_AGE ? kExploreAge
                                            : pol == SPIN_EXPLORE_STALENESS ? kExploreStaleness
                                                                            : kExploreRandom,
                    last_obs, inv};
}

PredictPlan predict_plan(const spin_config& c, const spin_batch& b, const float* V, int64_t v_ld,
                         const float* D, int64_t d_ld, const float* vmax, float* S,
                         int32_t* qpos_snap, const int32_t* tag) {
  const int per_req = (b.max_blocks + kPredBlocksPerWg - 1) / kPredBlocksPerWg;
  return PredictPlan{PredictArgs{c.combine, c.flags & SPIN_POOL_MASK, b.max_blocks, per_req,
                                 b.ctx_len, b.q_pos, V, v_ld, D, d_ld,
                                 vmax_usable(c) ? vmax : nullptr, S, b.err, qpos_snap, b.step,
                                 tag},
                     b.batch * per_req};
}

// blocks per thread of the 1,024-thread selection (max_blocks <= 8,192)
static int select_ept(int max_blocks) {
  const int ept = (max_blocks + kSelectThreads - 1) / kSelectThreads;
  return ept <= 1 ? 1 : ept <= 2 ? 2 : ept <= 4 ? 4 : 8;
}

template <int EPT>
static void select_t(const spin_config& c, const spin_batch& b, const float* S,
                     const int32_t* budget, uint8_t* code, int32_t* sel, int32_t* n_sel,
                     int32_t* last_obs, hipStream_t st, int32_t* inv) {
  const int compact = b.n_rows == 1;
  hipLaunchKernelGGL(k_select<EPT>, dim3(b.n_rows, b.batch), dim3(kSelectThreads), 0, st,
                     select_args(c, b, code, sel, n_sel, last_obs, inv), b.ctx_len, b.q_pos,
                     b.step,
                     b.req_id, S, budget, compact);
}

template <int EPT>
static void a0_select_t(const spin_config& c, const spin_batch& b, const float* S,
                        const int32_t* topk, uint8_t* code, int32_t* sel, int32_t* n_sel,
                        int32_t* last_obs, hipStream_t st) {
  const int compact = b.n_rows == 1;
  hipLaunchKernelGGL(k_a0_select<EPT>, dim3(b.n_rows, b.batch), dim3(kSelectThreads), 0, st,
                     select_args(c, b, code, sel, n_sel, last_obs), b.ctx_len, b.q_pos, b.step,
                     b.req_id, S, topk, compact);
}

template <int EPT>
static void union_t(const spin_config& c, const spin_batch& b, uint8_t* code, int32_t* sel,
                    int32_t* n_sel, int32_t* last_obs, hipStream_t st, int32_t* inv) {
  // row-0 sharing scores row 0's mask alone
  const int n_use = (c.flags & SPIN_MTP_ROW0_MASK) ? 1 : b.n_rows;
  hipLaunchKernelGGL(k_union<EPT>, dim3(b.batch), dim3(kSelThreads), 0, st, b.n_rows, n_use,
                     b.max_blocks, b.ctx_len, b.q_pos, b.step, code, sel, n_sel, last_obs, inv);
}

static void launch_union(const spin_config& c, const spin_batch& b, uint8_t* code, int32_t* sel,
                         int32_t* n_sel, int32_t* last_obs, hipStream_t st,
                         int32_t* inv = nullptr) {
  const int eu = (b.max_blocks + kSelThreads - 1) / kSelThreads;
  if (eu <= 1) union_t<1>(c, b, code, sel, n_sel, last_obs, st, inv);
  else if (eu <= 2) union_t<2>(c, b, code, sel, n_sel, last_obs, st, inv);
  else if (eu <= 4) union_t<4>(c, b, code, sel, n_sel, last_obs, st, inv);
  else union_t<8>(c, b, code, sel, n_sel, last_obs, st, inv);
}

SelectPlan select_plan(const spin_config& c, const spin_batch& b, const float* S,
                       const int32_t* budget, uint8_t* code, int32_t* sel, int32_t* n_sel,
                       int32_t* last_obs, int32_t* inv) {
  return SelectPlan{select_args(c, b, code, sel, n_sel, last_obs, inv),
                    SelectInputs{b.ctx_len, b.q_pos, b.step, b.req_id, S, budget}, b.batch,
                    select_ept(b.max_blocks)};
}

hipError_t launch_select(const spin_config& c, const spin_batch& b, const float* S,
                         const int32_t* budget, uint8_t* code, int32_t* sel, int32_t* n_sel,
                         int32_t* last_obs, hipStream_t st, int32_t* inv) {
  switch (select_ept(b.max_blocks)) {
    case 1: select_t<1>(c, b, S, budget, code, sel, n_sel, last_obs, st, inv); break;
    case 2: select_t<2>(c, b, S, budget, code, sel, n_sel, last_obs, st, inv); break;
    case 4: select_t<4>(c, b, S, budget, code, sel, n_sel, last_obs, st, inv); break;
    default: select_t<8>(c, b, S, budget, code, sel, n_sel, last_obs, st, inv); break;
  }
  if (b.n_rows > 1) launch_union(c, b, code, sel, n_sel, last_obs, st, inv);  // the rows' masks
  return hipGetLastError();
}

hipError_t launch_predict_a2(const spin_config& c, const spin_batch& b, const float* V,
                             int64_t v_ld, const float* D, int64_t d_ld, float* S,
                             hipStream_t st, int32_t* qpos_snap) {
  dim3 grid((b.max_blocks + 255) / 256, b.n_rows, b.batch);
  hipLaunchKernelGGL(k_predict_a2, grid, dim3(256), 0, st, c.combine, b.n_rows, b.max_blocks,
                     b.ctx_len, b.q_pos, V, v_ld, D, d_ld, S, b.err, qpos_snap);
  return hipGetLastError();
}

hipError_t launch_predict_slots(const spin_config& c, const spin_batch& b, const float* V,
                                int64_t v_ld, const float* D, int64_t d_ld, float* z,
                                int64_t z_ld, int32_t* sel, int32_t* n_sel, hipStream_t st) {
  dim3 grid((SPIN_BLOCK * b.max_blocks + 255) / 256, b.n_rows, b.batch);
  hipLaunchKernelGGL(k_predict_slots, grid, dim3(256), 0, st, c.combine, b.n_rows, b.max_blocks,
                     b.ctx_len, b.q_pos, V, v_ld, D, d_ld, z, z_ld, sel, n_sel);
  return hipGetLastError();
}

hipError_t launch_a0_select(const spin_config& c, const spin_batch& b, const float* S,
                            const int32_t* topk, uint8_t* code, int32_t* sel, int32_t* n_sel,
                            int32_t* last_obs, hipStream_t st) {
  switch (select_ept(b.max_blocks)) {
    case 1: a0_select_t<1>(c, b, S, topk, code, sel, n_sel, last_obs, st); break;
    case 2: a0_select_t<2>(c, b, S, topk, code, sel, n_sel, last_obs, st); break;
    case 4: a0_select_t<4>(c, b, S, topk, code, sel, n_sel, last_obs, st); break;
    default: a0_select_t<8>(c, b, S, topk, code, sel, n_sel, last_obs, st); break;
  }
  if (b.n_rows > 1) launch_union(c, b, code, sel, n_sel, last_obs, st);
  return hipGetLastError();
}

hipError_t launch_advance(int R, int rows, const int32_t* n_valid, int32_t* qpos, int32_t* step,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_advance, dim3((R + 255) / 256), dim3(256), 0, st, R, rows, n_valid, qpos,
                     step);
  return hipGetLastError();
}

hipError_t launch_reset(int R, float* V, int64_t v_ld, float* D, int64_t d_ld, int64_t vmax_ld,
                        float* vmax, int32_t* step, hipStream_t st) {
  const int64_t nv = (int64_t)R * v_ld, nd = (int64_t)R * d_ld, nm = (int64_t)R * vmax_ld;
  if (nv > 0) hipLaunchKernelGGL(k_fill_zero, dim3(1024), dim3(256), 0, st, V, nv);
  if (nd > 0) hipLaunchKernelGGL(k_fill_zero, dim3(1024), dim3(256), 0, st, D, nd);
  if (vmax && nm > 0) hipLaunchKernelGGL(k_fill_zero, dim3(256), dim3(256), 0, st, vmax, nm);
  if (step) hipLaunchKernelGGL(k_zero_i32, dim3((R + 255) / 256), dim3(256), 0, st, step, R);
  return hipGetLastError();
}

}  // namespace spin
