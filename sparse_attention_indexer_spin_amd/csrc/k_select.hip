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
                                                      int32_t* __restrict__ qpos_snap) {
  const int r = blockIdx.z;
  const int N = ctx[r], q0 = qpos[r];
  if (qpos_snap && blockIdx.x == 0 && threadIdx.x == 0) qpos_snap[r] = q0;
  const int e = request_error(N, q0, ROWS, max_blocks, v_ld, d_ld);
  if (e) {
    if (blockIdx.x == 0 && threadIdx.x == 0) raise_error(err, e);
    return;
  }
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
                                                 int32_t* __restrict__ qpos_snap) {
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
                                          int* sh) {
  const int j0 = threadIdx.x * EPT;
  uint32_t any = 0u;
  for (int row = 0; row < n_use; ++row) {  // the first n_use rows' masks
    const uint8_t* crow = code + ((int64_t)r * rows + row) * max_blocks;
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (j0 + e < B && crow[j0 + e] != SPIN_CODE_SKIP) any |= 1u << e;
  }
  compact_blocks<EPT>(any, max_blocks, sel + (int64_t)r * max_blocks, n_sel + r, sh);
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
                                                       const uint8_t* __restrict__ code,
                                                       int32_t* __restrict__ sel,
                                                       int32_t* __restrict__ n_sel) {
  __shared__ int sh[32];
  const int r = blockIdx.x;
  const int N = ctx[r];
  const bool bad = request_error(N, qpos[r], rows, max_blocks, 0, 0) != 0;
  const int B = bad ? 0 : (N + SPIN_BLOCK - 1) / SPIN_BLOCK;
  union_row<EPT>(rows, n_use, max_blocks, r, B, code, sel, n_sel, sh);
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
                           float* S, hipStream_t st, int32_t* qpos_snap) {
  dim3 grid((b.max_blocks + 4 * kPredBlocksPerWave - 1) / (4 * kPredBlocksPerWave), 1, b.batch);
  const int pooling = c.flags & SPIN_POOL_MASK;
  hipLaunchKernelGGL(k_predict_rows<ROWS>, grid, dim3(256), 0, st, c.combine, pooling,
                     b.max_blocks, b.ctx_len, b.q_pos, V, v_ld, D, d_ld,
                     vmax_usable(c) ? vmax : nullptr, S, b.err, qpos_snap);
}

hipError_t launch_predict(const spin_config& c, const spin_batch& b, const float* V, int64_t v_ld,
                          const float* D, int64_t d_ld, const float* vmax, float* S,
                          hipStream_t st, int32_t* qpos_snap) {
  if (b.n_rows > 1) {  // every row from one load of V and D
    switch (b.n_rows) {
      case 2: predict_rows_t<2>(c, b, V, v_ld, D, d_ld, vmax, S, st, qpos_snap); break;
      case 3: predict_rows_t<3>(c, b, V, v_ld, D, d_ld, vmax, S, st, qpos_snap); break;
      default: predict_rows_t<4>(c, b, V, v_ld, D, d_ld, vmax, S, st, qpos_snap); break;
    }
    return hipGetLastError();
  }
  dim3 grid((b.max_blocks + 4 * kPredBlocksPerWave - 1) / (4 * kPredBlocksPerWave), b.n_rows,
            b.batch);
  hipLaunchKernelGGL(k_predict, grid, dim3(256), 0, st, c.combine, c.flags & SPIN_POOL_MASK,
                     b.n_rows, b.max_blocks, b.ctx_len, b.q_pos, V, v_ld, D, d_ld,
                     vmax_usable(c) ? vmax : nullptr, S, b.err, qpos_snap);
  return hipGetLastError();
}

static SelectArgs select_args(const spin_config& c, const spin_batch& b, uint8_t* code,
                              int32_t* sel, int32_t* n_sel) {
  return SelectArgs{c.topk, c.sparsity_bp, c.explore_bp, c.layer,
                    (c.flags & SPIN_EXPLORE_PER_ROW) != 0,
                    (uint32_t)(c.seed & 0xFFFFFFFFu), (uint32_t)(c.seed >> 32), b.n_rows,
                    b.max_blocks, code, sel, n_sel};
}

PredictPlan predict_plan(const spin_config& c, const spin_batch& b, const float* V, int64_t v_ld,
                         const float* D, int64_t d_ld, const float* vmax, float* S,
                         int32_t* qpos_snap) {
  const int per_req = (b.max_blocks + kPredBlocksPerWg - 1) / kPredBlocksPerWg;
  return PredictPlan{PredictArgs{c.combine, c.flags & SPIN_POOL_MASK, b.max_blocks, per_req,
                                 b.ctx_len, b.q_pos, V, v_ld, D, d_ld,
                                 vmax_usable(c) ? vmax : nullptr, S, b.err, qpos_snap},
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
                     hipStream_t st) {
  const int compact = b.n_rows == 1;
  hipLaunchKernelGGL(k_select<EPT>, dim3(b.n_rows, b.batch), dim3(kSelectThreads), 0, st,
                     select_args(c, b, code, sel, n_sel), b.ctx_len, b.q_pos, b.step, b.req_id,
                     S, budget, compact);
}

template <int EPT>
static void union_t(const spin_config& c, const spin_batch& b, uint8_t* code, int32_t* sel,
                    int32_t* n_sel, hipStream_t st) {
  // row-0 sharing scores row 0's mask alone
  const int n_use = (c.flags & SPIN_MTP_ROW0_MASK) ? 1 : b.n_rows;
  hipLaunchKernelGGL(k_union<EPT>, dim3(b.batch), dim3(kSelThreads), 0, st, b.n_rows, n_use,
                     b.max_blocks, b.ctx_len, b.q_pos, code, sel, n_sel);
}

SelectPlan select_plan(const spin_config& c, const spin_batch& b, const float* S,
                       const int32_t* budget, uint8_t* code, int32_t* sel, int32_t* n_sel) {
  return SelectPlan{select_args(c, b, code, sel, n_sel),
                    SelectInputs{b.ctx_len, b.q_pos, b.step, b.req_id, S, budget}, b.batch,
                    select_ept(b.max_blocks)};
}

hipError_t launch_select(const spin_config& c, const spin_batch& b, const float* S,
                         const int32_t* budget, uint8_t* code, int32_t* sel, int32_t* n_sel,
                         hipStream_t st) {
  switch (select_ept(b.max_blocks)) {
    case 1: select_t<1>(c, b, S, budget, code, sel, n_sel, st); break;
    case 2: select_t<2>(c, b, S, budget, code, sel, n_sel, st); break;
    case 4: select_t<4>(c, b, S, budget, code, sel, n_sel, st); break;
    default: select_t<8>(c, b, S, budget, code, sel, n_sel, st); break;
  }
  if (b.n_rows > 1) {  // union of the rows' masks
    const int eu = (b.max_blocks + kSelThreads - 1) / kSelThreads;
    if (eu <= 1) union_t<1>(c, b, code, sel, n_sel, st);
    else if (eu <= 2) union_t<2>(c, b, code, sel, n_sel, st);
    else if (eu <= 4) union_t<4>(c, b, code, sel, n_sel, st);
    else union_t<8>(c, b, code, sel, n_sel, st);
  }
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
