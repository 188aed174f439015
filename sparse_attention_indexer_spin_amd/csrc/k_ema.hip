// Stage 4 of the SPIN decode step: EMA update of the vertical (per slot) and
// diagonal (per query offset) states from the fresh indexer scores
// ("SPIN: Shadow Predictive Indexer for Sparse Attention", Algorithm 1 steps
// 8-10), replayed for the prefix-valid verifier rows in row order under
// speculative decoding (Sec. 3.2.2).
//
// Every update is  x <- (alpha * x) + (beta * z)  with each product and the
// sum rounded to fp32 separately (no fused multiply-add), beta = 1 - alpha in
// fp32, so the state is bit-reproducible.
//
// Ownership (race-free, rows applied in order per element):
//   * V[i]: the lane of slot i applies rows 0..L-1.
//   * D[o]: offset o is touched by row r at slot s0 + r where s0 = q - o is the
//     row-0 slot.  The lane of slot s0 owns o when s0's block is selected;
//     otherwise the next selected block owns it through up to L-1 "extension"
//     slots just left of its first slot (L <= 4 < 64, so no other block can
//     reach o).
#include "ema_dev.h"
#include "plan_dev.h"
#include "spin_launch.h"

namespace spin {

// Block reduction A2 (Sec. 4.6, "Block reduction"): block-level V / D updated
// from each scored block's pooled score, rows in order.  One wave per
// selected block k (block j).  Row r updates V[j] and D[floor(q_r / 64) - j];
// with b0 = floor(q / 64), rows [0, c) have floor(q_r / 64) = b0 and rows
// [c, L) (if any) b0 + 1.  Ownership, every element by one wave:
//   * V[j]: block j's wave, all rows.
//   * D[b0 - j]: block j's wave -- rows [0, c) with block j's pooled score,
//     rows [c, L) with block j + 1's when j + 1 is selected.
//   * D[b0 + 1 - j] when block j - 1 is not selected (else block j - 1's wave
//     owns it): block j's wave, rows [c, L), with block j's score.
__global__ __launch_bounds__(256) void k_ema_a2(EmaArgs A, int pooling) {
  const int r = blockIdx.y;
  const int k = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int N = A.ctx[r], q = A.qpos[r];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (A.qpos_out) A.qpos_out[r] = q + (A.n_valid ? A.n_valid[r] : A.rows);
    if (A.step_out) A.step_out[r] += 1;
  }
  if (request_error(N, q, A.rows, A.max_blocks, A.v_ld, A.d_ld)) return;
  const int ns = clamp_nsel(A.n_sel[r], A.max_blocks);
  if (k >= ns) return;
  int L = A.row0_only ? 1 : (A.n_valid ? A.n_valid[r] : A.rows);
  L = L < 0 ? 0 : (L > A.rows ? A.rows : L);
  if (L == 0) return;
  const int32_t* sr = A.sel + (int64_t)r * A.max_blocks;
  const int j = __builtin_amdgcn_readfirstlane(sr[k]);
  if (j < 0 || j >= A.max_blocks || j * SPIN_BLOCK >= N) return;
  const bool next_sel = k + 1 < ns && sr[k + 1] == j + 1;
  const bool prev_sel = k > 0 && sr[k - 1] == j - 1;
  const int b0 = q / SPIN_BLOCK;
  int c = L;
  for (int row = 1; row < L; ++row)
    if ((q + row) / SPIN_BLOCK > b0) { c = row; break; }
  const bool own_b = !prev_sel && c < L;
  const float a = A.alpha, b = __fsub_rn(1.0f, A.alpha);
  const float* zr = A.z + (int64_t)r * A.rows * A.z_ld;
  float* Vr = A.V + (int64_t)r * A.v_ld;
  float* Dr = A.D + (int64_t)r * A.d_ld;
  const int nj = min(SPIN_BLOCK, N - j * SPIN_BLOCK);
  const int nn = next_sel ? min(SPIN_BLOCK, N - (j + 1) * SPIN_BLOCK) : 0;
  float v = Vr[j], da = Dr[b0 - j], db = own_b ? Dr[b0 + 1 - j] : 0.0f;
  for (int row = 0; row < L; ++row) {
    const float zj = zr[row * A.z_ld + (int64_t)k * SPIN_BLOCK + lane];
    const float pj = pool_block_wave(zj, lane < nj, nj, pooling) + 0.0f;
    v = ema_step(v, pj, a, b);
    if (row < c) {
      da = ema_step(da, pj, a, b);
    } else {
      if (own_b) db = ema_step(db, pj, a, b);
      if (next_sel) {
        const float zn = zr[row * A.z_ld + (int64_t)(k + 1) * SPIN_BLOCK + lane];
        da = ema_step(da, pool_block_wave(zn, lane < nn, nn, pooling) + 0.0f, a, b);
      }
    }
  }
  if (lane == 0) {
    Vr[j] = v;
    Dr[b0 - j] = da;
    if (own_b) Dr[b0 + 1 - j] = db;
  }
}

hipError_t launch_ema_a2(const spin_config& c, const spin_batch& b, const float* z, int64_t z_ld,
                         const int32_t* sel, const int32_t* n_sel, const int32_t* n_valid,
                         float* V, int64_t v_ld, float* D, int64_t d_ld, hipStream_t st,
                         const int32_t* qpos_snap, int32_t* qpos_out, int32_t* step_out) {
  dim3 grid((b.max_blocks + 3) / 4, b.batch);
  const EmaArgs A{c.ema_alpha, b.n_rows, b.max_blocks, b.ctx_len, qpos_snap ? qpos_snap : b.q_pos,
                  n_valid, z, z_ld, sel, n_sel, V, v_ld, D, d_ld, qpos_out, step_out, nullptr,
                  (c.flags & SPIN_MTP_ROW0_UPDATE) != 0};
  hipLaunchKernelGGL(k_ema_a2, grid, dim3(256), 0, st, A, c.flags & SPIN_POOL_MASK);
  return hipGetLastError();
}

// BPW blocks per wave: kEmaBlocksPerWave with one row; with several rows a
// wave's blocks are one chunk of the several-row update (kEmaChunkRows), whose
// loads are unconditional, so a wave's last chunk should not be a partial one.
template <int BPW>
__global__ __launch_bounds__(256) void k_ema(EmaArgs A) {
  const int r = blockIdx.y;
  const int k0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * BPW;
  ema_blocks<BPW>(A, r, k0, k0 + BPW, blockIdx.x == 0 && threadIdx.x == 0);
}

// The EMA update and the next step's block scores (SPIN_PREDICT_AHEAD, one
// row): wave w of each request's n takes blocks [w nb / n, (w + 1) nb / n).
__global__ __launch_bounds__(256) void k_ema_predict(EmaPredArgs P) {
  const int r = blockIdx.y;
  const int n = (int)gridDim.x * 4, w = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  ema_predict_blocks<4>(P, r, w, n, blockIdx.x == 0 && threadIdx.x == 0);
}

hipError_t launch_ema(const spin_config& c, const spin_batch& b, const float* z, int64_t z_ld,
                      const int32_t* sel, const int32_t* n_sel, const int32_t* n_valid, float* V,
                      int64_t v_ld, float* D, int64_t d_ld, float* vmax, hipStream_t st,
                      const int32_t* qpos_snap, int32_t* qpos_out, int32_t* step_out,
                      const Ahead* ahead) {
  const EmaArgs A{c.ema_alpha, b.n_rows, b.max_blocks, b.ctx_len, qpos_snap ? qpos_snap : b.q_pos,
                  n_valid, z, z_ld, sel, n_sel, V, v_ld, D, d_ld, qpos_out, step_out, vmax,
                  (c.flags & SPIN_MTP_ROW0_UPDATE) != 0};
  if (ahead) {
    // every block (and the one past the last, whose first lanes hold the
    // offset of the slot just beyond the context), 4 blocks per wave
    if (b.n_rows != 1) return hipErrorInvalidValue;
    dim3 grid((b.max_blocks + 1 + 15) / 16, b.batch);
    hipLaunchKernelGGL(k_ema_predict, grid, dim3(256), 0, st, ema_pred_args(c, A, ahead));
    return hipGetLastError();
  }
  if (b.n_rows > 1 && !A.row0_only) {
    constexpr int W = kEmaChunkRows;
    dim3 grid((b.max_blocks + 4 * W - 1) / (4 * W), b.batch);
    hipLaunchKernelGGL(k_ema<W>, grid, dim3(256), 0, st, A);
  } else {
    constexpr int W = kEmaBlocksPerWave;
    dim3 grid((b.max_blocks + 4 * W - 1) / (4 * W), b.batch);
    hipLaunchKernelGGL(k_ema<W>, grid, dim3(256), 0, st, A);
  }
  return hipGetLastError();
}

}  // namespace spin
