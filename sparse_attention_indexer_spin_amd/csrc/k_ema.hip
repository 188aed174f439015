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
#include "spin_launch.h"

namespace spin {

__global__ __launch_bounds__(256) void k_ema(EmaArgs A) {
  const int r = blockIdx.y;
  const int k0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kEmaBlocksPerWave;
  ema_wave(A, r, k0, blockIdx.x == 0 && threadIdx.x == 0);
}

hipError_t launch_ema(const spin_config& c, const spin_batch& b, const float* z, int64_t z_ld,
                      const int32_t* sel, const int32_t* n_sel, const int32_t* n_valid, float* V,
                      int64_t v_ld, float* D, int64_t d_ld, float* vmax, hipStream_t st,
                      const int32_t* qpos_snap, int32_t* qpos_out, int32_t* step_out) {
  dim3 grid((b.max_blocks + 4 * kEmaBlocksPerWave - 1) / (4 * kEmaBlocksPerWave), b.batch);
  const EmaArgs A{c.ema_alpha, b.n_rows, b.max_blocks, b.ctx_len, qpos_snap ? qpos_snap : b.q_pos,
                  n_valid, z, z_ld, sel, n_sel, V, v_ld, D, d_ld, qpos_out, step_out, vmax,
                  (c.flags & SPIN_MTP_ROW0_UPDATE) != 0};
  hipLaunchKernelGGL(k_ema, grid, dim3(256), 0, st, A);
  return hipGetLastError();
}

}  // namespace spin
