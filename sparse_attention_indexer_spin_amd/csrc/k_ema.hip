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
#include "spin_dev.h"
#include "spin_launch.h"

namespace spin {

struct EmaCtx {
  float a, b;
  int L, N, q, j, k, ns;
  const float* zb;  // z of this request, row 0
  int64_t z_ld;
  const int32_t* sel;  // this request's selected blocks
};

__device__ __forceinline__ float ema_step(float x, float zv, float a, float b) {
  return __fadd_rn(__fmul_rn(a, x), __fmul_rn(b, zv));
}

__device__ __forceinline__ void ema_offset(const EmaCtx& e, int s0, float* Dr) {
  if (s0 >= e.N) return;
  const int o = e.q - s0;
  float d = 0.0f;
  bool upd = false;
  for (int row = 0; row < e.L; ++row) {
    const int slot = s0 + row;
    if (slot < 0 || slot >= e.N) continue;
    const int blk = slot >> 6;
    int kk = -1;
    if (blk == e.j) kk = e.k;
    else if (blk == e.j + 1 && e.k + 1 < e.ns && e.sel[e.k + 1] == e.j + 1) kk = e.k + 1;
    if (kk < 0) continue;
    if (!upd) d = Dr[o];
    d = ema_step(d, e.zb[row * e.z_ld + kk * 64 + (slot & 63)], e.a, e.b);
    upd = true;
  }
  if (upd) Dr[o] = d;
}

constexpr int kEmaBlocksPerWave = 4;

__global__ __launch_bounds__(256) void k_ema(float alpha, int rows, int max_blocks,
                                             const int32_t* __restrict__ ctx,
                                             const int32_t* __restrict__ qpos,
                                             const int32_t* __restrict__ n_valid,
                                             const float* __restrict__ z, int64_t z_ld,
                                             const int32_t* __restrict__ sel,
                                             const int32_t* __restrict__ n_sel,
                                             float* __restrict__ V, int64_t v_ld,
                                             float* __restrict__ D, int64_t d_ld,
                                             int32_t* __restrict__ qpos_out,
                                             int32_t* __restrict__ step_out) {
  const int r = blockIdx.y;
  const int k0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kEmaBlocksPerWave;
  const int lane = threadIdx.x & 63;
  const int N = ctx[r], q = qpos[r];
  // fused counter advance (qpos is then the step's snapshot, not qpos_out)
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (qpos_out) qpos_out[r] = q + (n_valid ? n_valid[r] : rows);
    if (step_out) step_out[r] += 1;
  }
  if (request_error(N, q, rows, max_blocks, v_ld, d_ld)) return;
  const int ns = clamp_nsel(n_sel[r], max_blocks);
  if (k0 >= ns) return;
  int L = n_valid ? n_valid[r] : rows;
  L = L < 0 ? 0 : (L > rows ? rows : L);
  if (L == 0) return;
  const int32_t* sr = sel + (int64_t)r * max_blocks;
  const float a = alpha, b = __fsub_rn(1.0f, alpha);
  const float* zb = z + (int64_t)r * rows * z_ld;
  float* Vr = V + (int64_t)r * v_ld;
  float* Dr = D + (int64_t)r * d_ld;
  if (L == 1) {
    // one observation per slot: V[i] and D[q - i] from row 0, loads batched
    float vv[kEmaBlocksPerWave], dd[kEmaBlocksPerWave], zz[kEmaBlocksPerWave];
    int ii[kEmaBlocksPerWave];
#pragma unroll
    for (int u = 0; u < kEmaBlocksPerWave; ++u) {
      const int k = k0 + u;
      const int j = k < ns ? sr[k] : -1;
      const int i = j * 64 + lane;
      const bool ok = k < ns && j >= 0 && j < max_blocks && i < N;
      ii[u] = ok ? i : -1;
      vv[u] = ok ? Vr[i] : 0.0f;
      dd[u] = ok ? Dr[q - i] : 0.0f;
      zz[u] = ok ? zb[(int64_t)k * 64 + lane] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kEmaBlocksPerWave; ++u) {
      if (ii[u] < 0) continue;
      Vr[ii[u]] = ema_step(vv[u], zz[u], a, b);
      Dr[q - ii[u]] = ema_step(dd[u], zz[u], a, b);
    }
    return;
  }
  for (int u = 0; u < kEmaBlocksPerWave; ++u) {
    const int k = k0 + u;
    if (k >= ns) break;
    EmaCtx e;
    e.a = a; e.b = b;
    e.L = L; e.N = N; e.q = q; e.k = k; e.ns = ns;
    e.j = sr[k];
    if (e.j < 0 || e.j >= max_blocks) continue;
    e.zb = zb;
    e.z_ld = z_ld;
    e.sel = sr;
    const int i = e.j * 64 + lane;
    if (i < N) {
      float v = Vr[i];
      for (int row = 0; row < L; ++row) v = ema_step(v, zb[row * z_ld + (int64_t)k * 64 + lane], a, b);
      Vr[i] = v;
    }
    ema_offset(e, i, Dr);
    if (lane < L - 1) {
      const bool prev_selected = k > 0 && sr[k - 1] == e.j - 1;
      if (!prev_selected) ema_offset(e, e.j * 64 - 1 - lane, Dr);
    }
  }
}

hipError_t launch_ema(const spin_config& c, const spin_batch& b, const float* z, int64_t z_ld,
                      const int32_t* sel, const int32_t* n_sel, const int32_t* n_valid, float* V,
                      int64_t v_ld, float* D, int64_t d_ld, hipStream_t st,
                      const int32_t* qpos_snap, int32_t* qpos_out, int32_t* step_out) {
  dim3 grid((b.max_blocks + 4 * kEmaBlocksPerWave - 1) / (4 * kEmaBlocksPerWave), b.batch);
  hipLaunchKernelGGL(k_ema, grid, dim3(256), 0, st, c.ema_alpha, b.n_rows, b.max_blocks,
                     b.ctx_len, qpos_snap ? qpos_snap : b.q_pos, n_valid, z, z_ld, sel, n_sel, V,
                     v_ld, D, d_ld, qpos_out, step_out);
  return hipGetLastError();
}

}  // namespace spin
