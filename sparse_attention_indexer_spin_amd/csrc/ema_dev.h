// EMA update device code (Algorithm 1 steps 8-10 of "SPIN: Shadow Predictive
// Indexer for Sparse Attention"; deferred in-order replay of Sec. 3.2.2),
// shared by the EMA kernel and the kernel that runs it beside the top-K.
#pragma once
#include "spin_dev.h"

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
constexpr int kEmaChunkRows = 3;  // blocks whose loads a several-row EMA wave issues together

struct EmaArgs {
  float alpha;
  int rows, max_blocks;
  const int32_t* ctx;
  const int32_t* qpos;      // the step's q positions (a snapshot when advancing)
  const int32_t* n_valid;
  const float* z;
  int64_t z_ld;
  const int32_t* sel;
  const int32_t* n_sel;
  float* V;
  int64_t v_ld;
  float* D;
  int64_t d_ld;
  int32_t* qpos_out;        // optional counter advance
  int32_t* step_out;
  float* vmax;              // optional V block maxima [R][max_blocks]
  int row0_only;            // SPIN_MTP_ROW0_UPDATE: the EMA takes row 0 alone
};

// After block j's V update: its max over all 64 slots (slots >= N hold 0),
// `v` being lane i's new V[i] where i < N.
__device__ __forceinline__ void ema_vmax(const EmaArgs& A, int r, int j, bool in, float v) {
  const float m = wave_max_f32(in ? v : 0.0f);
  if (A.vmax && (threadIdx.x & 63) == 0) A.vmax[(int64_t)r * A.max_blocks + j] = m;
}

// One wave: the EMA update of selected blocks [k0, k1) of request r, CH
// blocks' loads at a time with one row; `advance`: this thread also advances
// r's counters.
template <int CH>
__device__ __forceinline__ void ema_blocks(const EmaArgs& A, int r, int k0, int k1, bool advance) {
  const int rows = A.rows, max_blocks = A.max_blocks;
  const int32_t* n_valid = A.n_valid;
  const float* z = A.z;
  const int64_t z_ld = A.z_ld, v_ld = A.v_ld, d_ld = A.d_ld;
  const int32_t* sel = A.sel;
  float* V = A.V;
  float* D = A.D;
  const int lane = threadIdx.x & 63;
  const int N = A.ctx[r], q = A.qpos[r];
  if (advance) {
    if (A.qpos_out) A.qpos_out[r] = q + (n_valid ? n_valid[r] : rows);
    if (A.step_out) A.step_out[r] += 1;
  }
  const float alpha = A.alpha;
  const int32_t* n_sel = A.n_sel;
  if (request_error(N, q, rows, max_blocks, v_ld, d_ld)) return;
  const int ns = clamp_nsel(n_sel[r], max_blocks);
  k1 = min(k1, ns);
  if (k0 >= k1) return;
  int L = A.row0_only ? 1 : (n_valid ? n_valid[r] : rows);
  L = L < 0 ? 0 : (L > rows ? rows : L);
  if (L == 0) return;
  const int32_t* sr = sel + (int64_t)r * max_blocks;
  const float a = alpha, b = __fsub_rn(1.0f, alpha);
  const float* zb = z + (int64_t)r * rows * z_ld;
  float* Vr = V + (int64_t)r * v_ld;
  float* Dr = D + (int64_t)r * d_ld;
  if (L == 1) {
    // one observation per slot: V[i] and D[q - i] from row 0, CH blocks'
    // loads at a time, two chunks in flight: chunk c + 1's loads go out
    // before chunk c's stores, so a wave's writes overlap its next reads
    // (different blocks touch disjoint V and D elements)
    struct Chunk {
      float vv[CH], dd[CH], zz[CH];
      int ii[CH], jj[CH];
    };
    const auto load = [&](Chunk& C, int kb) {
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int k = kb + u;
        const int j = k < k1 ? __builtin_amdgcn_readfirstlane(sr[k]) : -1;  // uniform
        const int i = j * 64 + lane;
        const bool ok = k < k1 && j >= 0 && j < max_blocks && i < N;
        C.jj[u] = k < k1 && j >= 0 && j < max_blocks ? j : -1;
        C.ii[u] = ok ? i : -1;
        C.vv[u] = ok ? Vr[i] : 0.0f;
        C.dd[u] = ok ? Dr[q - i] : 0.0f;
        C.zz[u] = ok ? zb[(int64_t)k * 64 + lane] : 0.0f;
      }
    };
    const auto finish = [&](const Chunk& C) {
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const float vn = ema_step(C.vv[u], C.zz[u], a, b);
        if (C.ii[u] >= 0) {
          Vr[C.ii[u]] = vn;
          Dr[q - C.ii[u]] = ema_step(C.dd[u], C.zz[u], a, b);
        }
        // (the block id from before the stores: sel may alias V or D for all
        // the compiler knows, and a reload would wait for them)
        if (A.vmax && C.jj[u] >= 0) ema_vmax(A, r, C.jj[u], C.ii[u] >= 0, vn);
      }
    };
    Chunk c0, c1;
    load(c0, k0);
    for (int kb = k0; kb < k1; kb += 2 * CH) {
      if (kb + CH < k1) load(c1, kb + CH);
      finish(c0);
      if (kb + CH >= k1) break;
      if (kb + 2 * CH < k1) load(c0, kb + 2 * CH);
      finish(c1);
    }
    return;
  }
  // several rows: kEmaChunkRows blocks at a time, every load of the chunk
  // (V, the rows' z, the D offsets the lanes own and the z values that reach
  // them) issued before any update.  The blocks of a chunk touch disjoint V
  // and D elements, so no load can depend on a store of the same chunk.
  constexpr int CR = kEmaChunkRows;
  // the block ids of 64 of the wave's blocks and of their neighbours in the
  // list, one lane each, loaded ahead of the chunks that use them
  int lb = k0, s_cur = -1, s_next = -1, s_prev = -1;
  const auto load_ids = [&](int base) {
    lb = base;
    const int k = base + lane;
    s_cur = k < k1 ? sr[k] : -1;
    s_next = k + 1 < ns ? sr[k + 1] : -1;
    s_prev = k > 0 && k - 1 < ns ? sr[k - 1] : -1;
  };
  load_ids(k0);
  for (int kb = k0; kb < k1; kb += CR) {
    if (kb + CR - 1 - lb >= 64) load_ids(kb);
    int jj[CR], kn[CR];
    bool pe[CR];
    float vV[CR], zV[CR][SPIN_MAX_ROWS];
    float dM[CR], zM[CR][SPIN_MAX_ROWS];
    float dE[CR], zE[CR][SPIN_MAX_ROWS];
    uint32_t mM[CR], mE[CR];  // bit row: that row updates the offset
#pragma unroll
    for (int u = 0; u < CR; ++u) {
      const int k = kb + u;
      const int j = k < k1 ? __builtin_amdgcn_readlane(s_cur, k - lb) : -1;  // uniform
      jj[u] = (j >= 0 && j < max_blocks) ? j : -1;
      // block j + 1 selected (rows past the block's end land there) and
      // block j - 1 not selected (this block then owns the offsets of the up
      // to L - 1 slots left of it)
      const bool next_sel =
          jj[u] >= 0 && k + 1 < ns && __builtin_amdgcn_readlane(s_next, k - lb) == j + 1;
      pe[u] = jj[u] >= 0 && !(k > 0 && __builtin_amdgcn_readlane(s_prev, k - lb) == j - 1) &&
              lane < L - 1;
      kn[u] = next_sel ? k + 1 : -1;
      const int i = j * 64 + lane;
      vV[u] = 0.0f;
      dM[u] = 0.0f;
      dE[u] = 0.0f;
      mM[u] = 0u;
      mE[u] = 0u;
#pragma unroll
      for (int row = 0; row < SPIN_MAX_ROWS; ++row) {
        zV[u][row] = 0.0f;
        zM[u][row] = 0.0f;
        zE[u][row] = 0.0f;
      }
      if (jj[u] < 0) continue;
      if (i < N) {
        vV[u] = Vr[i];
        dM[u] = Dr[q - i];
      }
#pragma unroll
      for (int row = 0; row < SPIN_MAX_ROWS; ++row) {
        if (row >= L) break;
        if (i < N) zV[u][row] = zb[row * z_ld + (int64_t)k * 64 + lane];
        // offset q - i, row `row`: slot i + row, in block j or (if selected) j + 1
        const int sm = i + row;
        if (i < N && sm < N) {
          const int kk = (sm >> 6) == j ? k : kn[u];
          if (kk >= 0) {
            zM[u][row] = zb[row * z_ld + (int64_t)kk * 64 + (sm & 63)];
            mM[u] |= 1u << row;
          }
        }
        // extension offset q - s0, s0 = 64 j - 1 - lane: slot s0 + row in block j
        const int se = j * 64 - 1 - lane + row;
        if (pe[u] && se >= j * 64 && se < N) {
          zE[u][row] = zb[row * z_ld + (int64_t)k * 64 + (se & 63)];
          mE[u] |= 1u << row;
        }
      }
      if (mE[u]) dE[u] = Dr[q - (j * 64 - 1 - lane)];
    }
#pragma unroll
    for (int u = 0; u < CR; ++u) {
      if (jj[u] < 0) continue;
      const int i = jj[u] * 64 + lane;
      float v = vV[u], d = dM[u], de = dE[u];
#pragma unroll
      for (int row = 0; row < SPIN_MAX_ROWS; ++row) {
        if (row >= L) break;
        v = ema_step(v, zV[u][row], a, b);
        if (mM[u] >> row & 1u) d = ema_step(d, zM[u][row], a, b);
        if (mE[u] >> row & 1u) de = ema_step(de, zE[u][row], a, b);
      }
      if (i < N) {
        Vr[i] = v;
        Dr[q - i] = d;
      }
      if (mE[u]) Dr[q - (jj[u] * 64 - 1 - lane)] = de;
      if (A.vmax) ema_vmax(A, r, jj[u], i < N, v);
    }
  }
}

// One wave: selected blocks k0 .. k0 + kEmaBlocksPerWave - 1 of request r.
__device__ __forceinline__ void ema_wave(const EmaArgs& A, int r, int k0, bool advance) {
  ema_blocks<kEmaBlocksPerWave>(A, r, k0, k0 + kEmaBlocksPerWave, advance);
}

}  // namespace spin
