// EMA update device code (Algorithm 1 steps 8-10 of "SPIN: Shadow Predictive
// Indexer for Sparse Attention"; deferred in-order replay of Sec. 3.2.2),
// shared by the EMA kernel and the kernel that runs it beside the top-K.
#pragma once
#include "spin_dev.h"
#include "plan_dev.h"

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
    // (different blocks touch disjoint V and D elements).  The block ids
    // come one per lane from one load per 64 blocks, and every load is
    // unconditional (lanes without an element read element 0): a block id
    // moved to a scalar right after its load, or loads under branches, made
    // the compiler wait for every outstanding load, the other chunk's too.
    struct Chunk {
      float vv[CH], dd[CH], zz[CH];
      int ii[CH], jj[CH];
    };
    int sg = k0, s1 = k1, ids = -1;
    const auto load = [&](Chunk& C, int kb) {
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int k = kb + u;
        const int j = k < s1 ? __builtin_amdgcn_readlane(ids, k - sg) : -1;  // uniform
        const int i = j * 64 + lane;
        const bool ok = k < s1 && j >= 0 && j < max_blocks && i < N;
        C.jj[u] = k < s1 && j >= 0 && j < max_blocks ? j : -1;
        C.ii[u] = ok ? i : -1;
        const float vx = Vr[ok ? i : 0], dx = Dr[ok ? q - i : 0];
        const float zx = zb[ok ? (int64_t)k * 64 + lane : 0];
        C.vv[u] = ok ? vx : 0.0f;
        C.dd[u] = ok ? dx : 0.0f;
        C.zz[u] = ok ? zx : 0.0f;
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
    for (; sg < k1; sg += 64) {
      s1 = min(k1, sg + 64);
      {
        const int kk = sg + lane;
        const int idx = sr[kk < s1 ? kk : sg];
        ids = kk < s1 ? idx : -1;
      }
      Chunk c0, c1;
      load(c0, sg);
      for (int kb = sg; kb < s1; kb += 2 * CH) {
        if (kb + CH < s1) load(c1, kb + CH);
        finish(c0);
        if (kb + CH >= s1) break;
        if (kb + 2 * CH < s1) load(c0, kb + 2 * CH);
        finish(c1);
      }
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
      // every load unconditional, lanes without an element reading element
      // 0 of the same array (rows past L read row 0): loads under branches
      // made the compiler wait for all outstanding loads where they joined
      const bool on = jj[u] >= 0, in = on && i < N;
      const float vx = Vr[in ? i : 0], dx = Dr[in ? q - i : 0];
      vV[u] = in ? vx : 0.0f;
      dM[u] = in ? dx : 0.0f;
      mM[u] = 0u;
      mE[u] = 0u;
#pragma unroll
      for (int row = 0; row < SPIN_MAX_ROWS; ++row) {
        const bool rw = row < L;
        const int64_t ro = (int64_t)(rw ? row : 0) * z_ld;
        const float zv = zb[ro + (rw && in ? (int64_t)k * 64 + lane : 0)];
        zV[u][row] = rw && in ? zv : 0.0f;
        // offset q - i, row `row`: slot i + row, in block j or (if selected) j + 1
        const int sm = i + row;
        const int kk = (sm >> 6) == j ? k : kn[u];
        const bool mm = rw && in && sm < N && kk >= 0;
        const float zm = zb[ro + (mm ? (int64_t)kk * 64 + (sm & 63) : 0)];
        zM[u][row] = mm ? zm : 0.0f;
        mM[u] |= mm ? 1u << row : 0u;
        // extension offset q - s0, s0 = 64 j - 1 - lane: slot s0 + row in block j
        const int se = j * 64 - 1 - lane + row;
        const bool me = rw && on && pe[u] && se >= j * 64 && se < N;
        const float ze = zb[ro + (me ? (int64_t)k * 64 + (se & 63) : 0)];
        zE[u][row] = me ? ze : 0.0f;
        mE[u] |= me ? 1u << row : 0u;
      }
      const float dex = Dr[mE[u] ? q - (j * 64 - 1 - lane) : 0];
      dE[u] = mE[u] ? dex : 0.0f;
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


// ---------------------------------------------------------------------------
// The EMA update of a whole step fused with the next step's prediction
// (SPIN_PREDICT_AHEAD, block reduction A1, one verifier row): the block scores
// the next step would predict from the updated V and D at its position
// q' = q + A (A = the step's counter advance, 0 or 1), written to S beside a
// tag (step, q', N) that lets that step skip its own prediction.  Work goes
// by block j, selected or not, one wave per block, lane l for slot
// i = 64 j + l:
//  * V[i]: the update where block j is selected (and the row counts);
//  * D at offset q' - i, owned by lane l for i < N + A: its update at this
//    step comes from slot i - A, in block j or (lane 0, A = 1) the last slot
//    of block j - 1.  The owned offsets [q' - N - A + 1, q'] contain every
//    offset the step updates, [q - N + 1, q + L - 1], each once, and the next
//    step's prediction of block j reads exactly block j's, so no wave reads
//    what another writes.  (With several rows the next step's row r would
//    also read r offsets of block j - 1's range, written by another wave:
//    there the flag leaves the EMA as it is and the next step predicts.)
// The predicted scores are those of predict_block_scores on the updated
// state: the same pooling code, on the same fp32 values.
// ---------------------------------------------------------------------------
struct EmaPredArgs {
  EmaArgs e;            // the EMA's (qpos: the step's q positions; rows == 1)
  const int32_t* inv;   // [R][max_blocks]: position of block j in sel, -1 if not selected
  int combine, pooling;
  float* S;             // [R][max_blocks]: the next step's block scores
  int32_t* tag;         // [R][4]: step, q', N the scores are for (-1: none)
};

// Where a whole step's EMA also puts the next step's block scores
// (SPIN_PREDICT_AHEAD): the step's inverse block map, S and the tags.
struct Ahead {
  const int32_t* inv;
  float* S;
  int32_t* tag;
};

inline EmaPredArgs ema_pred_args(const spin_config& c, const EmaArgs& e, const Ahead* a) {
  return EmaPredArgs{e, a ? a->inv : nullptr, c.combine, c.flags & SPIN_POOL_MASK,
                     a ? a->S : nullptr, a ? a->tag : nullptr};
}

// Request r's blocks [w nb / n, (w + 1) nb / n) for worker w of n, nb the
// blocks whose lanes own offsets; `advance`: this thread also advances r's
// counters and writes its tag.  The blocks' positions in sel come from one
// vector load per 63 blocks (lane l: block base + l), and CH blocks' loads
// are issued together, two such chunks in flight: a chunk's loads depend on
// no load of its own, so a wave waits about one memory round per chunk.
template <int CH>
__device__ __forceinline__ void ema_predict_blocks(const EmaPredArgs& P, int r, int w, int n,
                                                   bool advance) {
  const EmaArgs& E = P.e;
  const int lane = threadIdx.x & 63;
  const int max_blocks = E.max_blocks;
  const int N = E.ctx[r], q = E.qpos[r];
  const int adv = E.n_valid ? E.n_valid[r] : 1;
  const int A = adv < 0 ? 0 : (adv > 1 ? 1 : adv);
  const int q1 = q + A;
  const bool bad = request_error(N, q, 1, max_blocks, E.v_ld, E.d_ld) != 0;
  const bool pred = !bad && A == adv && E.step_out &&
                    request_error(N, q1, 1, max_blocks, E.v_ld, E.d_ld) == 0;
  if (advance) {
    int st = 0;
    if (E.qpos_out) E.qpos_out[r] = q + adv;
    if (E.step_out) {
      st = E.step_out[r] + 1;
      E.step_out[r] = st;
    }
    if (P.tag) {
      int32_t* t = P.tag + 4 * (int64_t)r;
      t[0] = pred ? st : -1;
      t[1] = q1;
      t[2] = N;
      t[3] = 0;
    }
  }
  if (bad) return;
  const bool upd = (E.row0_only ? 1 : A) > 0;  // the row counts
  const int B = (N + SPIN_BLOCK - 1) / SPIN_BLOCK;
  const int nb = (N + A + SPIN_BLOCK - 1) / SPIN_BLOCK;
  const int j0 = (int)((int64_t)w * nb / n), j1 = (int)((int64_t)(w + 1) * nb / n);
  if (j0 >= j1) return;
  const float a = E.alpha, b = __fsub_rn(1.0f, E.alpha);
  const float* zb = E.z + (int64_t)r * E.z_ld;
  const int32_t* ir = P.inv + (int64_t)r * max_blocks;
  float* Vr = E.V + (int64_t)r * E.v_ld;
  float* Dr = E.D + (int64_t)r * E.d_ld;
  const int64_t dcap = E.d_ld > 0 ? E.d_ld : INT64_MAX;
  struct Chunk {
    float v[CH], d[CH], zv[CH], zd[CH];
    bool md[CH];
    int kj[CH];
  };
  // lane l of pos: the position of block base + l (-1 past B), base = the
  // segment's first block - 1; the window is fixed within a segment, so the
  // chunk loads below wait for no earlier load
  int base = 0, pos = 0, s1 = j0;
  // Every load is unconditional, lanes without an element reading element 0
  // of the same array: loads under branches made the compiler wait for all
  // outstanding loads where the branches join, the next chunk's too.
  const auto load = [&](Chunk& C, int jc) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int j = jc + u;
      const bool on = j < s1;
      C.kj[u] = on ? __builtin_amdgcn_readlane(pos, j - base) : -1;
      const int kjm = on ? __builtin_amdgcn_readlane(pos, j - 1 - base) : -1;
      const int i = j * SPIN_BLOCK + lane;
      const bool vin = on && i < N;
      const bool zin = upd && C.kj[u] >= 0 && i < N;
      const bool own = on && i < N + A;
      const int64_t o = (int64_t)q1 - i;
      const bool din = own && o < dcap;
      const int s = i - A;  // the slot whose score updates offset q' - i
      const int kk = (s >= 0 && s < N) ? ((s >> 6) == j ? C.kj[u] : kjm) : -1;
      C.md[u] = upd && own && kk >= 0;
      const float vx = Vr[vin ? i : 0];
      const float zx = zb[zin ? (int64_t)C.kj[u] * 64 + lane : 0];
      const float dx = Dr[din ? o : 0];
      const float zy = zb[C.md[u] ? (int64_t)kk * 64 + (s & 63) : 0];
      C.v[u] = vin ? vx : 0.0f;
      C.zv[u] = zin ? zx : 0.0f;
      C.d[u] = din ? dx : 0.0f;
      C.zd[u] = C.md[u] ? zy : 0.0f;
    }
  };
  const auto finish = [&](Chunk& C, int jc) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int j = jc + u;
      if (j >= s1) break;
      const int i = j * SPIN_BLOCK + lane;
      if (upd && C.kj[u] >= 0) {
        C.v[u] = ema_step(C.v[u], C.zv[u], a, b);
        if (i < N) Vr[i] = C.v[u];
        if (E.vmax) ema_vmax(E, r, j, i < N, C.v[u]);
      }
      if (C.md[u]) {
        C.d[u] = ema_step(C.d[u], C.zd[u], a, b);
        Dr[q1 - i] = C.d[u];
      }
      if (!pred || j >= B) continue;
      const float zhat =
          P.combine == SPIN_COMBINE_SUM ? __fadd_rn(C.v[u], C.d[u]) : fmaxf(C.v[u], C.d[u]);
      const float m = P.pooling == SPIN_POOL_MAX
                          ? wave_max_f32(i < N ? zhat : -INFINITY)
                          : pool_block_wave(zhat, i < N, min(SPIN_BLOCK, N - j * SPIN_BLOCK),
                                            P.pooling);
      if (lane == 0) P.S[(int64_t)r * max_blocks + j] = m + 0.0f;
    }
  };
  // segments of up to 63 blocks, each with its window of positions
  for (int sg = j0; sg < j1; sg += 63) {
    s1 = min(j1, sg + 63);
    base = sg - 1;
    {
      const int jj = base + lane;
      const int px = ir[jj >= 0 && jj < B ? jj : 0];
      pos = jj >= 0 && jj < B ? px : -1;
    }
    Chunk c0, c1;
    load(c0, sg);
    for (int jc = sg; jc < s1; jc += 2 * CH) {
      if (jc + CH < s1) load(c1, jc + CH);
      finish(c0, jc);
      if (jc + CH >= s1) break;
      if (jc + 2 * CH < s1) load(c0, jc + 2 * CH);
      finish(c1, jc + CH);
    }
  }
}

}  // namespace spin
