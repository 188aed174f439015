// Stage 3b of the SPIN decode step: the post-indexer top-K over the scored
// slots ("SPIN: Shadow Predictive Indexer for Sparse Attention", Algorithm 1
// step 7; Sec. 2 gives K between 512 and 2048 in practice).
//
// Scores map to order-preserving u32 keys; the result is the min(K, |dom|)
// valid slots with the largest keys (ties: lower slot), written in ascending
// slot order (the compact score layout is already in ascending slot order).
//
// Two kernels per call:
//   1. filter (one workgroup per 4096-slot chunk of a row): keeps the valid
//      slots whose key is >= a per-row threshold hint, compacted in order.
//   2. select (one workgroup per row): if the kept count c satisfies
//      K' <= c <= 8192 (K' = min(K, |dom|)), the exact top-K' is taken among
//      the kept candidates in LDS.  This is exact for ANY hint: an element
//      below the hint is outranked by all c >= K' candidates.  Otherwise the
//      row falls back to a radix select over all of its scores.
// The hint lives in the caller's workspace and is refreshed every call so
// that about 2K candidates pass the next step's filter: scores of a layer are
// strongly correlated from one decode step to the next, the observation the
// method itself rests on.  Its value only affects speed, never results.
#include "ema_dev.h"
#include "spin_dev.h"
#include "spin_launch.h"

namespace spin {

constexpr int kChunk = 4096;              // filter chunk (64 blocks)
constexpr int kFilterThreads = 256;       // 16 candidates per thread
constexpr int kCap = kSelThreads * 8;     // candidates the LDS path takes
constexpr int kTopEPT = 8;                // fallback: candidates per thread per pass
constexpr int kTopChunk = kSelThreads * kTopEPT;

struct TopkWs {
  uint32_t* hint;   // [rows_total]
  int32_t* cnt;     // [rows_total][n_chunks] candidates kept
  int32_t* valid;   // [rows_total][n_chunks] valid slots
  uint2* cand;      // [rows_total][n_cap] (key, slot), chunk c at offset c * kChunk
  int32_t* pcnt;    // [rows_total][max_blocks] kept per block (filter inside the score kernel)
  int n_chunks;
  int64_t n_cap;
};

__host__ __device__ inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

__host__ __device__ inline TopkWs carve(void* ws, int rows_total, int max_blocks) {
  TopkWs w;
  w.n_cap = (int64_t)max_blocks * 64;
  w.n_chunks = (int)((w.n_cap + kChunk - 1) / kChunk);
  char* p = reinterpret_cast<char*>(ws);
  int64_t off = 0;
  w.hint = reinterpret_cast<uint32_t*>(p + off);
  off = align256(off + 4LL * rows_total);
  w.cnt = reinterpret_cast<int32_t*>(p + off);
  off = align256(off + 4LL * rows_total * w.n_chunks);
  w.valid = reinterpret_cast<int32_t*>(p + off);
  off = align256(off + 4LL * rows_total * w.n_chunks);
  w.cand = reinterpret_cast<uint2*>(p + off);
  off = align256(off + 8LL * rows_total * w.n_cap);
  w.pcnt = reinterpret_cast<int32_t*>(p + off);
  return w;
}

static int64_t ws_size(int rows_total, int max_blocks) {
  const int64_t n_cap = (int64_t)max_blocks * 64;
  const int64_t n_chunks = (n_cap + kChunk - 1) / kChunk;
  return align256(4LL * rows_total) + 2 * align256(4LL * rows_total * n_chunks) +
         align256(8LL * rows_total * n_cap) + 4LL * rows_total * max_blocks;
}

__device__ __forceinline__ int row_candidates(int N, int qpos, int rows, int max_blocks,
                                              const int32_t* n_sel, int r) {
  if (request_error(N, qpos, rows, max_blocks, 0, 0)) return 0;
  return clamp_nsel(n_sel[r], max_blocks) * 64;
}

// ---------------------------------------------------------------------------
// 1. filter
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kFilterThreads) void k_topk_filter(
    int rows, int max_blocks, const int32_t* __restrict__ ctx, const int32_t* __restrict__ qpos,
    const float* __restrict__ z, int64_t z_ld, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ n_sel, TopkWs ws) {
  __shared__ int sh[32];
  const int rowid = blockIdx.y, r = rowid / rows, chunk = blockIdx.x;
  const int N = ctx[r];
  const int n = row_candidates(N, qpos[r], rows, max_blocks, n_sel, r);
  const int c0 = chunk * kChunk;
  if (c0 >= n) return;
  const uint32_t tau = ws.hint[rowid];
  const int cb = c0 + threadIdx.x * 16;
  const float* zr = z + (int64_t)rowid * z_ld;
  uint32_t key[16];
  uint32_t pass = 0u, valid = 0u;
  int slot0 = 0;
  if (cb < n) {
    slot0 = sel[(int64_t)r * max_blocks + (cb >> 6)] * 64 + (cb & 63);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float4 x = *reinterpret_cast<const float4*>(zr + cb + 4 * v);
      key[4 * v + 0] = float_key(x.x);
      key[4 * v + 1] = float_key(x.y);
      key[4 * v + 2] = float_key(x.z);
      key[4 * v + 3] = float_key(x.w);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (slot0 + e < N) {
        valid |= 1u << e;
        if (key[e] >= tau) pass |= 1u << e;
      }
    }
  }
  int total;
  int pos = block_excl_scan<kFilterThreads>(__popc(pass), sh, &total);
  uint2* out = ws.cand + (int64_t)rowid * ws.n_cap + c0;
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if (pass >> e & 1u) out[pos++] = make_uint2(key[e], (uint32_t)(slot0 + e));
  const int nvalid = block_sum_i32<kFilterThreads>(__popc(valid), sh);
  if (threadIdx.x == 0) {
    ws.cnt[(int64_t)rowid * ws.n_chunks + chunk] = total;
    ws.valid[(int64_t)rowid * ws.n_chunks + chunk] = nvalid;
  }
}

// ---------------------------------------------------------------------------
// 2. select -- fallback helpers: radix passes over the whole row in global memory
// ---------------------------------------------------------------------------
struct TopkRow {
  const float* z;
  const int32_t* sel;
  int n;  // candidates (64 per selected block)
  int N;  // context length
};

__device__ __forceinline__ uint32_t load_keys(const TopkRow& R, int cb, uint32_t (&key)[kTopEPT],
                                              int& slot0) {
  const int c0 = cb + threadIdx.x * kTopEPT;
  slot0 = 0;
  if (c0 >= R.n) return 0u;
  slot0 = R.sel[c0 >> 6] * 64 + (c0 & 63);
  const float4 a = *reinterpret_cast<const float4*>(R.z + c0);
  const float4 b = *reinterpret_cast<const float4*>(R.z + c0 + 4);
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t valid = 0u;
#pragma unroll
  for (int e = 0; e < kTopEPT; ++e) {
    key[e] = float_key(v[e]);
    if (slot0 + e < R.N) valid |= 1u << e;
  }
  return valid;
}

// Threshold of the k largest valid keys of the row: on return, keys whose top
// (32 - nb) bits exceed prefix's are in, and `k` of those equal to it (lowest
// slots first) are in too.
__device__ void radix_threshold(const TopkRow& R, uint32_t mx, uint32_t mn, int& k, int& nb,
                                uint64_t& prefix, int* hist, int* sh) {
  nb = (mx == mn) ? 0 : 32 - __clz(mx ^ mn);
  prefix = ((uint64_t)mx >> nb) << nb;
  while (nb > 0) {
    const int db = nb < 8 ? nb : 8, pos = nb - db;
    for (int i = threadIdx.x; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int cb = 0; cb < R.n; cb += kTopChunk) {
      uint32_t key[kTopEPT];
      int s0;
      const uint32_t v = load_keys(R, cb, key, s0);
#pragma unroll
      for (int e = 0; e < kTopEPT; ++e)
        if ((v >> e & 1u) && ((uint64_t)key[e] >> nb) == (prefix >> nb))
          atomicAdd(&hist[(key[e] >> pos) & ((1u << db) - 1u)], 1);
    }
    __syncthreads();
    if (threadIdx.x < 64) radix_pick_digit(hist, k, sh);
    __syncthreads();
    const int d = sh[0], bc = sh[2];
    k = sh[1];
    __syncthreads();
    prefix |= (uint64_t)d << pos;
    nb = pos;
    if (bc == k) break;
  }
}

__device__ void fallback_row(const TopkRow& R, int K, int32_t* orow, uint32_t* hint, int* hist,
                             int* sh, uint32_t* tmpu) {
  int cnt = 0;
  uint32_t mx = 0u, mn = 0xFFFFFFFFu;
  for (int cb = 0; cb < R.n; cb += kTopChunk) {
    uint32_t key[kTopEPT];
    int s0;
    const uint32_t v = load_keys(R, cb, key, s0);
    cnt += __popc(v);
#pragma unroll
    for (int e = 0; e < kTopEPT; ++e)
      if (v >> e & 1u) { mx = max(mx, key[e]); mn = min(mn, key[e]); }
  }
  const int nvalid = block_sum_i32<kSelThreads>(cnt, sh);
  mx = block_max_u32<kSelThreads>(mx, tmpu);
  mn = block_min_u32<kSelThreads>(mn, tmpu);
  const int take = min(K, nvalid);
  int nb = 0, k = take;
  uint64_t prefix = 0;
  const bool take_all = take >= nvalid;
  if (!take_all) radix_threshold(R, mx, mn, k, nb, prefix, hist, sh);
  const uint64_t hp = prefix >> nb;
  int written = 0, eq_before = 0;
  for (int cb = 0; cb < R.n; cb += kTopChunk) {
    uint32_t key[kTopEPT];
    int s0;
    const uint32_t v = load_keys(R, cb, key, s0);
    uint32_t gt = 0u, eq = 0u;
#pragma unroll
    for (int e = 0; e < kTopEPT; ++e) {
      if (!(v >> e & 1u)) continue;
      const uint64_t hk = (uint64_t)key[e] >> nb;
      if (take_all || hk > hp) gt |= 1u << e;
      else if (hk == hp) eq |= 1u << e;
    }
    int eq_tot;
    int eq_rank = eq_before + block_excl_scan<kSelThreads>(__popc(eq), sh, &eq_tot);
    uint32_t chosen = gt;
#pragma unroll
    for (int e = 0; e < kTopEPT; ++e)
      if (eq >> e & 1u) { if (eq_rank < k) chosen |= 1u << e; ++eq_rank; }
    eq_before += eq_tot;
    int tot;
    int pos = written + block_excl_scan<kSelThreads>(__popc(chosen), sh, &tot);
#pragma unroll
    for (int e = 0; e < kTopEPT; ++e)
      if ((chosen >> e & 1u) && pos < K) orow[pos++] = s0 + e;
    written += tot;
  }
  for (int i = written + threadIdx.x; i < K; i += kSelThreads) orow[i] = -1;
  // next hint: the key of rank min(|dom|, 2 K') so about 2 K' slots pass the filter
  const int r2 = min(nvalid, 2 * take);
  if (r2 > 0 && r2 < nvalid) {
    int k2 = r2, nb2;
    uint64_t p2;
    radix_threshold(R, mx, mn, k2, nb2, p2, hist, sh);
    if (threadIdx.x == 0) *hint = (uint32_t)p2;  // low bits zero: a slightly lower bound
  } else if (threadIdx.x == 0) {
    *hint = 0u;
  }
}

// ---------------------------------------------------------------------------
// 2. select
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSelThreads) void k_topk_select(
    int K, int rows, int max_blocks, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ qpos, const float* __restrict__ z, int64_t z_ld,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel,
    int32_t* __restrict__ out, TopkWs ws) {
  __shared__ uint32_t lkey[kCap];
  __shared__ int off[kSelThreads / 4 + 1];
  __shared__ int hist[kRadixHist];
  __shared__ int sh[32];
  __shared__ uint32_t tmpu[32];
  const int rowid = blockIdx.x, r = rowid / rows;
  int32_t* orow = out + (int64_t)rowid * K;
  const int N = ctx[r];
  const int n = row_candidates(N, qpos[r], rows, max_blocks, n_sel, r);
  const int nch = (n + kChunk - 1) / kChunk;
  // chunk offsets of the kept candidates, and the valid count
  int c_mine = 0, v_mine = 0;
  for (int i = threadIdx.x; i < nch; i += kSelThreads) {
    c_mine += ws.cnt[(int64_t)rowid * ws.n_chunks + i];
    v_mine += ws.valid[(int64_t)rowid * ws.n_chunks + i];
  }
  // nch <= 128 < kSelThreads: one chunk per thread at most
  int c_tot;
  const int c_off = block_excl_scan<kSelThreads>(c_mine, sh, &c_tot);
  if (threadIdx.x < nch) off[threadIdx.x] = c_off;
  if (threadIdx.x == nch) off[nch] = c_tot;
  const int nvalid = block_sum_i32<kSelThreads>(v_mine, sh);
  const int take = min(K, nvalid);
  __syncthreads();
  if (take == 0) {
    for (int i = threadIdx.x; i < K; i += kSelThreads) orow[i] = -1;
    return;
  }
  if (c_tot < take || c_tot > kCap) {
    TopkRow R{z + (int64_t)rowid * z_ld, sel + (int64_t)r * max_blocks, n, N};
    fallback_row(R, K, orow, ws.hint + rowid, hist, sh, tmpu);
    return;
  }
  // gather the kept keys (ascending slot order) into LDS, all loads in flight
  const uint2* cand = ws.cand + (int64_t)rowid * ws.n_cap;
  for (int p = threadIdx.x; p < c_tot; p += kSelThreads) {
    int lo = 0, hi = nch - 1;  // chunk holding kept candidate p
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= p) lo = mid; else hi = mid - 1;
    }
    lkey[p] = cand[(int64_t)lo * kChunk + (p - off[lo])].x;
  }
  __syncthreads();
  uint32_t key[8];
  uint32_t elig = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int p = threadIdx.x * 8 + e;
    key[e] = p < c_tot ? lkey[p] : 0u;
    if (p < c_tot) elig |= 1u << e;
  }
  const uint32_t chosen = block_select_top<8>(key, elig, take, hist, sh, tmpu);
  int tot;
  int pos = block_excl_scan<kSelThreads>(__popc(chosen), sh, &tot);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (!(chosen >> e & 1u)) continue;
    const int p = threadIdx.x * 8 + e;
    int lo = 0, hi = nch - 1;  // chunk holding kept candidate p
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= p) lo = mid; else hi = mid - 1;
    }
    if (pos < K) orow[pos++] = (int32_t)cand[(int64_t)lo * kChunk + (p - off[lo])].y;
  }
  for (int i = tot + threadIdx.x; i < K; i += kSelThreads) orow[i] = -1;
  // keep the hint while it passes a comfortable number of candidates; raise
  // it to rank 2 K' when too many pass
  if (c_tot > 4 * take) {
    const uint32_t top2 = block_select_top<8>(key, elig, 2 * take, hist, sh, tmpu);
    uint32_t m = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (top2 >> e & 1u) m = min(m, key[e]);
    m = block_min_u32<kSelThreads>(m, tmpu);
    if (threadIdx.x == 0) ws.hint[rowid] = m;
  }
}


// ---------------------------------------------------------------------------
// 2'. select after a score kernel that filtered (CandSink): the candidates of
// selected block k are cand[64 k .. 64 k + pcnt[k]), so concatenating the
// blocks in list order gives them in ascending slot order.
// ---------------------------------------------------------------------------
constexpr int kPagesPerThread = SPIN_MAX_BLOCKS / kSelThreads;

struct PagesShared {
  uint32_t lkey[kCap];
  int32_t lslot[kCap];
  int32_t lsrc[kCap];  // first candidate of each selected block (boff)
  int hist[kRadixHist];
  int sh[32];
  uint32_t tmpu[32];
};

__device__ __forceinline__ void topk_pages_row(int rowid, int K, int rows, int max_blocks,
                               const int32_t* __restrict__ ctx, const int32_t* __restrict__ qpos,
                               const float* __restrict__ z, int64_t z_ld,
                               const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel,
                               int32_t* __restrict__ out, const TopkWs& ws, PagesShared& L) {
  uint32_t* lkey = L.lkey;
  int32_t* lslot = L.lslot;
  int32_t* lsrc = L.lsrc;
  int* hist = L.hist;
  int* sh = L.sh;
  uint32_t* tmpu = L.tmpu;
  const int r = rowid / rows;
  int32_t* orow = out + (int64_t)rowid * K;
  const int N = ctx[r];
  const int n = row_candidates(N, qpos[r], rows, max_blocks, n_sel, r);
  const int ns = n / 64;  // selected blocks
  const int32_t* srow = sel + (int64_t)r * max_blocks;
  // per-block kept counts: thread t owns blocks [t * PPT, t * PPT + PPT)
  constexpr int PPT = kPagesPerThread;
  const int32_t* prow = ws.pcnt + (int64_t)rowid * max_blocks;
  int c[PPT];
  int mine = 0;
#pragma unroll
  for (int e = 0; e < PPT; ++e) {
    const int k = threadIdx.x * PPT + e;
    c[e] = k < ns ? prow[k] : 0;
    mine += c[e];
  }
  // valid slots: every selected block is full except the one holding slot N - 1
  const int nvalid = ns == 0 ? 0 : 64 * ns - max(0, 64 * (srow[ns - 1] + 1) - N);
  const int take = min(K, nvalid);
  if (take == 0) {
    for (int i = threadIdx.x; i < K; i += kSelThreads) orow[i] = -1;
    return;
  }
  int c_tot;
  int off = block_excl_scan<kSelThreads>(mine, sh, &c_tot);
  if (c_tot < take || c_tot > kCap) {
    TopkRow R{z + (int64_t)rowid * z_ld, srow, n, N};
    fallback_row(R, K, orow, ws.hint + rowid, hist, sh, tmpu);
    return;
  }
  // candidate q comes from block k = the last with boff[k] <= q (the
  // candidates of block k sit at cand[64 k ..], a worker's run at its first
  // block), at cand[64 k + q - boff[k]]; the loads of a run are contiguous
  int* boff = lsrc;
#pragma unroll
  for (int e = 0; e < PPT; ++e) {
    const int k = threadIdx.x * PPT + e;
    if (k < ns) boff[k] = off;
    off += c[e];
  }
  __syncthreads();
  const uint2* crow = ws.cand + (int64_t)rowid * ws.n_cap;
  uint2 v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int q = threadIdx.x + e * kSelThreads;
    v[e] = make_uint2(0u, 0u);
    if (q < c_tot) {
      int a = 0, b = ns - 1;
      while (a < b) {
        const int mid = (a + b + 1) >> 1;
        if (boff[mid] <= q) a = mid; else b = mid - 1;
      }
      v[e] = crow[(int64_t)a * 64 + q - boff[a]];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int q = threadIdx.x + e * kSelThreads;
    if (q < c_tot) { lkey[q] = v[e].x; lslot[q] = (int32_t)v[e].y; }
  }
  __syncthreads();
  uint32_t key[8];
  uint32_t elig = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int q = threadIdx.x * 8 + e;
    key[e] = q < c_tot ? lkey[q] : 0u;
    if (q < c_tot) elig |= 1u << e;
  }
  const uint32_t chosen = block_select_top<8>(key, elig, take, hist, sh, tmpu);
  int tot;
  int pos = block_excl_scan<kSelThreads>(__popc(chosen), sh, &tot);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if ((chosen >> e & 1u) && pos < K) orow[pos++] = lslot[threadIdx.x * 8 + e];
  for (int i = tot + threadIdx.x; i < K; i += kSelThreads) orow[i] = -1;
  // keep the hint while it passes a comfortable number of candidates; raise
  // it to rank 2 K' when too many pass
  if (c_tot > 4 * take) {
    const uint32_t top2 = block_select_top<8>(key, elig, 2 * take, hist, sh, tmpu);
    uint32_t m = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (top2 >> e & 1u) m = min(m, key[e]);
    m = block_min_u32<kSelThreads>(m, tmpu);
    if (threadIdx.x == 0) ws.hint[rowid] = m;
  }
}

__global__ __launch_bounds__(kSelThreads) void k_topk_select_pages(
    int K, int rows, int max_blocks, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ qpos, const float* __restrict__ z, int64_t z_ld,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel,
    int32_t* __restrict__ out, TopkWs ws) {
  __shared__ PagesShared L;
  topk_pages_row(blockIdx.x, K, rows, max_blocks, ctx, qpos, z, z_ld, sel, n_sel, out, ws, L);
}

// The top-K of a whole step and its EMA update (+ counter advance) in one
// launch, because neither reads what the other writes: blocks [0, rows_total)
// run the per-row select (dispatched first), the others the EMA, ema_x of
// them per request, sized to fill the CUs the few select workgroups leave
// idle (one workgroup per CU: the select's LDS).
// blocks whose loads an EMA wave issues together (two such chunks are in
// flight; 16 made the 1,024-thread kernel spill)
constexpr int kEmaChunk = 6;
// blocks whose loads a wave of the fused EMA + next-step prediction issues
// together
constexpr int kAheadChunk = 4;

// SEPT > 0: the last `sel_wgs` workgroups select the blocks of another layer
// (one verifier row, SEPT blocks per thread), one request each.
template <int SEPT>
__global__ __launch_bounds__(kSelThreads) void k_topk_ema(
    int K, int rows, int max_blocks, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ qpos, const float* __restrict__ z, int64_t z_ld,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel,
    int32_t* __restrict__ out, TopkWs ws, int rows_total, EmaPredArgs PA, int ema_x,
    SelectArgs sa, SelectInputs si, int sel_wgs) {
  const EmaArgs& A = PA.e;
  __shared__ __align__(16) PagesShared L;
  if constexpr (SEPT > 0) {
    const int s0 = (int)gridDim.x - sel_wgs;
    if ((int)blockIdx.x >= s0) {
      static_assert(sizeof(SelectLds) <= sizeof(PagesShared), "LDS");
      select_request<SEPT>(sa, si, (int)blockIdx.x - s0, *reinterpret_cast<SelectLds*>(&L));
      return;
    }
  }
  if ((int)blockIdx.x < rows_total) {
    topk_pages_row(blockIdx.x, K, rows, max_blocks, ctx, qpos, z, z_ld, sel, n_sel, out, ws, L);
    return;
  }
  // ema_x blocks per request; wave w of the request's team takes an even
  // share of its selected blocks, all of one share's loads issued together
  const int e = blockIdx.x - rows_total, r = e / ema_x, bx = e % ema_x;
  constexpr int kWaves = kSelThreads / 64;
  const int n_waves = ema_x * kWaves, w = bx * kWaves + (int)(threadIdx.x >> 6);
  if (PA.S) {  // SPIN_PREDICT_AHEAD (one row): every block, and the next step's scores
    ema_predict_blocks<kAheadChunk>(PA, r, w, n_waves, w == 0 && threadIdx.x == 0);
    return;
  }
  const int ns = clamp_nsel(A.n_sel[r], A.max_blocks);
  const int k0 = (int)((int64_t)w * ns / n_waves), k1 = (int)((int64_t)(w + 1) * ns / n_waves);
  ema_blocks<kEmaChunk>(A, r, k0, k1, w == 0 && threadIdx.x == 0);
}

size_t topk_workspace_bytes(const spin_config&, int R, int rows, int max_blocks) {
  return (size_t)ws_size(R * rows, max_blocks);
}

size_t step_workspace_bytes(const spin_config& c, int R, int rows, int max_blocks) {
  return (size_t)align256((int64_t)topk_workspace_bytes(c, R, rows, max_blocks)) +
         (size_t)align256(4LL * R) +
         ((c.flags & SPIN_PREDICT_AHEAD) ? (size_t)align256(4LL * R * max_blocks) : 0);
}

template <int SEPT>
static void topk_ema_t(const spin_config& c, const spin_batch& b, const float* z, int64_t z_ld,
                       const int32_t* sel, const int32_t* n_sel, int32_t* out, const TopkWs& ws,
                       const EmaPredArgs& A, const SelectArgs& sa, const SelectInputs& si,
                       int sel_wgs, hipStream_t st, bool ema) {
  const int rows_total = b.batch * b.n_rows;
  constexpr int per_block = (kSelThreads / 64) * kEmaChunk;
  const int most = (b.max_blocks + per_block - 1) / per_block;
  const int resident = resident_workgroups((const void*)k_topk_ema<SEPT>, kSelThreads);
  // With one row the EMA workgroups fill the CUs the selects leave free.  With
  // several rows the selects hold many CUs (a workgroup per request and row)
  // and the EMA has several rows of work per block: it gets workgroups for
  // every CU, and those beyond the free ones start where a select workgroup
  // has finished.
  const int ema_cus = b.n_rows > 1 ? resident - sel_wgs : resident - rows_total - sel_wgs;
  // no EMA workgroups when the update is deferred (the launch is then the
  // top-K and, with SEPT > 0, the next layer's selection)
  const int ema_x = ema ? max(1, min(most, ema_cus / max(1, b.batch))) : 0;
  hipLaunchKernelGGL(k_topk_ema<SEPT>, dim3(rows_total + ema_x * b.batch + sel_wgs),
                     dim3(kSelThreads), 0, st, c.topk, b.n_rows, b.max_blocks, b.ctx_len,
                     A.e.qpos, z, z_ld, sel, n_sel, out, ws, rows_total, A, ema_x, sa, si,
                     sel_wgs);
}

hipError_t launch_topk_ema(const spin_config& c, const spin_batch& b, const float* z,
                           int64_t z_ld, const int32_t* sel, const int32_t* n_sel, int32_t* out,
                           void* wsp, const int32_t* n_valid, float* V, int64_t v_ld, float* D,
                           int64_t d_ld, float* vmax, const int32_t* qpos_snap,
                           int32_t* qpos_out, int32_t* step_out, hipStream_t st,
                           const SelectPlan* next, bool ema, const Ahead* ahead) {
  const int rows_total = b.batch * b.n_rows;
  const TopkWs ws = carve(wsp, rows_total, b.max_blocks);
  const EmaPredArgs A = ema_pred_args(
      c, EmaArgs{c.ema_alpha, b.n_rows, b.max_blocks, b.ctx_len, qpos_snap, n_valid, z, z_ld,
                 sel, n_sel, V, v_ld, D, d_ld, qpos_out, step_out, vmax,
                 (c.flags & SPIN_MTP_ROW0_UPDATE) != 0},
      ahead);
  if (!next) {
    topk_ema_t<0>(c, b, z, z_ld, sel, n_sel, out, ws, A, SelectArgs{}, SelectInputs{}, 0, st,
                  true);
  } else {
    const int n = next->requests;
    switch (next->ept) {
      case 1: topk_ema_t<1>(c, b, z, z_ld, sel, n_sel, out, ws, A, next->args, next->in, n, st, ema); break;
      case 2: topk_ema_t<2>(c, b, z, z_ld, sel, n_sel, out, ws, A, next->args, next->in, n, st, ema); break;
      case 4: topk_ema_t<4>(c, b, z, z_ld, sel, n_sel, out, ws, A, next->args, next->in, n, st, ema); break;
      default: topk_ema_t<8>(c, b, z, z_ld, sel, n_sel, out, ws, A, next->args, next->in, n, st, ema); break;
    }
  }
  return hipGetLastError();
}

CandSink topk_sink(void* wsp, int R, int rows, int max_blocks) {
  const TopkWs ws = carve(wsp, R * rows, max_blocks);
  return CandSink{ws.hint, ws.cand, ws.pcnt, ws.n_cap, max_blocks};
}

hipError_t launch_topk(const spin_config& c, const spin_batch& b, const float* z, int64_t z_ld,
                       const int32_t* sel, const int32_t* n_sel, int32_t* out, void* wsp, size_t,
                       hipStream_t st, bool prefiltered) {
  const int rows_total = b.batch * b.n_rows;
  const TopkWs ws = carve(wsp, rows_total, b.max_blocks);
  if (prefiltered) {
    hipLaunchKernelGGL(k_topk_select_pages, dim3(rows_total), dim3(kSelThreads), 0, st, c.topk,
                       b.n_rows, b.max_blocks, b.ctx_len, b.q_pos, z, z_ld, sel, n_sel, out, ws);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_topk_filter, dim3(ws.n_chunks, rows_total), dim3(kFilterThreads), 0, st,
                     b.n_rows, b.max_blocks, b.ctx_len, b.q_pos, z, z_ld, sel, n_sel, ws);
  hipLaunchKernelGGL(k_topk_select, dim3(rows_total), dim3(kSelThreads), 0, st, c.topk, b.n_rows,
                     b.max_blocks, b.ctx_len, b.q_pos, z, z_ld, sel, n_sel, out, ws);
  return hipGetLastError();
}

}  // namespace spin
