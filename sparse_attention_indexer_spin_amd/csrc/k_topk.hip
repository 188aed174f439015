// Stage 3b of the SPIN decode step: the post-indexer top-K over the scored
// slots ("SPIN: Shadow Predictive Indexer for Sparse Attention", Algorithm 1
// step 7; Sec. 2 gives K between 512 and 2048 in practice).
//
// One 1024-thread workgroup per (request, verifier row).  Scores are mapped to
// order-preserving u32 keys and the K-th largest is found by radix select in
// 8-bit digits, starting below the common prefix of the row's max and min so
// the first histogram spreads well.  Ties at the threshold go to the lower
// slot; the selected slots are written in ascending slot order (the compact
// score layout is already in ascending slot order), padded with -1.
#include "spin_dev.h"
#include "spin_launch.h"

namespace spin {

constexpr int kTopThreads = 1024;
constexpr int kTopEPT = 8;
constexpr int kTopChunk = kTopThreads * kTopEPT;

struct TopkRow {
  const float* z;
  const int32_t* sel;
  int n;  // candidates (64 per selected block)
  int N;  // context length
};

// Load this thread's 8 consecutive candidates of chunk `cb`; returns a valid mask.
__device__ __forceinline__ uint32_t load_keys(const TopkRow& R, int cb, uint32_t (&key)[kTopEPT],
                                              int& slot0) {
  const int c0 = cb + threadIdx.x * kTopEPT;
  slot0 = 0;
  if (c0 >= R.n) return 0u;
  const int blk = R.sel[c0 >> 6];
  slot0 = blk * 64 + (c0 & 63);
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

__global__ __launch_bounds__(kTopThreads) void k_topk(int K, int rows, int max_blocks,
                                                      const int32_t* __restrict__ ctx,
                                                      const int32_t* __restrict__ qpos,
                                                      const float* __restrict__ z, int64_t z_ld,
                                                      const int32_t* __restrict__ sel,
                                                      const int32_t* __restrict__ n_sel,
                                                      int32_t* __restrict__ out) {
  __shared__ int hist[256];
  __shared__ int sh[32];
  __shared__ uint32_t tmpu[16];
  const int row = blockIdx.x, r = blockIdx.y;
  int32_t* orow = out + ((int64_t)r * rows + row) * K;
  const int N = ctx[r];
  const bool bad = request_error(N, qpos[r], rows, max_blocks, 0, 0) != 0;
  TopkRow R{z + ((int64_t)r * rows + row) * z_ld, sel + (int64_t)r * max_blocks,
            bad ? 0 : clamp_nsel(n_sel[r], max_blocks) * 64, N};

  // pass 1: valid count and key range
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
  const int nvalid = block_sum_i32<kTopThreads>(cnt, sh);
  mx = block_max_u32<kTopThreads>(mx, tmpu);
  mn = block_min_u32<kTopThreads>(mn, tmpu);
  const int take = min(K, nvalid);

  // radix select of the take-th largest key (skipped when every valid slot is taken)
  int nb = 0, k = take;
  uint64_t prefix = 0;
  if (take < nvalid && take > 0) {
    nb = (mx == mn) ? 0 : 32 - __clz(mx ^ mn);
    prefix = ((uint64_t)mx >> nb) << nb;
    while (nb > 0) {
      const int db = nb < 8 ? nb : 8, pos = nb - db;
      for (int i = threadIdx.x; i < 256; i += kTopThreads) hist[i] = 0;
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
  const bool take_all = take >= nvalid;
  const uint64_t hp = prefix >> nb;

  // emit in ascending slot order
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
    int eq_rank = eq_before + block_excl_scan<kTopThreads>(__popc(eq), sh, &eq_tot);
    uint32_t chosen = gt;
#pragma unroll
    for (int e = 0; e < kTopEPT; ++e)
      if (eq >> e & 1u) { if (eq_rank < k) chosen |= 1u << e; ++eq_rank; }
    eq_before += eq_tot;
    int tot;
    int pos = written + block_excl_scan<kTopThreads>(__popc(chosen), sh, &tot);
#pragma unroll
    for (int e = 0; e < kTopEPT; ++e)
      if ((chosen >> e & 1u) && pos < K) orow[pos++] = s0 + e;
    written += tot;
  }
  for (int i = written + threadIdx.x; i < K; i += kTopThreads) orow[i] = -1;
}

size_t topk_workspace_bytes(const spin_config&, int, int, int) { return 0; }

hipError_t launch_topk(const spin_config& c, const spin_batch& b, const float* z, int64_t z_ld,
                       const int32_t* sel, const int32_t* n_sel, int32_t* out, void*, size_t,
                       hipStream_t st) {
  hipLaunchKernelGGL(k_topk, dim3(b.n_rows, b.batch), dim3(kTopThreads), 0, st, c.topk, b.n_rows,
                     b.max_blocks, b.ctx_len, b.q_pos, z, z_ld, sel, n_sel, out);
  return hipGetLastError();
}

}  // namespace spin
