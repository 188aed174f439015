// Per-layer block budgets: the miss curve of a dense probe step, the
// device-side budget table, and the host allocation between layers.
//
// Source: the project blog "Sparse Attention Still Has a Dense Problem",
// section "Per-layer block budgets" (miss rate = share of the dense
// indexer's top-K slots in skipped blocks; a dense probe step every P steps
// measures each layer's miss rate at each budget; budgets sized per layer at
// a fixed total, minimising the worst layer's miss rate; a device-side
// budget table), and the paper's Algorithm 1 (block budget, forced blocks,
// ranked blocks) with Sec. 3.2.1 (exploration share).
#include <algorithm>
#include <cmath>
#include <vector>

#include "spin_dev.h"
#include "spin_launch.h"

namespace spin {

// Blocks kept at budget level g of `levels`: the selection's budget rule at
// target sparsity 10000 - (10000 / levels) g basis points.
__host__ __device__ inline int level_budget(int B, int K, int g, int levels) {
  const int sp = 10000 - (10000 / levels) * g;
  const int kb = (K + SPIN_BLOCK - 1) / SPIN_BLOCK;
  const int keep = (int)(((int64_t)(10000 - sp) * B + 9999) / 10000);
  return min(B, max(kb, keep));
}

constexpr int kMissThreads = 1024;

// ---------------------------------------------------------------------------
// Miss curve of one (request, row) of a dense probe step.  covered[g] = the
// number of top-K slots that lie in the blocks the selection keeps without
// exploration at level g: the forced blocks {0, B-1} and the first
// n_r(g) = m_g - n_f - n_e(m_g) non-forced blocks in the order (S desc,
// lower block first).  The order comes from a bitonic sort of
// (order-preserving key of S, complement of the block id) in LDS, NPAD
// entries (a power of two >= B); forced and absent blocks sort last.
// ---------------------------------------------------------------------------
template <int NPAD>
__global__ __launch_bounds__(kMissThreads) void k_miss_curve(
    int K, int explore_bp, int rows, int max_blocks, int levels, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ qpos, const float* __restrict__ S,
    const int32_t* __restrict__ topk, int32_t* __restrict__ covered,
    int32_t* __restrict__ kprime) {
  __shared__ uint64_t ord[NPAD];
  __shared__ int cnt[NPAD];
  __shared__ int sh[32];
  const int row = blockIdx.x, r = blockIdx.y;
  const int64_t rr = (int64_t)r * rows + row;
  const int N = ctx[r];
  const bool bad = request_error(N, qpos[r], rows, max_blocks, 0, 0) != 0;
  const int B = bad ? 0 : (N + SPIN_BLOCK - 1) / SPIN_BLOCK;
  const float* Srow = S + rr * max_blocks;
  for (int j = threadIdx.x; j < NPAD; j += kMissThreads) {
    cnt[j] = 0;
    uint64_t key = 0;  // forced or absent: last
    if (j < B && j != 0 && j != B - 1)
      key = ((uint64_t)float_key(Srow[j]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
    ord[j] = key;
  }
  __syncthreads();
  // top-K slots per block
  const int32_t* trow = topk + rr * K;
  int mine = 0;
  for (int k = threadIdx.x; k < K; k += kMissThreads) {
    const int i = trow[k];
    if (i >= 0 && i < SPIN_BLOCK * B) {
      atomicAdd(&cnt[i / SPIN_BLOCK], 1);
      ++mine;
    }
  }
  const int kp = block_sum_i32<kMissThreads>(mine, sh);  // barrier inside
  // bitonic sort, descending
  for (int size = 2; size <= NPAD; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < NPAD / 2; t += kMissThreads) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t a = ord[lo], b = ord[hi];
        if ((a < b) == desc) {
          ord[lo] = b;
          ord[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  // prefix of the per-block counts in rank order: EPT positions per thread
  constexpr int EPT = (NPAD + kMissThreads - 1) / kMissThreads;
  const int p0 = threadIdx.x * EPT;
  int part = 0;
  int vals[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int p = p0 + e;
    int v = 0;
    if (p < NPAD && ord[p] != 0)
      v = cnt[(int)(0xFFFFFFFFu - (uint32_t)(ord[p] & 0xFFFFFFFFu))];
    vals[e] = v;
    part += v;
  }
  int tot;
  const int base = block_excl_scan<kMissThreads>(part, sh, &tot);
  __syncthreads();
  // inclusive prefix of rank positions reuses the key array (as ints)
  int* pre = reinterpret_cast<int*>(ord);
  {
    int run = base;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      run += vals[e];
      if (p0 + e < NPAD) pre[p0 + e] = run;
    }
  }
  const int c_forced = B > 0 ? cnt[0] + (B > 1 ? cnt[B - 1] : 0) : 0;
  __syncthreads();
  int32_t* crow = covered + rr * (levels + 1);
  for (int g = threadIdx.x; g <= levels; g += kMissThreads) {
    int cov = 0;
    if (B > 0) {
      const int n_f = B > 1 ? 2 : 1;
      const int m = max(level_budget(B, K, g, levels), n_f);
      const int n_e = min((int)((int64_t)m * explore_bp / 10000), m - n_f);
      const int n_r = m - n_f - n_e;
      cov = c_forced + (n_r > 0 ? pre[n_r - 1] : 0);
    }
    crow[g] = cov;
  }
  if (threadIdx.x == 0) kprime[rr] = kp;
}

// budget[r] = blocks kept at the level in level_table[0] (device-side table)
__global__ void k_budget_fill(int R, int K, int max_blocks, int levels,
                              const int32_t* __restrict__ ctx,
                              const int32_t* __restrict__ level_table,
                              int32_t* __restrict__ budget) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const int N = ctx[r];
  const int g = min(max(level_table[0], 0), levels);
  const int B = (N < 1 || N > SPIN_BLOCK * max_blocks) ? 1 : (N + SPIN_BLOCK - 1) / SPIN_BLOCK;
  budget[r] = level_budget(B, K, g, levels);
}

template <int NPAD>
static void miss_t(const spin_config& c, const spin_batch& b, const float* S,
                   const int32_t* topk, int levels, int32_t* covered, int32_t* kprime,
                   hipStream_t st) {
  hipLaunchKernelGGL(k_miss_curve<NPAD>, dim3(b.n_rows, b.batch), dim3(kMissThreads), 0, st,
                     c.topk, c.explore_bp, b.n_rows, b.max_blocks, levels, b.ctx_len, b.q_pos, S,
                     topk, covered, kprime);
}

hipError_t launch_miss_curve(const spin_config& c, const spin_batch& b, const float* S,
                             const int32_t* topk, int levels, int32_t* covered, int32_t* kprime,
                             hipStream_t st) {
  if (b.max_blocks <= 2048) miss_t<2048>(c, b, S, topk, levels, covered, kprime, st);
  else if (b.max_blocks <= 4096) miss_t<4096>(c, b, S, topk, levels, covered, kprime, st);
  else miss_t<8192>(c, b, S, topk, levels, covered, kprime, st);
  return hipGetLastError();
}

hipError_t launch_budget_fill(const spin_config& c, const spin_batch& b, const int32_t* level,
                              int levels, int32_t* budget, hipStream_t st) {
  hipLaunchKernelGGL(k_budget_fill, dim3((b.batch + 255) / 256), dim3(256), 0, st, b.batch,
                     c.topk, b.max_blocks, levels, b.ctx_len, level, budget);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The allocation on the device, after a probe step (one workgroup): sum each
// layer's curves over its requests and rows, update the running miss rates
// (proportional rule), re-size the layers' levels into the level table.  The
// same arithmetic as the host allocation below, so both give the same levels.
// With a drift threshold the new levels are published only when some
// layer's miss rate at some level moved by more than drift_bp / 10000 since
// the curves of the last publication (the first probe always publishes); the
// running miss rates advance at every probe.
// State (caller-owned, budget_state_bytes()): f64 miss sums [L], f64 probe
// count, i64 curve sums [L][levels + 1], i64 valid top-K totals [L], f64 miss
// rates of the last publication [L][levels + 1], f64 flag "published once".
// ---------------------------------------------------------------------------
struct BudgetState {
  double* miss_sum;
  double* n_probes;
  int64_t* cov;
  int64_t* tot;
  double* ref;
  double* has_ref;
};

__host__ __device__ inline BudgetState budget_state(void* p, int L, int levels) {
  char* b = static_cast<char*>(p);
  BudgetState s;
  s.miss_sum = reinterpret_cast<double*>(b);
  s.n_probes = s.miss_sum + L;
  s.cov = reinterpret_cast<int64_t*>(s.n_probes + 1);
  s.tot = s.cov + (int64_t)L * (levels + 1);
  s.ref = reinterpret_cast<double*>(s.tot + L);
  s.has_ref = s.ref + (int64_t)L * (levels + 1);
  return s;
}

size_t budget_state_bytes(int L, int levels) {
  const size_t W = (size_t)levels + 1;
  const size_t n = 8 * ((size_t)L + 1 + (size_t)L * W + (size_t)L + (size_t)L * W + 1);
  return (n + 255) & ~size_t(255);
}

// Layer l's miss rate at level g from the summed curves (binary64).
__device__ __forceinline__ double state_miss(const BudgetState& st, int W, int i) {
  const int64_t t = st.tot[i / W], c = st.cov[i];
  return t == 0 ? 0.0 : (double)(t - c) / (double)t;
}

// lane-held (miss numerator, denominator, layer) candidates; the wave's
// largest miss rate, ties to the lower layer, exactly (products < 2^63)
__device__ __forceinline__ bool cand_better(int64_t na, int64_t da, int la, int64_t nb, int64_t db,
                                            int lb) {
  if (la < 0) return false;
  if (lb < 0) return true;
  const int64_t x = na * db, y = nb * da;
  return x > y || (x == y && la < lb);
}

__device__ __forceinline__ int64_t shfl_xor_i64(int64_t v, int m) {
  const int lo = __shfl_xor((int)(uint32_t)v, m), hi = __shfl_xor((int)(v >> 32), m);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

constexpr int kBudgetLanes = 64;
constexpr int kBudgetMaxPerLane = (SPIN_MAX_LAYERS + kBudgetLanes - 1) / kBudgetLanes;

__global__ __launch_bounds__(256) void k_budget_update(int policy, int L, int levels, int target,
                                                       int drift_bp, int RR,
                                                       const int32_t* __restrict__ cov,
                                                       const int32_t* __restrict__ kp,
                                                       void* state, int32_t* level_table) {
  const BudgetState st = budget_state(state, L, levels);
  const int W = levels + 1;
  for (int i = threadIdx.x; i < L * W; i += blockDim.x) {
    const int l = i / W, g = i % W;
    int64_t s = 0;
    for (int k = 0; k < RR; ++k) s += cov[((int64_t)l * RR + k) * W + g];
    st.cov[i] = s;
  }
  for (int l = threadIdx.x; l < L; l += blockDim.x) {
    int64_t s = 0;
    for (int k = 0; k < RR; ++k) s += kp[(int64_t)l * RR + k];
    st.tot[l] = s;
  }
  __syncthreads();
  // the drift since the last publication: the largest change of any miss rate
  __shared__ double wave_drift[256 / 64];
  __shared__ int publish_s;
  const bool gate = drift_bp > 0 && *st.has_ref != 0.0;
  if (gate) {
    double d = 0.0;
    for (int i = threadIdx.x; i < L * W; i += blockDim.x)
      d = fmax(d, fabs(state_miss(st, W, i) - st.ref[i]));
    for (int m = 32; m > 0; m >>= 1) d = fmax(d, __shfl_xor(d, m));
    if ((threadIdx.x & 63) == 0) wave_drift[threadIdx.x >> 6] = d;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double d = 0.0;
    if (gate)
      for (int w = 0; w < (int)(blockDim.x >> 6); ++w) d = fmax(d, wave_drift[w]);
    publish_s = !gate || d > (double)drift_bp / 10000.0;
  }
  __syncthreads();
  const bool publish = publish_s != 0;
  if (publish) {  // these curves become the reference (read above, before the barrier)
    for (int i = threadIdx.x; i < L * W; i += blockDim.x) st.ref[i] = state_miss(st, W, i);
    if (threadIdx.x == 0) *st.has_ref = 1.0;
  }
  if (threadIdx.x >= kBudgetLanes) return;
  const int lane = threadIdx.x;
  if (policy == SPIN_BUDGET_MINIMAX) {
    if (!publish) return;
    // raise the layer of the largest miss rate by one level, from all zero
    int g[kBudgetMaxPerLane];
#pragma unroll
    for (int u = 0; u < kBudgetMaxPerLane; ++u) g[u] = 0;
    const int64_t budget = (int64_t)L * target;
    for (int64_t it = 0; it < budget; ++it) {
      int64_t bn = 0, bd = 1;
      int bl = -1;
#pragma unroll
      for (int u = 0; u < kBudgetMaxPerLane; ++u) {
        const int l = lane + kBudgetLanes * u;
        if (l >= L || g[u] >= levels) continue;
        const int64_t t = st.tot[l], c = st.cov[(int64_t)l * W + g[u]];
        const int64_t n = t == 0 ? 0 : t - c, d = t == 0 ? 1 : t;
        if (cand_better(n, d, l, bn, bd, bl)) {
          bn = n;
          bd = d;
          bl = l;
        }
      }
#pragma unroll
      for (int m = 1; m < kBudgetLanes; m <<= 1) {
        const int64_t on = shfl_xor_i64(bn, m), od = shfl_xor_i64(bd, m);
        const int ol = __shfl_xor(bl, m);
        if (cand_better(on, od, ol, bn, bd, bl)) {
          bn = on;
          bd = od;
          bl = ol;
        }
      }
      if (bl < 0) break;  // every layer at the top level
      if (bl % kBudgetLanes == lane) g[bl / kBudgetLanes] += 1;
    }
#pragma unroll
    for (int u = 0; u < kBudgetMaxPerLane; ++u) {
      const int l = lane + kBudgetLanes * u;
      if (l < L) level_table[l] = g[u];
    }
    return;
  }
  // proportional (lane 0): the running mean of each layer's miss rate at the
  // level it ran at, then shares of L * target in proportion to miss + 1e-3
  __shared__ double w[SPIN_MAX_LAYERS], share[SPIN_MAX_LAYERS];
  __shared__ int fixed[SPIN_MAX_LAYERS], gl[SPIN_MAX_LAYERS];
  __shared__ bool used[SPIN_MAX_LAYERS];
  if (lane != 0) return;
  const double np = *st.n_probes + 1.0;
  *st.n_probes = np;
  for (int l = 0; l < L; ++l) {
    const int64_t t = st.tot[l], c = st.cov[(int64_t)l * W + level_table[l]];
    st.miss_sum[l] += t == 0 ? 0.0 : (double)(t - c) / (double)t;
    w[l] = st.miss_sum[l] / np + 1e-3;
    fixed[l] = -1;
    share[l] = 0.0;
  }
  if (!publish) return;
  const int64_t T = (int64_t)L * target;
  for (;;) {
    int64_t rem = T;
    double ws = 0.0;
    for (int l = 0; l < L; ++l) {
      if (fixed[l] >= 0) rem -= fixed[l];
      else ws += w[l];
    }
    bool changed = false;
    for (int l = 0; l < L; ++l)
      if (fixed[l] < 0) share[l] = (double)rem * w[l] / ws;
    for (int l = 0; l < L; ++l) {
      if (fixed[l] >= 0) continue;
      if (share[l] > levels) { fixed[l] = levels; changed = true; }
      else if (share[l] < 0) { fixed[l] = 0; changed = true; }
    }
    if (!changed) break;
  }
  int64_t sum = 0;
  for (int l = 0; l < L; ++l) {
    gl[l] = fixed[l] >= 0 ? fixed[l] : (int)floor(share[l]);
    sum += gl[l];
  }
  // one more level to the largest fractional parts (ties: lower layer), in
  // that order, skipping layers at the top
  int64_t left = T - sum;
  for (int l = 0; l < L; ++l) used[l] = fixed[l] >= 0;
  while (left > 0) {
    int best = -1;
    double bf = 0.0;
    for (int l = 0; l < L; ++l) {
      if (used[l]) continue;
      const double f = share[l] - gl[l];
      if (best < 0 || f > bf) { best = l; bf = f; }
    }
    if (best < 0) break;
    used[best] = true;
    if (gl[best] < levels) { ++gl[best]; --left; }
  }
  for (int l = 0; l < L; ++l) level_table[l] = gl[l];
}

hipError_t launch_budget_update(int policy, int L, int levels, int target, int drift_bp, int RR,
                                const int32_t* covered, const int32_t* kprime, void* state,
                                int32_t* level_table, hipStream_t st) {
  hipLaunchKernelGGL(k_budget_update, dim3(1), dim3(256), 0, st, policy, L, levels, target,
                     drift_bp, RR, covered, kprime, state, level_table);
  return hipGetLastError();
}

// Start of a policy: every layer at the target level, no probe history,
// the probe budget (every block) in place.
__global__ void k_budget_reset(int L, int levels, int target, int R, void* state,
                               int32_t* level_table, int32_t* probe_budget) {
  const BudgetState st = budget_state(state, L, levels);
  for (int i = threadIdx.x; i < L; i += blockDim.x) {
    level_table[i] = target;
    st.miss_sum[i] = 0.0;
  }
  for (int i = threadIdx.x; i < R; i += blockDim.x) probe_budget[i] = SPIN_MAX_BLOCKS;
  if (threadIdx.x == 0) {
    *st.n_probes = 0.0;
    *st.has_ref = 0.0;
  }
}

hipError_t launch_budget_reset(int L, int levels, int target, int R, void* state,
                               int32_t* level_table, int32_t* probe_budget, hipStream_t st) {
  hipLaunchKernelGGL(k_budget_reset, dim3(1), dim3(256), 0, st, L, levels, target, R, state,
                     level_table, probe_budget);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host allocation between layers (no device work).
// ---------------------------------------------------------------------------
namespace {

// miss_a > miss_b for miss = (t - c) / t (0 when t == 0), exactly
bool miss_greater(int64_t ca, int64_t ta, int64_t cb, int64_t tb) {
  const int64_t na = ta == 0 ? 0 : ta - ca, da = ta == 0 ? 1 : ta;
  const int64_t nb = tb == 0 ? 0 : tb - cb, db = tb == 0 ? 1 : tb;
  return (__int128)na * db > (__int128)nb * da;
}

}  // namespace

void allocate_minimax(int L, int levels, int target, const int64_t* covered,
                      const int64_t* total, int32_t* out) {
  std::vector<int> g(L, 0);
  const int64_t budget = (int64_t)L * target;
  int64_t sum = 0;
  while (sum < budget) {
    int best = -1;
    for (int l = 0; l < L; ++l) {
      if (g[l] >= levels) continue;
      const int64_t* cl = covered + (int64_t)l * (levels + 1);
      if (best < 0) {
        best = l;
        continue;
      }
      const int64_t* cb = covered + (int64_t)best * (levels + 1);
      if (miss_greater(cl[g[l]], total[l], cb[g[best]], total[best])) best = l;
    }
    if (best < 0) break;
    ++g[best];
    ++sum;
  }
  for (int l = 0; l < L; ++l) out[l] = g[l];
}

void allocate_proportional(int L, int levels, int target, const double* miss, int32_t* out) {
  const int64_t T = (int64_t)L * target;
  std::vector<double> w(L), share(L, 0.0);
  std::vector<int> fixed(L, -1);
  for (int l = 0; l < L; ++l) w[l] = miss[l] + 1e-3;
  for (;;) {
    int64_t rem = T;
    double ws = 0.0;
    for (int l = 0; l < L; ++l) {
      if (fixed[l] >= 0) rem -= fixed[l];
      else ws += w[l];
    }
    bool changed = false;
    for (int l = 0; l < L; ++l) {
      if (fixed[l] >= 0) continue;
      share[l] = (double)rem * w[l] / ws;
    }
    for (int l = 0; l < L; ++l) {
      if (fixed[l] >= 0) continue;
      if (share[l] > levels) { fixed[l] = levels; changed = true; }
      else if (share[l] < 0) { fixed[l] = 0; changed = true; }
    }
    if (!changed) break;
  }
  std::vector<int> g(L);
  std::vector<std::pair<double, int>> frac;
  int64_t sum = 0;
  for (int l = 0; l < L; ++l) {
    if (fixed[l] >= 0) g[l] = fixed[l];
    else {
      g[l] = (int)std::floor(share[l]);
      frac.push_back({share[l] - g[l], l});
    }
    sum += g[l];
  }
  std::stable_sort(frac.begin(), frac.end(), [](const std::pair<double, int>& a,
                                               const std::pair<double, int>& b) {
    return a.first > b.first || (a.first == b.first && a.second < b.second);
  });
  int64_t left = T - sum;
  for (const auto& f : frac) {
    if (left <= 0) break;
    if (g[f.second] < levels) {
      ++g[f.second];
      --left;
    }
  }
  for (int l = 0; l < L; ++l) out[l] = g[l];
}

}  // namespace spin
