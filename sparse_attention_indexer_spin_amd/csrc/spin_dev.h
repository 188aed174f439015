// Internal device helpers of the SPIN library (gfx950, wave64).  Not part of
// the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spin.h"

namespace spin {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Order-preserving float -> u32 map.  -0 is folded onto +0 first (x + 0.0f is
// +0 for x = -0 under round-to-nearest), so equal floats get equal keys and
// a larger float always gets a larger key.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t float_key(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11): ten rounds of the 4x32 S-box with
// multipliers 0xD2511F53 / 0xCD9E8D57 and Weyl key increments 0x9E3779B9 /
// 0xBB67AE85.  Only word 0 of the output is needed for block priorities.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
  }
  return c0;
}

// ---------------------------------------------------------------------------
// Request validity shared by every stage (SPIN_DERR_* bits, 0 = valid).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int request_error(int N, int q, int rows, int max_blocks,
                                             int64_t v_ld, int64_t d_ld) {
  int e = 0;
  if (N < 1 || N > SPIN_BLOCK * max_blocks || (v_ld > 0 && (int64_t)N > v_ld)) e |= SPIN_DERR_CTX;
  if (q < N || (d_ld > 0 && (int64_t)q + rows - 1 >= d_ld)) e |= SPIN_DERR_QPOS;
  return e;
}

// Number of selected blocks of a request, clamped to the block capacity.
__device__ __forceinline__ int clamp_nsel(int ns, int max_blocks) {
  return ns < 0 ? 0 : (ns > max_blocks ? max_blocks : ns);
}

__device__ __forceinline__ void raise_error(int32_t* err, int bits) {
  if (err && bits) atomicOr(err, bits);
}

// ---------------------------------------------------------------------------
// wave64 reductions and scans on DPP lane moves (no LDS crossbar round trips):
// a Hillis-Steele scan inside each row of 16 lanes (row_shr 1, 2, 4, 8), then
// row_bcast:15 carries each even row's total into the next row and
// row_bcast:31 carries lanes 0-31's total into rows 2-3.  Lanes whose DPP
// source is outside the row, or whose row is masked off, take the identity.
// A reduction is the inclusive scan's lane 63, read into a scalar.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_move(int identity, int v) {
  return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROW_MASK, 0xF, false);
}

template <class Op>
__device__ __forceinline__ int dpp_incl_scan(int v, int identity, Op op) {
  v = op(v, dpp_move<0x111>(identity, v));  // row_shr:1
  v = op(v, dpp_move<0x112>(identity, v));  // row_shr:2
  v = op(v, dpp_move<0x114>(identity, v));  // row_shr:4
  v = op(v, dpp_move<0x118>(identity, v));  // row_shr:8
  v = op(v, dpp_move<0x142, 0xA>(identity, v));  // row_bcast:15 into rows 1, 3
  v = op(v, dpp_move<0x143, 0xC>(identity, v));  // row_bcast:31 into rows 2, 3
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  const int s = dpp_incl_scan((int)v, 0, [](int a, int b) { return (int)max((uint32_t)a, (uint32_t)b); });
  return (uint32_t)__builtin_amdgcn_readlane(s, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  const int s = dpp_incl_scan((int)v, -1, [](int a, int b) { return (int)min((uint32_t)a, (uint32_t)b); });
  return (uint32_t)__builtin_amdgcn_readlane(s, 63);
}
__device__ __forceinline__ float wave_max_f32(float v) {
  const int s = dpp_incl_scan(__float_as_int(v), __float_as_int(-INFINITY), [](int a, int b) {
    return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
  });
  return __int_as_float(__builtin_amdgcn_readlane(s, 63));
}
// Maxima of NB values per lane over all 64 lanes at once (NB a power of two,
// at most 32), a reduce-scatter: lane l returns the max of value
// l >> (6 - log2 NB) over the wave.  Each step halves the values a lane holds:
// for lane bits 5 and 4 one permlane swap exchanges the halves of a pair of
// registers between partner lanes, so the lanes with the bit clear keep value
// k and the others value k + h, with no selects; for lane bits 3 .. 0 a DPP
// move brings the partner's value.  Lane bits left once one value remains
// are plain butterfly steps.  The max of a set does not depend on the order
// it is taken in.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// value of lane l ^ 2^b for b < 4 (within a row of 16 lanes)
template <int B>
__device__ __forceinline__ float xor_lane_low(float v) {
  if constexpr (B == 3) return dpp_f<0x128>(v);  // row_ror:8
  if constexpr (B == 2) {
    const bool up = (threadIdx.x >> 2) & 1;
    const float dn = dpp_f<0x104>(v), upv = dpp_f<0x114>(v);  // row_shl:4, row_shr:4
    return up ? upv : dn;
  }
  if constexpr (B == 1) return dpp_f<0x4E>(v);  // quad_perm [2, 3, 0, 1]
  return dpp_f<0xB1>(v);                        // quad_perm [1, 0, 3, 2]
}
template <int NB, int B>
__device__ __forceinline__ void scatter_step(float (&x)[NB], int h) {
  if constexpr (B >= 4) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k >= h) break;
      const auto s = B == 5 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x[k]),
                                                               __float_as_uint(x[k + h]), false,
                                                               false)
                            : __builtin_amdgcn_permlane16_swap(__float_as_uint(x[k]),
                                                               __float_as_uint(x[k + h]), false,
                                                               false);
      x[k] = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
    }
  } else {
    const bool up = (threadIdx.x >> B) & 1;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k >= h) break;
      const float keep = up ? x[k + h] : x[k], send = up ? x[k] : x[k + h];
      x[k] = fmaxf(keep, xor_lane_low<B>(send));
    }
  }
}
template <int NB>
__device__ __forceinline__ float wave_max_scatter(float (&x)[NB]) {
  static_assert(NB >= 1 && NB <= 32 && (NB & (NB - 1)) == 0, "a power of two up to 32");
  constexpr int LG = NB == 1 ? 0 : NB == 2 ? 1 : NB == 4 ? 2 : NB == 8 ? 3 : NB == 16 ? 4 : 5;
  if constexpr (LG >= 1) scatter_step<NB, 5>(x, NB / 2);
  if constexpr (LG >= 2) scatter_step<NB, 4>(x, NB / 4);
  if constexpr (LG >= 3) scatter_step<NB, 3>(x, NB / 8);
  if constexpr (LG >= 4) scatter_step<NB, 2>(x, NB / 16);
  if constexpr (LG >= 5) scatter_step<NB, 1>(x, NB / 32);
  float m = x[0];
  if constexpr (LG < 1) m = fmaxf(m, __shfl_xor(m, 32, 64));
  if constexpr (LG < 2) m = fmaxf(m, __shfl_xor(m, 16, 64));
  if constexpr (LG < 3) m = fmaxf(m, xor_lane_low<3>(m));
  if constexpr (LG < 4) m = fmaxf(m, xor_lane_low<2>(m));
  if constexpr (LG < 5) m = fmaxf(m, xor_lane_low<1>(m));
  m = fmaxf(m, xor_lane_low<0>(m));
  return m;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
  return __builtin_amdgcn_readlane(dpp_incl_scan(v, 0, [](int a, int b) { return a + b; }), 63);
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  return dpp_incl_scan(v, 0, [](int a, int b) { return a + b; });
}

// Block-wide exclusive scan for blockDim.x = NT (multiple of 64, <= 1024).
// `tmp` must hold 17 ints of LDS.  Returns the exclusive prefix; *total gets
// the block sum.  Ends with a barrier so `tmp` may be reused immediately.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) tmp[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    const int x = lane < NW ? tmp[lane] : 0;
    const int xi = wave_incl_scan(x);
    if (lane < NW) tmp[lane] = xi - x;
    if (lane == NW - 1) tmp[NW] = xi;
  }
  __syncthreads();
  const int out = incl - v + tmp[wid];
  *total = tmp[NW];
  __syncthreads();
  return out;
}

template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* tmp) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_max_u32(v);
  if (lane == 0) tmp[wid] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) r = max(r, tmp[i]);
  __syncthreads();
  return r;
}
template <int NT>
__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, uint32_t* tmp) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_min_u32(v);
  if (lane == 0) tmp[wid] = v;
  __syncthreads();
  uint32_t r = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) r = min(r, tmp[i]);
  __syncthreads();
  return r;
}
template <int NT>
__device__ __forceinline__ int block_sum_i32(int v, int* tmp) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_sum_i32(v);
  if (lane == 0) tmp[wid] = v;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) r += tmp[i];
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// Radix-select support: find, among a set of u32 keys, the threshold for the
// k largest.  Keys are examined in 8-bit digits, starting below the common
// prefix of the set's max and min so the first histogram is well spread.
// The caller provides per-pass histograms; see RadixState.
// ---------------------------------------------------------------------------
struct RadixState {
  uint64_t prefix;  // resolved high bits (bits below `nb` are zero)
  int nb;           // number of unresolved low bits
  int k;            // rank still to take among keys whose high part equals prefix
  int bin_count;    // keys in the last chosen bin (== k: take them all)
};

// Wave 0 picks the digit: the largest d with (#keys in bins >= d) >= k.
// hist holds 256 bins; writes {digit, k', count} into out[0..2].
__device__ __forceinline__ void radix_pick_digit(const int* hist, int k, int* out) {
  const int lane = threadIdx.x & 63;
  const int c0 = hist[4 * lane + 0], c1 = hist[4 * lane + 1];
  const int c2 = hist[4 * lane + 2], c3 = hist[4 * lane + 3];
  const int mine = c0 + c1 + c2 + c3;
  // keys in the bins of higher lanes (lane 63 holds the top bins)
  const int incl = wave_incl_scan(mine);
  int above = __builtin_amdgcn_readlane(incl, 63) - incl;
  const int cs[4] = {c0, c1, c2, c3};
#pragma unroll
  for (int b = 3; b >= 0; --b) {
    if (above < k && above + cs[b] >= k) {
      out[0] = 4 * lane + b;
      out[1] = k - above;
      out[2] = cs[b];
    }
    above += cs[b];
  }
}

constexpr int kSelThreads = 1024;

// ---------------------------------------------------------------------------
// Block-level selection of the k largest u32 keys among flagged elements
// (ties: lower element index).  Thread t of NT owns elements t*EPT ..
// t*EPT+EPT-1 (EPT <= 32).
// On return, bit e of the result mask marks the chosen elements.
//
// Each 8-bit radix pass costs one barrier: every wave reads the pass's
// histogram and picks the digit itself, and three histograms rotate -- pass
// i fills H[i % 3] and clears H[(i + 1) % 3], whose last readers (the picks
// of pass i - 2) finished before the previous barrier and whose next writers
// (pass i + 1) start after this pass's barrier.  When the last pass takes
// every key of its bin, the keys at or above the threshold are exactly the
// k largest and no rank among equal keys is needed.
// ---------------------------------------------------------------------------
constexpr int kRadixHist = 3 * 256;  // ints of LDS block_select_top needs for `hist`

// The largest digit d with (keys in bins >= d) >= k, in every lane of the
// calling wave: {d, k - keys in bins above d, keys in bin d}.
__device__ __forceinline__ int3 radix_pick_digit_wave(const int* h, int k) {
  const int lane = threadIdx.x & 63;
  const int4 cb = reinterpret_cast<const int4*>(h)[lane];
  const int cs[4] = {cb.x, cb.y, cb.z, cb.w};
  const int incl = wave_incl_scan(cb.x + cb.y + cb.z + cb.w);
  int above = __builtin_amdgcn_readlane(incl, 63) - incl;  // keys in the higher lanes' bins
  int d = 0, kk = 0, cnt = 0;
  bool found = false;
#pragma unroll
  for (int b = 3; b >= 0; --b) {
    if (above < k && above + cs[b] >= k) { d = 4 * lane + b; kk = k - above; cnt = cs[b]; found = true; }
    above += cs[b];
  }
  const int src = __builtin_ctzll(__ballot(found));
  return make_int3(__builtin_amdgcn_readlane(d, src), __builtin_amdgcn_readlane(kk, src),
                   __builtin_amdgcn_readlane(cnt, src));
}

template <int EPT, int NT = kSelThreads>
__device__ uint32_t block_select_top(const uint32_t (&key)[EPT], uint32_t elig, int k,
                                     int* hist, int* sh, uint32_t* tmpu) {
  // hist: kRadixHist ints, sh: 32 ints, tmpu: 2 NT/64
  if (k <= 0) return 0u;
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t mx = 0u, mn = 0xFFFFFFFFu;
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if (elig >> e & 1u) { mx = max(mx, key[e]); mn = min(mn, key[e]); }
  // max and min in one exchange; the first histogram cleared under the same barrier
  mx = wave_max_u32(mx);
  mn = wave_min_u32(mn);
  if (lane == 0) { tmpu[wid] = mx; tmpu[NW + wid] = mn; }
  for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i) { mx = max(mx, tmpu[i]); mn = min(mn, tmpu[NW + i]); }
  int nb = (mx == mn) ? 0 : 32 - __clz(mx ^ mn);
  uint64_t prefix = ((uint64_t)mx >> nb) << nb;
  int cur = 0;
  bool whole_bin = false;
  while (nb > 0) {
    const int db = nb < 8 ? nb : 8, pos = nb - db;
    int* h = hist + 256 * cur;
    int* hn = hist + 256 * (cur == 2 ? 0 : cur + 1);
    for (int i = threadIdx.x; i < 256; i += NT) hn[i] = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if ((elig >> e & 1u) && ((uint64_t)key[e] >> nb) == (prefix >> nb))
        atomicAdd(&h[(key[e] >> pos) & ((1u << db) - 1u)], 1);
    __syncthreads();
    const int3 pick = radix_pick_digit_wave(h, k);
    k = pick.y;
    prefix |= (uint64_t)pick.x << pos;
    nb = pos;
    cur = cur == 2 ? 0 : cur + 1;
    if (pick.z == k) { whole_bin = true; break; }  // every key of this bin is taken
  }
  const uint64_t hp = prefix >> nb;
  uint32_t out = 0u;
  if (whole_bin) {
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if ((elig >> e & 1u) && ((uint64_t)key[e] >> nb) >= hp) out |= 1u << e;
    // the next call clears histograms this call's slowest wave may still read
    __syncthreads();
    return out;
  }
  int eq = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if ((elig >> e & 1u) && ((uint64_t)key[e] >> nb) == hp) ++eq;
  int tot;
  int rank = block_excl_scan<NT>(eq, sh + 4, &tot);
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (!(elig >> e & 1u)) continue;
    const uint64_t hk = (uint64_t)key[e] >> nb;
    if (hk > hp) out |= 1u << e;
    else if (hk == hp) { if (rank < k) out |= 1u << e; ++rank; }
  }
  return out;
}

// Write the ascending list of flagged blocks; pad with -1 to max_blocks.
// inv_row (optional): each block's position in the list, -1 if not flagged.
template <int EPT, int NT = kSelThreads>
__device__ void compact_blocks(uint32_t flag, int max_blocks, int32_t* sel_row, int32_t* n_sel_r,
                               int* sh, int32_t* inv_row = nullptr) {
  int tot;
  int pos = block_excl_scan<NT>(__popc(flag), sh, &tot);
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int j = threadIdx.x * EPT + e;
    if (flag >> e & 1u) {
      if (inv_row) inv_row[j] = pos;
      sel_row[pos++] = j;
    } else if (inv_row && j < max_blocks) {
      inv_row[j] = -1;
    }
  }
  for (int i = tot + threadIdx.x; i < max_blocks; i += NT) sel_row[i] = -1;
  if (threadIdx.x == 0) *n_sel_r = tot;
}

}  // namespace spin
