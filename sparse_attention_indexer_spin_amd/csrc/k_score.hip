// Stage 3a of the SPIN decode step: the indexer on the selected blocks only,
// z[i] = sum_h w_h ReLU(q_h . k_i)  ("SPIN: Shadow Predictive Indexer for
// Sparse Attention", Sec. 2; Algorithm 1 step 6).
//
// Per selected 64-slot block the work is a small dense contraction
// [64 heads x 128] x [128 x 64 slots], so it runs on the matrix cores:
//   * fp8 keys: v_mfma_scale_f32_16x16x128_f8f6f4 with the keys fed straight
//     from HBM as OCP E4M3.  The query of each head is scaled by a power of
//     two and written as a sum of E4M3 terms (two reproduce a bf16 query,
//     three are used for fp32 queries), one MFMA per term, so the keys need
//     no conversion.  The head scale is folded into w; the per-slot key scale
//     (non-negative) multiplies the ReLU-weighted head sum.
//   * bf16 keys: v_mfma_f32_16x16x32_bf16, fp32 accumulation.
//   * fp32 keys + fp32 queries: a plain fp32 VALU kernel.
//
// Work split: the (request, row, selected block) items are cut into one
// contiguous chunk per resident wave.  A wave owns a whole block (4 sub-tiles
// of 16 slots x 64 heads): the ReLU / weight / head-sum epilogue stays in
// registers (each lane sums 4 heads of each of the 4 head tiles), a 3-step
// cross-lane reduce-scatter (v_permlane16/32_swap) leaves lane (n, g) with the
// score of slot 16 g + n, and the block's 64 scores go out as one 256-byte
// store.  Block descriptors (page, block id, row, position) are fetched 64 at
// a time, one per lane, so the key loads never wait on a page-table lookup,
// and the keys of block i+1 are in flight while block i is on the MFMAs.
#include "spin_dev.h"
#include "spin_launch.h"

namespace spin {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// 16-byte streaming load (keys are read once per step: non-temporal)
__device__ __forceinline__ v4u ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
}

struct ScoreParams {
  const void* q;
  const float* w;
  const void* kp;
  const float* ks;
  const int32_t* pt;
  int64_t pt_ld;
  const int32_t* sel;
  const int32_t* n_sel;
  const int32_t* ctx;
  const int32_t* qpos;
  float* z;
  int64_t z_ld;
  int R, rows, max_blocks, n_pages;
  int32_t* err;
};

__device__ __forceinline__ int items_of(const ScoreParams& p, int r) {
  const int N = p.ctx[r];
  if (request_error(N, p.qpos[r], p.rows, p.max_blocks, 0, 0)) return 0;
  return clamp_nsel(p.n_sel[r], p.max_blocks) * p.rows;
}

// This wave's item range [lo, hi).
__device__ __forceinline__ void wave_range(const ScoreParams& p, int n_waves, int wave, int& lo,
                                           int& hi) {
  int T = 0;
  for (int r = 0; r < p.R; ++r) T += items_of(p, r);
  const int per = (T + n_waves - 1) / n_waves;
  lo = min(T, wave * per);
  hi = min(T, lo + per);
}

// Descriptor of item g, computed by one lane: page (0 if invalid), block id j,
// row id (r * rows + row), position k in the request's block list, context N,
// and a flag for an out-of-range page.
struct Desc {
  int page, j, rowid, k, N, bad;
};

__device__ __forceinline__ Desc describe(const ScoreParams& p, int g) {
  Desc d{0, 0, 0, 0, 0, 1};
  int run = 0;
  for (int r = 0; r < p.R; ++r) {
    const int cnt = items_of(p, r);
    if (g >= run && g < run + cnt) {
      const int ns = cnt / p.rows, off = g - run;
      const int row = off / ns, k = off % ns;
      const int j = p.sel[(int64_t)r * p.max_blocks + k];
      const int page = (j >= 0 && j < p.max_blocks) ? p.pt[(int64_t)r * p.pt_ld + j] : -1;
      d.bad = !(page >= 0 && page < p.n_pages);
      d.page = d.bad ? 0 : page;
      d.j = j;
      d.rowid = r * p.rows + row;
      d.k = k;
      d.N = p.ctx[r];
    }
    run += cnt;
  }
  return d;
}

__device__ __forceinline__ int rl(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

__device__ __forceinline__ Desc pick(const Desc& m, int i) {
  return Desc{rl(m.page, i), rl(m.j, i), rl(m.rowid, i), rl(m.k, i), rl(m.N, i), rl(m.bad, i)};
}

// Value of lane l ^ 16 / l ^ 32 (VALU lane swaps, no LDS traffic).
__device__ __forceinline__ float xor16(float v) {
  const int lane = threadIdx.x & 63;
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(((lane >> 4) & 1) ? s[0] : s[1]);
}
__device__ __forceinline__ float xor32(float v) {
  const int lane = threadIdx.x & 63;
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float((lane >> 5) ? s[0] : s[1]);
}

// Lane (n, g) holds p[s] = its partial of sub-tile s (slot 16 s + n);
// returns the 4-lane total of sub-tile g.
__device__ __forceinline__ float reduce_scatter4(const float (&p)[4]) {
  const int g = (threadIdx.x & 63) >> 4;
  const bool odd = g & 1;
  // round 1 (partner g ^ 1): keep sub-tiles with bit0 == g & 1
  const float send0 = odd ? p[0] : p[1], send1 = odd ? p[2] : p[3];
  const float keep0 = odd ? p[1] : p[0], keep1 = odd ? p[3] : p[2];
  const float a0 = keep0 + xor16(send0), a1 = keep1 + xor16(send1);
  // round 2 (partner g ^ 2): keep the sub-tile with bit1 == g >> 1
  const bool hi = g >> 1;
  const float send = hi ? a0 : a1, keep = hi ? a1 : a0;
  return keep + xor32(send);
}

__device__ __forceinline__ float ld_q(const void* q, int q_bf16, int64_t idx) {
  if (q_bf16) {
    const uint16_t b = reinterpret_cast<const uint16_t*>(q)[idx];
    return __uint_as_float((uint32_t)b << 16);
  }
  return reinterpret_cast<const float*>(q)[idx];
}

// Pack 4 floats into 4 OCP E4M3 bytes (round to nearest even).
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
}

__device__ __forceinline__ void store_block(const ScoreParams& p, const Desc& d, float zv) {
  const int lane = threadIdx.x & 63;
  const int slot = d.j * 64 + lane;
  zv = (slot < d.N && !d.bad) ? zv + 0.0f : 0.0f;
  p.z[(int64_t)d.rowid * p.z_ld + (int64_t)d.k * 64 + lane] = zv;
  if (d.bad && lane == 0) raise_error(p.err, SPIN_DERR_PAGE);
}

// ---------------------------------------------------------------------------
// fp8 keys.  Lane (n = lane % 16, g = lane / 16).  MFMA B operand: 32 key
// bytes of slot 16 s + n, dims [16g, 16g+16) and [64+16g, 64+16g+16); the A
// operand holds the same dims of head 16 t + n, so C = q . k^T over all 128
// dims.  C lane layout: rows (heads) 4g + i, column (slot) n.
// ---------------------------------------------------------------------------
template <int NS>
struct QFp8 {
  v8i part[NS][4];
  float wq[4][4];
};

template <int NS>
__device__ __forceinline__ void load_q_fp8(const ScoreParams& p, int q_bf16, int rowid,
                                           QFp8<NS>& Q) {
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const int64_t qbase = (int64_t)rowid * 64;
  const float* wr = p.w + qbase;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t hb = (qbase + 16 * t + m) * 128;
    float x[32];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      x[u] = ld_q(p.q, q_bf16, hb + 16 * g + u);
      x[16 + u] = ld_q(p.q, q_bf16, hb + 64 + 16 * g + u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int u = 0; u < 32; ++u) amax = fmaxf(amax, fabsf(x[u]));
    amax = fmaxf(amax, xor16(amax));
    amax = fmaxf(amax, xor32(amax));
    // 2^e * amax lies in [128, 256): inside the E4M3 range (max 448)
    const int e = amax > 0.0f ? 7 - ilogbf(amax) : 0;
    int pw[NS][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float rem[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) rem[v] = ldexpf(x[4 * u + v], e);
#pragma unroll
      for (int sp = 0; sp < NS; ++sp) {
        const int packed = pack_fp8x4(rem[0], rem[1], rem[2], rem[3]);
        pw[sp][u] = packed;
        if (sp + 1 < NS) {
          rem[0] -= __builtin_amdgcn_cvt_f32_fp8(packed, 0);
          rem[1] -= __builtin_amdgcn_cvt_f32_fp8(packed, 1);
          rem[2] -= __builtin_amdgcn_cvt_f32_fp8(packed, 2);
          rem[3] -= __builtin_amdgcn_cvt_f32_fp8(packed, 3);
        }
      }
    }
#pragma unroll
    for (int sp = 0; sp < NS; ++sp)
      Q.part[sp][t] = v8i{pw[sp][0], pw[sp][1], pw[sp][2], pw[sp][3],
                          pw[sp][4], pw[sp][5], pw[sp][6], pw[sp][7]};
    // weights of the output heads 16t + 4g + i, divided by their head scale
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ei = __shfl(e, 4 * g + i, 64);
      Q.wq[t][i] = ldexpf(wr[16 * t + 4 * g + i], -ei);
    }
  }
}

struct KTileFp8 {
  v4u a[4], b[4];
  float sc[4];
};

__device__ __forceinline__ void issue_fp8(const ScoreParams& p, int page, KTileFp8& t) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const uint8_t* kb = reinterpret_cast<const uint8_t*>(p.kp) + (int64_t)page * (64 * 128);
  const float* sb = p.ks + (int64_t)page * 64;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint8_t* rowp = kb + (16 * s + n) * 128;
    t.a[s] = ld16_nt(rowp + 16 * g);
    t.b[s] = ld16_nt(rowp + 64 + 16 * g);
    t.sc[s] = sb[16 * s + n];
  }
}

template <int NS>
__device__ __forceinline__ float consume_fp8(const QFp8<NS>& Q, const KTileFp8& t) {
  const int g = (threadIdx.x & 63) >> 4;
  float part[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const v8i kf = v8i{(int)t.a[s].x, (int)t.a[s].y, (int)t.a[s].z, (int)t.a[s].w,
                       (int)t.b[s].x, (int)t.b[s].y, (int)t.b[s].z, (int)t.b[s].w};
    float acc_sum = 0.0f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int sp = 0; sp < NS; ++sp)
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Q.part[sp][tt], kf, acc, 0, 0, 0,
                                                               127, 0, 127);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc_sum = fmaf(Q.wq[tt][i], fmaxf(acc[i], 0.0f), acc_sum);
    }
    part[s] = acc_sum;
  }
  const float total = reduce_scatter4(part);
  const float sc = g == 0 ? t.sc[0] : g == 1 ? t.sc[1] : g == 2 ? t.sc[2] : t.sc[3];
  return total * sc;
}

template <int Q_BF16>
__global__ __launch_bounds__(256) void k_score_fp8(ScoreParams p) {
  constexpr int NS = Q_BF16 ? 2 : 3;
  const int lane = threadIdx.x & 63;
  int lo, hi;
  wave_range(p, gridDim.x * 4, blockIdx.x * 4 + (threadIdx.x >> 6), lo, hi);
  if (lo >= hi) return;
  QFp8<NS> Q;
  int q_rowid = -1;
  KTileFp8 t0, t1;
  Desc mine = describe(p, lo + lane);  // descriptors of items base .. base+63
  int base = lo;
  issue_fp8(p, rl(mine.page, 0), t0);
  for (int it = lo; it < hi; it += 2) {
    if (it - base >= 64) { base = it; mine = describe(p, it + lane); }
    const Desc d0 = pick(mine, it - base);
    const bool has1 = it + 1 < hi;
    Desc d1 = d0;
    if (has1) {
      if (it + 1 - base >= 64) { base = it + 1; mine = describe(p, it + 1 + lane); }
      d1 = pick(mine, it + 1 - base);
      issue_fp8(p, d1.page, t1);
    }
    if (d0.rowid != q_rowid) { load_q_fp8<NS>(p, Q_BF16, d0.rowid, Q); q_rowid = d0.rowid; }
    store_block(p, d0, consume_fp8<NS>(Q, t0));
    if (!has1) break;
    if (it + 2 < hi) {
      if (it + 2 - base >= 64) { base = it + 2; mine = describe(p, it + 2 + lane); }
      issue_fp8(p, rl(mine.page, it + 2 - base), t0);
    }
    if (d1.rowid != q_rowid) { load_q_fp8<NS>(p, Q_BF16, d1.rowid, Q); q_rowid = d1.rowid; }
    store_block(p, d1, consume_fp8<NS>(Q, t1));
  }
}

// ---------------------------------------------------------------------------
// bf16 keys.  MFMA 16x16x32: lane (n, g) holds 8 bf16 of slot n per k-step;
// k-step ks covers dims [32 ks + 8 g, +8), so each load instruction reads 64
// contiguous bytes of 16 key rows.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ v8bf as_v8bf(T x) {
  return __builtin_bit_cast(v8bf, x);
}

struct QBf16 {
  uint4 qa[4][4];
  float wq[4][4];
};

__device__ __forceinline__ void load_q_bf16(const ScoreParams& p, int rowid, QBf16& Q) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);
  const int64_t qbase = (int64_t)rowid * 64;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      Q.qa[t][ks] =
          *reinterpret_cast<const uint4*>(qp + (qbase + 16 * t + n) * 128 + 32 * ks + 8 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) Q.wq[t][i] = p.w[qbase + 16 * t + 4 * g + i];
  }
}

// Half a block (2 sub-tiles of 16 slots) per tile keeps the double buffer small.
struct KTileBf16 {
  v4u b[2][4];
};

__device__ __forceinline__ void issue_bf16(const ScoreParams& p, int page, int half,
                                           KTileBf16& t) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(p.kp) + (int64_t)page * (64 * 128);
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      t.b[s][ks] = ld16_nt(kb + (16 * (2 * half + s) + n) * 128 + 32 * ks + 8 * g);
}

__device__ __forceinline__ void consume_bf16(const QBf16& Q, const KTileBf16& t, float* part) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float acc_sum = 0.0f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(Q.qa[tt][ks]), as_v8bf(t.b[s][ks]),
                                                      acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc_sum = fmaf(Q.wq[tt][i], fmaxf(acc[i], 0.0f), acc_sum);
    }
    part[s] = acc_sum;
  }
}

__global__ __launch_bounds__(256) void k_score_bf16(ScoreParams p) {
  const int lane = threadIdx.x & 63;
  int lo, hi;
  wave_range(p, gridDim.x * 4, blockIdx.x * 4 + (threadIdx.x >> 6), lo, hi);
  if (lo >= hi) return;
  QBf16 Q;
  int q_rowid = -1;
  KTileBf16 t0, t1;
  Desc mine = describe(p, lo + lane);
  int base = lo;
  issue_bf16(p, rl(mine.page, 0), 0, t0);
  for (int it = lo; it < hi; ++it) {
    if (it - base >= 64) { base = it; mine = describe(p, it + lane); }
    const Desc d = pick(mine, it - base);
    float part[4];
    issue_bf16(p, d.page, 1, t1);  // second half of this block
    if (d.rowid != q_rowid) { load_q_bf16(p, d.rowid, Q); q_rowid = d.rowid; }
    consume_bf16(Q, t0, part);
    if (it + 1 < hi) {  // first half of the next block
      if (it + 1 - base >= 64) { base = it + 1; mine = describe(p, it + 1 + lane); }
      issue_bf16(p, rl(mine.page, it + 1 - base), 0, t0);
    }
    consume_bf16(Q, t1, part + 2);
    store_block(p, d, reduce_scatter4(part));
  }
}

// ---------------------------------------------------------------------------
// fp32 keys and queries: one thread per slot, fp32 FMA accumulation over the
// 128 dims, then the ReLU-weighted head sum.  Query and weights in LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_score_f32(ScoreParams p) {
  __shared__ float qs[64 * 128];
  __shared__ float ws[64];
  const int k = blockIdx.x, row = blockIdx.y, r = blockIdx.z;
  const int N = p.ctx[r];
  if (request_error(N, p.qpos[r], p.rows, p.max_blocks, 0, 0)) return;
  if (k >= clamp_nsel(p.n_sel[r], p.max_blocks)) return;
  const int64_t qbase = ((int64_t)r * p.rows + row) * 64;
  const float* qf = reinterpret_cast<const float*>(p.q) + qbase * 128;
  for (int i = threadIdx.x; i < 64 * 128; i += 64) qs[i] = qf[i];
  ws[threadIdx.x] = p.w[qbase + threadIdx.x];
  __syncthreads();
  const int j = p.sel[(int64_t)r * p.max_blocks + k];
  const int page = (j >= 0 && j < p.max_blocks) ? p.pt[(int64_t)r * p.pt_ld + j] : -1;
  float* zr = p.z + ((int64_t)r * p.rows + row) * p.z_ld + (int64_t)k * 64;
  if (page < 0 || page >= p.n_pages) {
    if (threadIdx.x == 0) raise_error(p.err, SPIN_DERR_PAGE);
    zr[threadIdx.x] = 0.0f;
    return;
  }
  const float* key =
      reinterpret_cast<const float*>(p.kp) + ((int64_t)page * 64 + threadIdx.x) * 128;
  float kr[128];
#pragma unroll
  for (int d = 0; d < 128; d += 4) {
    const float4 v = *reinterpret_cast<const float4*>(key + d);
    kr[d] = v.x; kr[d + 1] = v.y; kr[d + 2] = v.z; kr[d + 3] = v.w;
  }
  float zsum = 0.0f;
  for (int h = 0; h < 64; ++h) {
    float s = 0.0f;
#pragma unroll
    for (int d = 0; d < 128; ++d) s = fmaf(qs[h * 128 + d], kr[d], s);
    zsum = fmaf(ws[h], fmaxf(s, 0.0f), zsum);
  }
  const int slot = j * 64 + threadIdx.x;
  zr[threadIdx.x] = slot < N ? zsum + 0.0f : 0.0f;
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
hipError_t launch_score(const spin_config& c, const spin_batch& b, const void* q, const float* w,
                        const void* kp, const float* ks, const int32_t* pt, int64_t pt_ld,
                        const int32_t* sel, const int32_t* n_sel, float* z, int64_t z_ld,
                        hipStream_t st) {
  ScoreParams p{q, w, kp, ks, pt, pt_ld, sel, n_sel, b.ctx_len, b.q_pos, z, z_ld,
                b.batch, b.n_rows, b.max_blocks, b.n_pages, b.err};
  if (c.key_dtype == SPIN_FP8_E4M3) {
    if (c.q_dtype == SPIN_BF16) {
      const int g = resident_workgroups((const void*)k_score_fp8<1>, 256);
      hipLaunchKernelGGL(k_score_fp8<1>, dim3(g), dim3(256), 0, st, p);
    } else {
      const int g = resident_workgroups((const void*)k_score_fp8<0>, 256);
      hipLaunchKernelGGL(k_score_fp8<0>, dim3(g), dim3(256), 0, st, p);
    }
  } else if (c.key_dtype == SPIN_BF16) {
    const int g = resident_workgroups((const void*)k_score_bf16, 256);
    hipLaunchKernelGGL(k_score_bf16, dim3(g), dim3(256), 0, st, p);
  } else {
    hipLaunchKernelGGL(k_score_f32, dim3(b.max_blocks, b.n_rows, b.batch), dim3(64), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace spin
