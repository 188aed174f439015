// Stage 3a of the SPIN decode step: the indexer on the selected blocks only,
// z[i] = sum_h w_h ReLU(q_h . k_i)  ("SPIN: Shadow Predictive Indexer for
// Sparse Attention", Sec. 2; Algorithm 1 step 6).
//
// Per selected 64-slot block the work is a small dense contraction
// [64 heads x 128] x [128 x 64 slots], so it runs on the matrix cores:
//   * fp8 keys: v_mfma_scale_f32_16x16x128_f8f6f4 with the keys fed straight
//     from HBM as OCP E4M3; the query is split per head into hi + lo E4M3
//     parts after a power-of-two head scale (hi + lo carries the 8
//     significant bits of a bf16 query), so one 16x16 tile costs two MFMAs
//     and no key conversion.  The head scale is folded into w; the per-slot
//     key scale (non-negative) multiplies the ReLU-weighted head sum.
//   * bf16 keys: v_mfma_f32_16x16x32_bf16, fp32 accumulation.
//   * fp32 keys + fp32 queries: a plain fp32 VALU kernel.
// A wave owns 16 slots x 64 heads per MFMA group (4 head tiles of 16), so the
// ReLU / weight / head-sum epilogue stays in registers: each lane sums its 4
// heads of every tile, then two cross-lane adds finish the 64-head sum.
// Work: the (request, row, selected block) items are split into one
// contiguous chunk per resident wave; keys are read exactly once.
#include "spin_dev.h"
#include "spin_launch.h"

namespace spin {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

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

// Item cursor over (request, row, selected block k).
struct Cursor {
  int r, row, k, nsel;
};

__device__ __forceinline__ bool find_chunk(const ScoreParams& p, int n_waves, int wave, int& lo,
                                           int& hi, Cursor& c) {
  int T = 0;
  for (int r = 0; r < p.R; ++r) T += items_of(p, r);
  const int per = (T + n_waves - 1) / n_waves;
  lo = wave * per;
  hi = min(T, lo + per);
  if (lo >= hi) return false;
  int run = 0;
  for (int r = 0; r < p.R; ++r) {
    const int cnt = items_of(p, r);
    if (lo < run + cnt) {
      const int off = lo - run, ns = cnt / p.rows;
      c.r = r; c.row = off / ns; c.k = off % ns; c.nsel = ns;
      return true;
    }
    run += cnt;
  }
  return false;
}

__device__ __forceinline__ void advance(const ScoreParams& p, Cursor& c) {
  if (++c.k < c.nsel) return;
  c.k = 0;
  if (++c.row < p.rows) return;
  c.row = 0;
  do {
    ++c.r;
    c.nsel = c.r < p.R ? items_of(p, c.r) / p.rows : 1;
  } while (c.nsel == 0);
}

__device__ __forceinline__ int page_of(const ScoreParams& p, const Cursor& c, int& j) {
  j = p.sel[(int64_t)c.r * p.max_blocks + c.k];
  const int page = (j >= 0 && j < p.max_blocks) ? p.pt[(int64_t)c.r * p.pt_ld + j] : -1;
  return page;
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

// ---------------------------------------------------------------------------
// fp8 keys.  Lane (n = lane % 16, g = lane / 16).  For the MFMA B operand the
// lane holds 32 key bytes of slot n: dims [16g, 16g+16) and [64+16g, 64+16g+16);
// the A operand holds the same dims of head m = lane % 16, so C = q . k^T over
// all 128 dims.  C lane layout: rows (heads) 4g + i, column (slot) n.
// ---------------------------------------------------------------------------
struct QFp8 {
  v8i hi[4], lo[4];
  float wq[4][4];
};

__device__ __forceinline__ void load_q_fp8(const ScoreParams& p, int q_bf16, const Cursor& c,
                                           QFp8& Q) {
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const int64_t qbase = ((int64_t)c.r * p.rows + c.row) * 64;
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
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    // 2^e * amax lies in [128, 256): well inside the E4M3 range (max 448)
    const int e = amax > 0.0f ? 7 - ilogbf(amax) : 0;
    int hw[8], lw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float s[4], h[4], l[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) s[v] = ldexpf(x[4 * u + v], e);
      hw[u] = pack_fp8x4(s[0], s[1], s[2], s[3]);
      h[0] = __builtin_amdgcn_cvt_f32_fp8(hw[u], 0);
      h[1] = __builtin_amdgcn_cvt_f32_fp8(hw[u], 1);
      h[2] = __builtin_amdgcn_cvt_f32_fp8(hw[u], 2);
      h[3] = __builtin_amdgcn_cvt_f32_fp8(hw[u], 3);
#pragma unroll
      for (int v = 0; v < 4; ++v) l[v] = s[v] - h[v];
      lw[u] = pack_fp8x4(l[0], l[1], l[2], l[3]);
    }
    Q.hi[t] = v8i{hw[0], hw[1], hw[2], hw[3], hw[4], hw[5], hw[6], hw[7]};
    Q.lo[t] = v8i{lw[0], lw[1], lw[2], lw[3], lw[4], lw[5], lw[6], lw[7]};
    // weights of the output heads 16t + 4g + i, divided by their head scale
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ei = __shfl(e, 4 * g + i, 64);
      Q.wq[t][i] = ldexpf(wr[16 * t + 4 * g + i], -ei);
    }
  }
}

template <int Q_BF16>
__global__ __launch_bounds__(256) void k_score_fp8(ScoreParams p) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int n_waves = gridDim.x * 4;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lo, hi;
  Cursor c;
  if (!find_chunk(p, n_waves, wave, lo, hi, c)) return;
  const uint8_t* kp = reinterpret_cast<const uint8_t*>(p.kp);
  QFp8 Q;
  int qr = -1, qrow = -1;
  for (int it = lo; it < hi; ++it, advance(p, c)) {
    if (c.r != qr || c.row != qrow) {
      load_q_fp8(p, Q_BF16, c, Q);
      qr = c.r;
      qrow = c.row;
    }
    int j;
    const int page = page_of(p, c, j);
    const int N = p.ctx[c.r];
    float* zr = p.z + ((int64_t)c.r * p.rows + c.row) * p.z_ld + (int64_t)c.k * 64;
    if (page < 0 || page >= p.n_pages) {
      if (lane == 0) raise_error(p.err, SPIN_DERR_PAGE);
      zr[lane] = 0.0f;
      continue;
    }
    const uint8_t* kb = kp + (int64_t)page * (64 * 128);
    const float* sb = p.ks + (int64_t)page * 64;
    uint4 b0[4], b1[4];
    float sc[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint8_t* rowp = kb + (16 * s + n) * 128;
      b0[s] = *reinterpret_cast<const uint4*>(rowp + 16 * g);
      b1[s] = *reinterpret_cast<const uint4*>(rowp + 64 + 16 * g);
      sc[s] = sb[16 * s + n];
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v8i kf = v8i{(int)b0[s].x, (int)b0[s].y, (int)b0[s].z, (int)b0[s].w,
                         (int)b1[s].x, (int)b1[s].y, (int)b1[s].z, (int)b1[s].w};
      float part = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Q.hi[t], kf, acc, 0, 0, 0, 127, 0,
                                                               127);
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Q.lo[t], kf, acc, 0, 0, 0, 127, 0,
                                                               127);
#pragma unroll
        for (int i = 0; i < 4; ++i) part = fmaf(Q.wq[t][i], fmaxf(acc[i], 0.0f), part);
      }
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      const int slot = j * 64 + 16 * s + n;
      const float zv = slot < N ? part * sc[s] + 0.0f : 0.0f;
      if (g == 0) zr[16 * s + n] = zv;
    }
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

__global__ __launch_bounds__(256) void k_score_bf16(ScoreParams p) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int n_waves = gridDim.x * 4;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lo, hi;
  Cursor c;
  if (!find_chunk(p, n_waves, wave, lo, hi, c)) return;
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(p.kp);
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);
  uint4 qa[4][4];
  float wq[4][4];
  int qr = -1, qrow = -1;
  for (int it = lo; it < hi; ++it, advance(p, c)) {
    if (c.r != qr || c.row != qrow) {
      const int64_t qbase = ((int64_t)c.r * p.rows + c.row) * 64;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          qa[t][ks] = *reinterpret_cast<const uint4*>(qp + (qbase + 16 * t + n) * 128 + 32 * ks +
                                                      8 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) wq[t][i] = p.w[qbase + 16 * t + 4 * g + i];
      }
      qr = c.r;
      qrow = c.row;
    }
    int j;
    const int page = page_of(p, c, j);
    const int N = p.ctx[c.r];
    float* zr = p.z + ((int64_t)c.r * p.rows + c.row) * p.z_ld + (int64_t)c.k * 64;
    if (page < 0 || page >= p.n_pages) {
      if (lane == 0) raise_error(p.err, SPIN_DERR_PAGE);
      zr[lane] = 0.0f;
      continue;
    }
    const uint16_t* kb = kp + (int64_t)page * (64 * 128);
    uint4 b[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        b[s][ks] = *reinterpret_cast<const uint4*>(kb + (16 * s + n) * 128 + 32 * ks + 8 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float part = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(qa[t][ks]), as_v8bf(b[s][ks]), acc,
                                                        0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) part = fmaf(wq[t][i], fmaxf(acc[i], 0.0f), part);
      }
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      const int slot = j * 64 + 16 * s + n;
      const float zv = slot < N ? part + 0.0f : 0.0f;
      if (g == 0) zr[16 * s + n] = zv;
    }
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
  const float* key = reinterpret_cast<const float*>(p.kp) + ((int64_t)page * 64 + threadIdx.x) * 128;
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
