// Stage 3a of the SPIN decode step: the indexer on the selected blocks only,
// z[i] = sum_h w_h ReLU(q_h . k_i)  ("SPIN: Shadow Predictive Indexer for
// Sparse Attention", Sec. 2; Algorithm 1 step 6).
//
// Per selected 64-slot block the work is a small dense contraction
// [rows x 64 heads x 128] x [128 x 64 slots], so it runs on the matrix cores:
//   * fp8 keys: v_mfma_scale_f32_16x16x128_f8f6f4 with the keys used as they
//     sit in HBM (OCP E4M3).  The query of each head is scaled by a power of
//     two and written as a sum of E4M3 terms (two reproduce a bf16 query,
//     three are used for fp32 queries), one MFMA per term, so the keys need
//     no conversion.  The head scale is folded into w; the per-slot key scale
//     (non-negative) multiplies the ReLU-weighted head sum.
//   * bf16 keys: v_mfma_f32_16x16x32_bf16, fp32 accumulation.
//   * fp32 keys + fp32 queries: a plain fp32 VALU kernel.
//
// MFMA kernels: every wave scores whole pages on its own, with the query of
// one verifier row (all 64 heads) in registers.  It loads each page straight
// from HBM into registers, two pages deep, and brings it into the operand
// layout of the MFMA (the dims a lane holds are the same for query and key):
// with one row by whole-line non-temporal loads and a lane swap, with several
// rows by loading in that layout (PageRegs).  It runs the 16-slot x 16-head
// tiles, applies ReLU and the head weights in registers and leaves lane l
// with slot l's total after a permlane reduce-scatter, so a page's 64 scores
// are one 256-byte row of z (with one row, queued and stored 16 pages at a
// time: ZQueue).  No LDS staging of keys, no barriers in the page loop.  With
// several verifier rows, a stream of `rows` waves walks the same pages (one
// row each); the page comes from HBM once and from L2 for the others.
// Work is split into request-aligned contiguous runs of selected blocks.
#include "plan_dev.h"
#include "spin_launch.h"

namespace spin {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

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
  CandSink sink;  // sink.hint == nullptr: no candidate output
  // another layer's prediction run by the last plan_wgs workgroups of the
  // launch, after the scoring workgroups (dispatched first) leave their CUs
  PredictArgs plan;
  int plan_wgs;
};

// Selected blocks of request r (0 for a request with invalid bounds).
__device__ __forceinline__ int items_of(const ScoreParams& p, int r) {
  const int N = p.ctx[r];
  if (request_error(N, p.qpos[r], p.rows, p.max_blocks, 0, 0)) return 0;
  return clamp_nsel(p.n_sel[r], p.max_blocks);
}

// Exclusive prefix of the per-request item counts in LDS (all requests'
// counters loaded in parallel) plus the total.
struct ItemTable {
  const int* pre;  // [R + 1]
  int total;
};

__device__ __forceinline__ ItemTable build_items(const ScoreParams& p, int* pre, int* tmp,
                                                int* ne_pre = nullptr, int* n_ne = nullptr) {
  constexpr int NT = 256;
  if (p.R <= 64) {  // one wave: one load round and in-wave scans, then one barrier
    if (threadIdx.x < 64) {
      const int r = threadIdx.x;
      const int c = r < p.R ? items_of(p, r) : 0;
      const int ci = wave_incl_scan(c), ne = wave_incl_scan(c > 0 ? 1 : 0);
      if (r < p.R) pre[r] = ci - c;
      if (r == 63) { pre[p.R] = ci; tmp[0] = ne; }
      if (ne_pre && r < p.R) ne_pre[r] = ne - (c > 0 ? 1 : 0);
    }
    __syncthreads();
    if (n_ne) *n_ne = tmp[0];
    return ItemTable{pre, pre[p.R]};
  }
  const int per = (p.R + NT - 1) / NT;  // requests per thread (R <= SPIN_MAX_BATCH)
  const int r0 = threadIdx.x * per;
  int cnt[SPIN_MAX_BATCH / NT];
  int mine = 0, mine_ne = 0;
#pragma unroll
  for (int u = 0; u < SPIN_MAX_BATCH / NT; ++u) {
    cnt[u] = (u < per && r0 + u < p.R) ? items_of(p, r0 + u) : 0;
    mine += cnt[u];
    mine_ne += cnt[u] > 0;
  }
  int total;
  int run = block_excl_scan<NT>(mine, tmp, &total);
#pragma unroll
  for (int u = 0; u < SPIN_MAX_BATCH / NT; ++u)
    if (u < per && r0 + u < p.R) { pre[r0 + u] = run; run += cnt[u]; }
  if (threadIdx.x == 0) pre[p.R] = total;
  if (ne_pre) {  // exclusive prefix count of the requests that have items
    int tot_ne;
    int run_ne = block_excl_scan<NT>(mine_ne, tmp, &tot_ne);
#pragma unroll
    for (int u = 0; u < SPIN_MAX_BATCH / NT; ++u)
      if (u < per && r0 + u < p.R) { ne_pre[r0 + u] = run_ne; run_ne += cnt[u] > 0; }
    *n_ne = tot_ne;
  }
  __syncthreads();
  return ItemTable{pre, total};
}

// Item range [lo, hi) of worker bx of gx (a workgroup or a wave), aligned to
// requests: every request with items gets one worker plus a share of the
// others in proportion to its items, and splits its groups of G items evenly
// over them.  A range then lies in one request, so the worker loads one
// query.  Needs gx >= the number of requests with items (else returns false).
template <int G>
__device__ __forceinline__ bool request_range(const ScoreParams& p, const ItemTable& tb,
                                              const int* ne_pre, int n_ne, int bx, int gx,
                                              int& lo, int& hi, int& req) {
  lo = hi = 0;
  req = -1;
  if (gx < n_ne) return false;
  if (tb.total == 0) return true;
  const auto first_wg = [&](int r) {  // first workgroup of request r; first_wg(R) = gx
    return ne_pre[r] + (int)((int64_t)(gx - n_ne) * tb.pre[r] / tb.total);
  };
  int a = 0, b = p.R - 1;  // last r with first_wg(r) <= bx
  while (a < b) {
    const int mid = (a + b + 1) >> 1;
    if (first_wg(mid) <= bx) a = mid; else b = mid - 1;
  }
  const int r = a;
  req = r;
  const int w = (r + 1 < p.R ? first_wg(r + 1) : gx) - first_wg(r), part = bx - first_wg(r);
  const int items = tb.pre[r + 1] - tb.pre[r], groups = (items + G - 1) / G;
  if (w <= 0 || items <= 0) return true;
  const int gl = (int)((int64_t)part * groups / w), gh = (int)((int64_t)(part + 1) * groups / w);
  lo = tb.pre[r] + gl * G;
  hi = min(tb.pre[r + 1], tb.pre[r] + gh * G);
  return true;
}

// Descriptor of item g (one lane each): page (0 if invalid), block id j,
// request r, position k in the request's block list, context N, and a flag
// for an out-of-range page.
struct Desc {
  int page, j, r, k, N, bad;
};

__device__ __forceinline__ Desc describe(const ScoreParams& p, const ItemTable& tb, int g) {
  Desc d{0, 0, 0, 0, 0, 1};
  if (g >= tb.total) return d;
  int lo = 0, hi = p.R - 1;  // last r with pre[r] <= g
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tb.pre[mid] <= g) lo = mid; else hi = mid - 1;
  }
  const int r = lo, k = g - tb.pre[r];
  const int j = p.sel[(int64_t)r * p.max_blocks + k];
  const int page = (j >= 0 && j < p.max_blocks) ? p.pt[(int64_t)r * p.pt_ld + j] : -1;
  d.bad = !(page >= 0 && page < p.n_pages);
  d.page = d.bad ? 0 : page;
  d.j = j;
  d.r = r;
  d.k = k;
  d.N = p.ctx[r];
  return d;
}

__device__ __forceinline__ int rl(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

__device__ __forceinline__ Desc pick(const Desc& m, int i) {
  return Desc{rl(m.page, i), rl(m.j, i), rl(m.r, i), rl(m.k, i), rl(m.N, i), rl(m.bad, i)};
}

// Descriptor cursor: 64 items' descriptors per wave, refreshed as it advances.
struct DescBatch {
  Desc mine;
  int base;
  __device__ __forceinline__ void init(const ScoreParams& p, const ItemTable& tb, int g) {
    base = g;
    mine = describe(p, tb, g + (int)(threadIdx.x & 63));
    // complete the descriptor loads here (once per 64 items) so later code
    // never has to drain the vector-memory counter to read them
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
  }
  __device__ __forceinline__ Desc get(const ScoreParams& p, const ItemTable& tb, int g) {
    if (g - base >= 64) init(p, tb, g);
    return pick(mine, g - base);
  }
};

// A stream's request-aligned run: blocks [lo, hi) of request r's selected
// list, with that request's context length.
struct Run {
  int r, N, lo, hi;
};

// request_range() for one wave on its own when there are at most 64
// requests: lane r loads request r's counters, in-wave scans give the
// prefixes, and a ballot over the teams' first workers names the request of
// worker bx.  One load round, no LDS and no barrier.  Needs gx >= the number
// of requests with items (the caller guarantees gx >= R).
__device__ __forceinline__ Run wave_run(const ScoreParams& p, int bx, int gx) {
  const int lane = threadIdx.x & 63;
  const bool in = lane < p.R;
  const int c = in ? items_of(p, lane) : 0;
  const int n_ctx = in ? p.ctx[lane] : 0;
  const int ci = wave_incl_scan(c), ne = wave_incl_scan(c > 0 ? 1 : 0);
  const int total = rl(ci, 63), n_ne = rl(ne, 63);
  Run run{0, 0, 0, 0};
  if (total == 0) return run;
  const int pre = ci - c, ne_pre = ne - (c > 0 ? 1 : 0);
  // first worker of request r, as in request_range(); gx past the last request
  const int first = in ? ne_pre + (int)((int64_t)(gx - n_ne) * pre / total) : gx;
  const uint64_t m = __ballot(first <= bx);  // lanes 0 .. r (first() is non-decreasing)
  const int r = 63 - __clzll(m);
  const int f0 = rl(first, r), f1 = r + 1 < p.R ? rl(first, r + 1) : gx;
  const int items = rl(c, r), w = f1 - f0, part = bx - f0;
  run.r = r;
  run.N = rl(n_ctx, r);
  if (w <= 0 || items <= 0) return run;
  // uniform results, kept in scalar registers
  run.lo = __builtin_amdgcn_readfirstlane((int)((int64_t)part * items / w));
  run.hi = __builtin_amdgcn_readfirstlane((int)((int64_t)(part + 1) * items / w));
  return run;
}

// Descriptor cursor over one request's run: lane i describes block
// base + i of the run (64 at a time); the request and its context length are
// the run's.
struct RunCursor {
  int page, j, bad, base;
  int r, N, hi;
  __device__ __forceinline__ void init(const ScoreParams& p, int k) {
    base = k;
    const int kk = k + (int)(threadIdx.x & 63);
    page = 0;
    j = 0;
    bad = 1;
    if (kk < hi) {
      j = p.sel[(int64_t)r * p.max_blocks + kk];
      const int pg = (j >= 0 && j < p.max_blocks) ? p.pt[(int64_t)r * p.pt_ld + j] : -1;
      bad = !(pg >= 0 && pg < p.n_pages);
      page = bad ? 0 : pg;
    }
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0), as in DescBatch
  }
  __device__ __forceinline__ Desc get(const ScoreParams& p, int k) {
    if (k - base >= 64) init(p, k);
    const int i = k - base;
    return Desc{rl(page, i), rl(j, i), r, k, N, rl(bad, i)};
  }
};

// Table-based cursor (runs may cross requests).
struct TableCursor {
  DescBatch b;
  ItemTable tb;
  __device__ __forceinline__ Desc get(const ScoreParams& p, int g) { return b.get(p, tb, g); }
};

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
  // first exchange (partner g ^ 1): keep sub-tiles with bit0 == g & 1
  const float send0 = odd ? p[0] : p[1], send1 = odd ? p[2] : p[3];
  const float keep0 = odd ? p[1] : p[0], keep1 = odd ? p[3] : p[2];
  const float a0 = keep0 + xor16(send0), a1 = keep1 + xor16(send1);
  // second exchange (partner g ^ 2): keep the sub-tile with bit1 == g >> 1
  const bool hi = g >> 1;
  const float send = hi ? a0 : a1, keep = hi ? a1 : a0;
  return keep + xor32(send);
}

// ReLU of a finite float as one integer max on its bits: negative values
// (sign bit set, so negative as int32) and -0 map to +0.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Pack 4 floats into 4 OCP E4M3 bytes (round to nearest even).
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
}

// 32 query values of lane (m, g) of head `head` (row base qrow): dims
// [16g, 16g+16) and [64+16g, 64+16g+16).
__device__ __forceinline__ void load_q32(const void* q, int q_bf16, int64_t hb, int g,
                                         float (&x)[32]) {
  if (q_bf16) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(q) + hb;
    const v4u rr[4] = {*reinterpret_cast<const v4u*>(qp + 16 * g),
                       *reinterpret_cast<const v4u*>(qp + 16 * g + 8),
                       *reinterpret_cast<const v4u*>(qp + 64 + 16 * g),
                       *reinterpret_cast<const v4u*>(qp + 64 + 16 * g + 8)};
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        x[8 * v + 2 * c] = __uint_as_float(rr[v][c] << 16);
        x[8 * v + 2 * c + 1] = __uint_as_float(rr[v][c] & 0xFFFF0000u);
      }
  } else {
    const float* qp = reinterpret_cast<const float*>(q) + hb;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float4 a = *reinterpret_cast<const float4*>(qp + 16 * g + 4 * v);
      const float4 b = *reinterpret_cast<const float4*>(qp + 64 + 16 * g + 4 * v);
      x[4 * v] = a.x; x[4 * v + 1] = a.y; x[4 * v + 2] = a.z; x[4 * v + 3] = a.w;
      x[16 + 4 * v] = b.x; x[16 + 4 * v + 1] = b.y; x[16 + 4 * v + 2] = b.z;
      x[16 + 4 * v + 3] = b.w;
    }
  }
}

// ---------------------------------------------------------------------------
// Query of one verifier row in registers, MFMA A-operand layout: lane (m, g)
// holds head 16 t + m (t = head tile) over the dims of its lane group g.
// ---------------------------------------------------------------------------
template <int KT, int NS>
struct QFull;

template <int NS>
struct QFull<0, NS> {  // fp8 keys: NS E4M3 terms per query value
  v8i part[NS][4];
  float wq[4][4];

  v4u raw[4][4];    // bf16 queries between fetch() and convert()
  float wraw[4][4];  // head weights between fetch() and convert()

  // Issue the loads of the head weights and of a bf16 query (fp32 queries are
  // read by convert()), so that convert() need not wait for later loads.
  __device__ __forceinline__ void fetch(const ScoreParams& p, int q_bf16, int rowid) {
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
    const int64_t qbase = (int64_t)rowid * 64;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) wraw[t][i] = p.w[qbase + 16 * t + 4 * g + i];
    if (!q_bf16) return;
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p.q);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint16_t* qp = q + (qbase + 16 * t + m) * 128;
      raw[t][0] = *reinterpret_cast<const v4u*>(qp + 16 * g);
      raw[t][1] = *reinterpret_cast<const v4u*>(qp + 16 * g + 8);
      raw[t][2] = *reinterpret_cast<const v4u*>(qp + 64 + 16 * g);
      raw[t][3] = *reinterpret_cast<const v4u*>(qp + 64 + 16 * g + 8);
    }
  }

  __device__ __forceinline__ void load(const ScoreParams& p, int q_bf16, int rowid) {
    fetch(p, q_bf16, rowid);
    convert(p, q_bf16, rowid);
  }

  // This lane's 32 values of head tile t (bf16 from raw[t], fp32 loaded here).
  __device__ __forceinline__ void tile_values(const ScoreParams& p, int q_bf16, int rowid, int t,
                                              float (&x)[32]) const {
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
    if (q_bf16) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          x[8 * v + 2 * c] = __uint_as_float(raw[t][v][c] << 16);
          x[8 * v + 2 * c + 1] = __uint_as_float(raw[t][v][c] & 0xFFFF0000u);
        }
    } else {
      load_q32(p.q, q_bf16, ((int64_t)rowid * 64 + 16 * t + m) * 128, g, x);
    }
  }

  // Split one head tile into NS E4M3 terms per value after a per-head
  // power-of-two scaling (2^e amax in [128, 256)); returns the lane's head
  // exponent e (2^-e folds into the head weight).
  __device__ static __forceinline__ int split_tile(const float (&x)[32], v8i (&out)[NS]) {
    float amax = 0.0f;
#pragma unroll
    for (int u = 0; u < 32; ++u) amax = fmaxf(amax, fabsf(x[u]));
    amax = fmaxf(amax, xor16(amax));
    amax = fmaxf(amax, xor32(amax));
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
      out[sp] = v8i{pw[sp][0], pw[sp][1], pw[sp][2], pw[sp][3],
                    pw[sp][4], pw[sp][5], pw[sp][6], pw[sp][7]};
    return e;
  }

  __device__ __forceinline__ void convert(const ScoreParams& p, int q_bf16, int rowid) {
    const int lane = threadIdx.x & 63, g = lane >> 4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float x[32];
      tile_values(p, q_bf16, rowid, t, x);
      v8i o[NS];
      const int e = split_tile(x, o);
#pragma unroll
      for (int sp = 0; sp < NS; ++sp) part[sp][t] = o[sp];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ei = __shfl(e, 4 * g + i, 64);
        wq[t][i] = ldexpf(wraw[t][i], -ei);
      }
    }
  }

  // Workgroup-shared query: LDS bytes per verifier row (the head weights go
  // to a separate 64-float array per row).
  static constexpr int kStageBytes = NS * 4 * 64 * 32;

  v4u sraw[SPIN_MAX_ROWS][8];  // tiles between stage_fetch() and stage_put()
  float sw[SPIN_MAX_ROWS];

  // LDS staging, step 1: issue the loads of head tile t of query row rowid,
  // the k-th tile this wave stages (bf16: 4 registers, fp32: 8).
  __device__ __forceinline__ void stage_fetch(const ScoreParams& p, int q_bf16, int rowid, int t,
                                              int k) {
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
    const int64_t hb = ((int64_t)rowid * 64 + 16 * t + m) * 128;
    if (q_bf16) {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + hb;
      sraw[k][0] = *reinterpret_cast<const v4u*>(qp + 16 * g);
      sraw[k][1] = *reinterpret_cast<const v4u*>(qp + 16 * g + 8);
      sraw[k][2] = *reinterpret_cast<const v4u*>(qp + 64 + 16 * g);
      sraw[k][3] = *reinterpret_cast<const v4u*>(qp + 64 + 16 * g + 8);
    } else {
      const float* qp = reinterpret_cast<const float*>(p.q) + hb;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sraw[k][v] = *reinterpret_cast<const v4u*>(qp + 16 * g + 4 * v);
        sraw[k][4 + v] = *reinterpret_cast<const v4u*>(qp + 64 + 16 * g + 4 * v);
      }
    }
    sw[k] = lane < 16 ? p.w[(int64_t)rowid * 64 + 16 * t + m] : 0.0f;
  }

  // Step 2: convert the k-th staged tile (head tile t) into the LDS stage of
  // `slot`: the MFMA operands of every lane, then the scaled head weights.
  __device__ __forceinline__ void stage_put(int q_bf16, int t, int k, unsigned char* lds,
                                            float* ws, int slot) {
    const int lane = threadIdx.x & 63, m = lane & 15;
    float x[32];
    if (q_bf16) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          x[8 * v + 2 * c] = __uint_as_float(sraw[k][v][c] << 16);
          x[8 * v + 2 * c + 1] = __uint_as_float(sraw[k][v][c] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          x[4 * v + c] = __uint_as_float(sraw[k][v][c]);
          x[16 + 4 * v + c] = __uint_as_float(sraw[k][4 + v][c]);
        }
    }
    v8i o[NS];
    const int e = split_tile(x, o);
    v4u* qs = reinterpret_cast<v4u*>(lds + slot * kStageBytes);
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) {
      qs[((sp * 4 + t) * 2 + 0) * 64 + lane] = v4u{(unsigned)o[sp][0], (unsigned)o[sp][1],
                                                   (unsigned)o[sp][2], (unsigned)o[sp][3]};
      qs[((sp * 4 + t) * 2 + 1) * 64 + lane] = v4u{(unsigned)o[sp][4], (unsigned)o[sp][5],
                                                   (unsigned)o[sp][6], (unsigned)o[sp][7]};
    }
    if (lane < 16) ws[64 * slot + 16 * t + m] = ldexpf(sw[k], -e);
  }

  __device__ __forceinline__ void from_lds(const unsigned char* lds, const float* ws, int slot) {
    const int lane = threadIdx.x & 63, g = lane >> 4;
    const v4u* qs = reinterpret_cast<const v4u*>(lds + slot * kStageBytes);
#pragma unroll
    for (int sp = 0; sp < NS; ++sp)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const v4u a = qs[((sp * 4 + t) * 2 + 0) * 64 + lane], b = qs[((sp * 4 + t) * 2 + 1) * 64 + lane];
        part[sp][t] = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
      }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) wq[t][i] = ws[64 * slot + 16 * t + 4 * g + i];
  }

  // the 16 heads x 16 slots of each head tile for the slots whose key bytes
  // are in kf (MFMA B operand): NS terms accumulated per tile
  __device__ __forceinline__ void mma(const v8i& kf, v4f (&acc)[4]) const {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int sp = 0; sp < NS; ++sp)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(part[sp][t], kf, acc[t], 0, 0, 0,
                                                                  127, 0, 127);
  }
  // One term of head tile t of staged row `slot`, as from_lds() reads it.
  __device__ static __forceinline__ v8i lds_part(const unsigned char* lds, int slot, int sp,
                                                 int t) {
    const int lane = threadIdx.x & 63;
    const v4u* qs = reinterpret_cast<const v4u*>(lds + slot * kStageBytes);
    const v4u a = qs[((sp * 4 + t) * 2 + 0) * 64 + lane], b = qs[((sp * 4 + t) * 2 + 1) * 64 + lane];
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  }

  // this lane's ReLU-weighted sum over its 16 heads of those tiles
  __device__ __forceinline__ float epi(const v4f (&acc)[4]) const {
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) s = fmaf(wq[t][i], relu(acc[t][i]), s);
    return s;
  }
  __device__ __forceinline__ float dot(const v8i& kf) const {
    v4f acc[4];
    mma(kf, acc);
    return epi(acc);
  }
};

template <int NS>
struct QFull<1, NS> {  // bf16 keys
  v4u qa[4][4];
  float wq[4][4];

  // bf16 queries feed the bf16 MFMA as they are: fetching is all there is
  __device__ __forceinline__ void convert(const ScoreParams&, int, int) {}
  __device__ __forceinline__ void load(const ScoreParams& p, int qb, int rowid) { fetch(p, qb, rowid); }

  __device__ __forceinline__ void fetch(const ScoreParams& p, int, int rowid) {
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);
    const int64_t qbase = (int64_t)rowid * 64;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qa[t][ks] = *reinterpret_cast<const v4u*>(qp + (qbase + 16 * t + n) * 128 + 32 * ks + 8 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) wq[t][i] = p.w[qbase + 16 * t + 4 * g + i];
    }
  }

  static constexpr int kStageBytes = 4 * 4 * 64 * 16;

  v4u sraw[SPIN_MAX_ROWS][4];  // tiles between stage_fetch() and stage_put()
  float sw[SPIN_MAX_ROWS];

  // LDS staging, step 1: issue the loads of head tile t of query row rowid,
  // the k-th tile this wave stages.
  __device__ __forceinline__ void stage_fetch(const ScoreParams& p, int, int rowid, int t, int k) {
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)rowid * 64 + 16 * t + n) * 128;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) sraw[k][ks] = *reinterpret_cast<const v4u*>(qp + 32 * ks + 8 * g);
    sw[k] = lane < 16 ? p.w[(int64_t)rowid * 64 + 16 * t + n] : 0.0f;
  }

  // Step 2: the k-th staged tile (head tile t) into the LDS stage of `slot`.
  __device__ __forceinline__ void stage_put(int, int t, int k, unsigned char* lds, float* ws,
                                            int slot) {
    const int lane = threadIdx.x & 63, n = lane & 15;
    v4u* qs = reinterpret_cast<v4u*>(lds + slot * kStageBytes);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qs[(t * 4 + ks) * 64 + lane] = sraw[k][ks];
    if (lane < 16) ws[64 * slot + 16 * t + n] = sw[k];
  }

  __device__ __forceinline__ void from_lds(const unsigned char* lds, const float* ws, int slot) {
    const int lane = threadIdx.x & 63, g = lane >> 4;
    const v4u* qs = reinterpret_cast<const v4u*>(lds + slot * kStageBytes);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qa[t][ks] = qs[(t * 4 + ks) * 64 + lane];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) wq[t][i] = ws[64 * slot + 16 * t + 4 * g + i];
  }

  // this lane's ReLU-weighted sum over its 16 heads for the 16 slots of
  // sub-tile st; kb[4 st + ks] holds the 8 dims 32 ks + 8 g .. of slot 16 st + n
  __device__ __forceinline__ float dot(const v4u (&kb)[16], int st) const {
    v4f acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, qa[t][ks]),
                                                         __builtin_bit_cast(v8bf, kb[4 * st + ks]),
                                                         acc[t], 0, 0, 0);
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) s = fmaf(wq[t][i], relu(acc[t][i]), s);
    return s;
  }
};

// ---------------------------------------------------------------------------
// A key page in registers.  fp8 (KT = 0): lane (n, g) holds, for sub-tile st,
// the key bytes [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g + 16) of slot
// 16 st + n (the dims its fp8 query registers hold), plus slot l's scale.
// bf16 (KT = 1): for sub-tile st and k-step ks, dims 32 ks + 8 g .. + 8 of
// slot 16 st + n.
//
// Loaded in that layout, one instruction touches half of each of 16 128-byte
// lines.  With one verifier row (WL) every load instruction instead reads 8
// whole lines (one kilobyte of the page, each line by 8 lanes), and a
// register pair is then brought into the MFMA layout by exchanging lane bit
// 3 with the pair's register bit (swap_pair: one row rotation by 8 lanes and
// a select per dword).  Whole-line loads can be marked non-temporal
// (streamed through the caches); half-line loads cannot, as the second half
// of a line would miss again.  With several rows the waves of a stream read
// each page in turn and the L2 must keep it, and the rows' epilogues already
// fill the VALU, so they keep the plain half-line loads.  In lane l (l3 =
// bit 3 of l, n' = l & 7) the pair members x (register bit 0) and y (bit 1)
// hold, as loaded, slots n' and 8 + n' of the sub-tile, both at the 16-byte
// chunk c(l3); after the swap both hold slot l & 15, x at chunk c(0) and y at
// chunk c(1), c(b) being the chunk the MFMA layout gives register b of lane l.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void swap_pair(v4u& x, v4u& y) {
  const bool hi = (threadIdx.x & 8) != 0;
  v4u nx, ny;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // row_ror:8 -- lane l reads lane l ^ 8 of its 16-lane row
    const unsigned ty = __builtin_amdgcn_update_dpp(0u, y[c], 0x128, 0xF, 0xF, false);
    const unsigned tx = __builtin_amdgcn_update_dpp(0u, x[c], 0x128, 0xF, 0xF, false);
    nx[c] = hi ? ty : x[c];
    ny[c] = hi ? y[c] : tx;
  }
  x = nx;
  y = ny;
}

__device__ __forceinline__ v4u load16_nt(const uint8_t* a) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4u*>(a));
}

template <int KT>
struct PageRegs;

template <>
struct PageRegs<0> {
  static constexpr int kRegs = 8;
  static constexpr int64_t kBytes = 8192;
  // WL: register 2 st + b holds slots 16 st + 8 b + (l & 7), chunk (l >> 4) + 4 l3.
  // idle: the same instructions, every lane at the page's first 16 bytes (one
  // line per instruction): a worker's loads past its last page keep the
  // loop's load counts, and so its waits, the same without moving a page.
  template <bool WL>
  __device__ static __forceinline__ void load(const ScoreParams& p, int page, v4u (&b)[8],
                                              float& sc, bool idle = false) {
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    const uint8_t* page_base = reinterpret_cast<const uint8_t*>(p.kp) + (int64_t)page * kBytes;
    const int step = idle ? 0 : 1;
    if constexpr (WL) {
      const uint8_t* base =
          page_base + step * ((lane & 7) * 128 + ((lane >> 3) & 1) * 64 + g * 16);
#pragma unroll
      for (int i = 0; i < 8; ++i) b[i] = load16_nt(base + step * i * 1024);
    } else {
      const uint8_t* base = page_base + step * (n * 128 + 16 * g);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        b[2 * st] = *reinterpret_cast<const v4u*>(base + step * st * 2048);
        b[2 * st + 1] = *reinterpret_cast<const v4u*>(base + step * (st * 2048 + 64));
      }
    }
    sc = p.ks[(int64_t)page * 64 + step * lane];
  }
  template <bool WL, class Q>
  __device__ static __forceinline__ float tile(const Q& q, v4u (&b)[8], int st) {
    if constexpr (WL) swap_pair(b[2 * st], b[2 * st + 1]);
    return q.dot(operand(b, st));
  }
  __device__ static __forceinline__ v8i operand(const v4u (&b)[8], int st) {
    const v4u a = b[2 * st], c = b[2 * st + 1];
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)c.x, (int)c.y, (int)c.z, (int)c.w};
  }
  // The page's 4 sub-tiles with several rows (half-line layout), software
  // pipelined: sub-tile st + 1's MFMAs go out before sub-tile st's epilogue,
  // whose accumulators are then complete, so the epilogue's VALU work runs
  // beside matrix-core work instead of waiting for it.
  template <class Q>
  __device__ static __forceinline__ void tiles(const Q& q, const v4u (&b)[8], float (&part)[4]) {
    v4f a0[4], a1[4], a2[4], a3[4];
    q.mma(operand(b, 0), a0);
    q.mma(operand(b, 1), a1);
    __builtin_amdgcn_sched_barrier(0);
    part[0] = q.epi(a0);
    q.mma(operand(b, 2), a2);
    interleave();
    part[1] = q.epi(a1);
    q.mma(operand(b, 3), a3);
    interleave();
    part[2] = q.epi(a2);
    part[3] = q.epi(a3);
  }
  // the scheduling region so far: its 2 NS x 4 MFMAs each followed by 4 VALU
  // instructions (the other sub-tile's epilogue), then a hard boundary
  __device__ static __forceinline__ void interleave() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
};

template <>
struct PageRegs<1> {
  static constexpr int kRegs = 16;
  static constexpr int64_t kBytes = 16384;
  // WL: register 4 st + 2 k1 + b holds slots 16 st + 8 b + (l & 7), bytes
  // 128 k1 + 64 l3 + 16 (l >> 4) of the slot (after the swap: k-step 2 k1 + b)
  template <bool WL>
  __device__ static __forceinline__ void load(const ScoreParams& p, int page, v4u (&b)[16],
                                              float& sc, bool idle = false) {
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    const uint8_t* page_base = reinterpret_cast<const uint8_t*>(p.kp) + (int64_t)page * kBytes;
    const int step = idle ? 0 : 1;  // as PageRegs<0>
    if constexpr (WL) {
      const uint8_t* base =
          page_base + step * ((lane & 7) * 256 + ((lane >> 3) & 1) * 64 + g * 16);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        b[i] = load16_nt(base + step * ((i >> 2) * 4096 + (i & 1) * 2048 + ((i >> 1) & 1) * 128));
    } else {
      const uint8_t* base = page_base + step * (n * 256 + 16 * g);
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          b[4 * st + ks] = *reinterpret_cast<const v4u*>(base + step * (st * 4096 + ks * 64));
    }
    sc = 1.0f;
  }
  template <bool WL, class Q>
  __device__ static __forceinline__ float tile(const Q& q, v4u (&b)[16], int st) {
    if constexpr (WL) {
      swap_pair(b[4 * st], b[4 * st + 1]);
      swap_pair(b[4 * st + 2], b[4 * st + 3]);
    }
    return q.dot(b, st);
  }
};

// ---------------------------------------------------------------------------
// Per-wave scoring.  Workers are streams of `rows` waves (wave w of a
// workgroup scores row w % rows); a stream owns a request-aligned run of
// selected blocks, and each of its waves loads the run's pages two deep into
// registers and scores them for its row.  Span: a run may cross requests
// (fewer streams than requests), so the query is reloaded inside the loop;
// without it the loop keeps no reload state (two waves per SIMD).  Mode:
// kRunWave (at most 64 requests, request-aligned): each wave finds its run by
// itself (wave_run); kRunTable: the workgroup first builds the item table in
// LDS and runs stay request-aligned; kRunSpan: the table, and runs may cross
// requests.
// ---------------------------------------------------------------------------

// The row's top-K threshold hint (0 without a sink).  hint_fetch issues its
// load and hint_use moves it into an SGPR, which waits for it: a worker
// fetches its first row's hint before its descriptors, whose wait then
// covers it, so that the page loop does not wait for the pages in flight.
__device__ __forceinline__ uint32_t hint_fetch(const ScoreParams& p, int rowid) {
  return p.sink.hint ? p.sink.hint[rowid] : 0u;
}
__device__ __forceinline__ uint32_t hint_use(uint32_t h) {
  return __builtin_amdgcn_readfirstlane(h);
}

// The worker's current candidate run (see CandSink): row, first block, the
// block expected next and the candidates so far (wave-uniform), and the last
// qn of them not yet stored, one per lane (lanes 0 .. qn - 1, in order).
// Stored page by page, the candidates cost ~1.4 us of the in-step launch:
// each page with a candidate wrote its few 8-byte pairs as a partial line.
// Queued, they leave in 512-byte stores, one per 64 candidates.
struct CandRun {
  int rowid = -1, k0 = 0, knext = 0, cnt = 0, qn = 0;
  uint32_t qkey = 0, qslot = 0;
};

__device__ __forceinline__ uint2* run_cand(const ScoreParams& p, const CandRun& rs) {
  return p.sink.cand + (int64_t)rs.rowid * p.sink.cand_ld + (int64_t)rs.k0 * 64;
}

// The run's queued candidates, and its counts: rs.cnt at its first block, 0
// at the others, in one coalesced store per 64 blocks (per-page stores of 4
// bytes each went to HBM as partial lines amid the page stream).
__device__ __forceinline__ void run_flush(const ScoreParams& p, const CandRun& rs) {
  if (!p.sink.hint || rs.rowid < 0) return;
  const int lane = threadIdx.x & 63;
  if (lane < rs.qn) run_cand(p, rs)[rs.cnt - rs.qn + lane] = make_uint2(rs.qkey, rs.qslot);
  int32_t* pc = p.sink.pcnt + (int64_t)rs.rowid * p.sink.pcnt_ld + rs.k0;
  const int n = rs.knext - rs.k0;
  for (int i = lane; i < n; i += 64) pc[i] = i == 0 ? rs.cnt : 0;
}

// A scored page: the 4 lane groups' partial sums become slot l's total in
// lane l (times the key scale), one 256-byte store of z, and with a sink the
// block's candidates at or above the row's hint appended to the run.
__device__ __forceinline__ void emit_page(const ScoreParams& p, const float (&part)[4], float sc,
                                          const Desc& d, int rowid, uint32_t hint, int& bad,
                                          CandRun& rs, float* zout = nullptr) {
  const int lane = threadIdx.x & 63;
  const float tot = reduce_scatter4(part);
  const int slot = d.j * 64 + lane;
  const float zv = (slot < d.N && !d.bad) ? tot * sc + 0.0f : 0.0f;
  if (zout) *zout = zv;  // the caller stores it later (ZQueue)
  else p.z[(int64_t)rowid * p.z_ld + (int64_t)d.k * 64 + lane] = zv;
  bad |= d.bad;
  if (p.sink.hint) {  // top-K pre-filter: this block's slots at or above the hint
    const uint32_t key = float_key(zv);
    const bool pass = slot < d.N && key >= hint;
    const uint64_t m = __ballot(pass);
    if (rowid != rs.rowid || d.k != rs.knext) {  // a new run
      run_flush(p, rs);
      rs.rowid = rowid;
      rs.k0 = d.k;
      rs.cnt = 0;
      rs.qn = 0;
    }
    rs.knext = d.k + 1;
    const int c = __popcll(m);
    if (c > 0) {  // (uniform)
      // candidate i of the page goes to queue lane (qn + i) mod 64 and the
      // other lanes to the rest, a permutation: a forward lane permute
      const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      const int dst = (pass ? rs.qn + pos : rs.qn + c + (lane - pos)) & 63;
      const uint32_t nkey = (uint32_t)__builtin_amdgcn_ds_permute(dst * 4, (int)key);
      const uint32_t nslot = (uint32_t)__builtin_amdgcn_ds_permute(dst * 4, slot);
      const int nq = rs.qn + c;
      if (lane >= rs.qn && lane < nq) {
        rs.qkey = nkey;
        rs.qslot = nslot;
      }
      if (nq >= 64) {  // full: 64 in order, then the rest of the page's
        run_cand(p, rs)[rs.cnt - rs.qn + lane] = make_uint2(rs.qkey, rs.qslot);
        if (lane < nq - 64) {
          rs.qkey = nkey;
          rs.qslot = nslot;
        }
        rs.qn = nq - 64;
      } else {
        rs.qn = nq;
      }
      rs.cnt += c;
    }
  }
}

// The z rows of the last (up to) kZQueue pages a wave scored, held in
// registers (lane l: slot l of each page) while the pages are consecutive
// blocks of one row, and stored together when the queue is full, the next
// page does not continue the run, or the loop ends.  Stored page by page,
// the z lines cost ~8 us of a 67 us launch although they are 3 % of its
// bytes (the same stores kept on a few L2-resident lines cost ~1 us, so it
// is their way to HBM amid the page stream, not the instructions); stored
// in bursts of 16 pages they cost ~3 us.
constexpr int kZQueue = 16;

struct ZQueue {
  float q[kZQueue];
  int n = 0, k = 0, rowid = 0;  // pages held; block index and row of the newest (uniform)

  __device__ __forceinline__ void flush(const ScoreParams& p) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kZQueue; ++i)
      if (i >= kZQueue - n)
        p.z[(int64_t)rowid * p.z_ld + (int64_t)(k - (kZQueue - 1 - i)) * 64 + lane] = q[i];
    n = 0;
  }
  __device__ __forceinline__ void push(const ScoreParams& p, float zv, int rid, int kk) {
    if (n > 0 && (n == kZQueue || kk != k + 1 || rid != rowid)) flush(p);
#pragma unroll
    for (int i = 0; i < kZQueue - 1; ++i) q[i] = q[i + 1];
    q[kZQueue - 1] = zv;
    k = kk;
    rowid = rid;
    ++n;
  }
};

// The page loop of one worker: blocks [lo, hi) through cursors `db` (the
// block being scored) and `dd` (the block being loaded, P - 1 ahead, whose
// first pages are already in kb), query row `row` of request q_req in Q.
template <int KT, int NS, int QB, int P, bool Span, bool WL, class Cur>
__device__ __forceinline__ void page_loop(const ScoreParams& p, Cur& db, Cur& dd,
                                          v4u (&kb)[P][PageRegs<KT>::kRegs], float (&sc)[P],
                                          QFull<KT, NS>& Q, int lo, int hi, int q_req, int row,
                                          uint32_t hint_raw) {
  using PR = PageRegs<KT>;
  const int lane = threadIdx.x & 63;
  int rowid = q_req * p.rows + row;
  uint32_t hint = hint_use(hint_raw);
  int bad = 0;
  CandRun rs;
  ZQueue zq;  // one row, runs inside one request: z stores queued
  for (int it = lo; it < hi; it += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int cur = it + u;
      if (cur >= hi) break;
      // refill: page cur + P - 1 (past the end an idle load of the last page)
      PR::template load<WL>(p, dd.get(p, min(cur + P - 1, hi - 1)).page,
                            kb[(u + P - 1) % P], sc[(u + P - 1) % P], cur + P - 1 >= hi);
      const Desc d = db.get(p, cur);
      if (Span && d.r != q_req) {
        q_req = d.r;
        rowid = q_req * p.rows + row;
        Q.load(p, QB, rowid);
        hint = hint_use(hint_fetch(p, rowid));
      }
      float part[4];
      if constexpr (KT == 0 && !WL) {
        PR::tiles(Q, kb[u], part);
      } else {
#pragma unroll
        for (int st = 0; st < 4; ++st) part[st] = PR::template tile<WL>(Q, kb[u], st);
      }
      if constexpr (WL && !Span) {
        float zv;
        emit_page(p, part, KT == 0 ? sc[u] : 1.0f, d, rowid, hint, bad, rs, &zv);
        zq.push(p, zv, rowid, d.k);
      } else {
        emit_page(p, part, KT == 0 ? sc[u] : 1.0f, d, rowid, hint, bad, rs);
      }
    }
  }
  if constexpr (WL && !Span)
    if (zq.n > 0) zq.flush(p);
  run_flush(p, rs);
  if (bad && lane == 0) raise_error(p.err, SPIN_DERR_PAGE);
}

template <int KT, int P, bool WL, class Cur>
__device__ __forceinline__ void first_pages(const ScoreParams& p, Cur& dd,
                                            v4u (&kb)[P][PageRegs<KT>::kRegs], float (&sc)[P],
                                            int lo, int hi) {
#pragma unroll
  for (int u = 0; u < P - 1; ++u)
    PageRegs<KT>::template load<WL>(p, dd.get(p, min(lo + u, hi - 1)).page, kb[u], sc[u],
                                    lo + u >= hi);
}

// One worker with its own query: descriptors first, then the first page, then
// the query, so that the descriptor loads do not queue behind the query loads
// and the query arrives while the page does.
template <int KT, int NS, int QB, int P, bool Span, bool WL, class Cur>
__device__ __forceinline__ void score_pages(const ScoreParams& p, Cur& db, int lo, int hi,
                                            int q_req, int row) {
  Cur dd = db;
  v4u kb[P][PageRegs<KT>::kRegs];
  float sc[P];
  first_pages<KT, P, WL>(p, dd, kb, sc, lo, hi);
  const uint32_t hint = hint_fetch(p, q_req * p.rows + row);  // the query's wait covers it
  QFull<KT, NS> Q;
  Q.fetch(p, QB, q_req * p.rows + row);
  Q.convert(p, QB, q_req * p.rows + row);
  page_loop<KT, NS, QB, P, Span, WL>(p, db, dd, kb, sc, Q, lo, hi, q_req, row, hint);
}

enum { kRunWave = 0, kRunTable = 1, kRunSpan = 2 };

// Worker of scoring workgroup b of g.  Workgroups go to the 8 XCDs round
// robin (b on XCD b % 8); each XCD takes a contiguous range of workers, so
// the workgroups of a request share one XCD's L2 (its query, block list and
// page-table entries, and the lines of z at run boundaries).  A bijection of
// [0, g) whatever the placement.  Used by the one-row kernel (its score
// launch 0.1-0.7 us shorter); the all-rows kernel gained nothing from it.
__device__ __forceinline__ int xcd_worker(int b, int g) {
  const int x = b & 7, i = b >> 3;
  int pre = 0;
  for (int y = 0; y < x; ++y) pre += (g - y + 7) >> 3;
  return pre + i;
}

// WL: whole-line page loads (one verifier row; see PageRegs)
template <int KT, int NS, int QB, int P, int Mode, bool WL>
__global__ __launch_bounds__(256) void k_score_wave(ScoreParams p) {
  extern __shared__ int pre_dyn[];
  __shared__ int tmp[32];
  const int gx = (int)gridDim.x - p.plan_wgs;  // scoring workgroups
  if ((int)blockIdx.x >= gx) {  // the plan role: no barrier, no LDS
    predict_wg(p.plan, (int)blockIdx.x - gx);
    return;
  }
  const int wave = threadIdx.x >> 6;
  const int spw = p.rows == 1 ? 4 : (p.rows == 2 ? 2 : 1);  // streams per workgroup
  const int row = wave % p.rows, stream_id = blockIdx.x * spw + wave / p.rows;
  const int n_streams = gx * spw;
  if constexpr (Mode == kRunWave) {
    // Teams of workgroups: a workgroup's streams split its request-aligned
    // run, found by each wave on its own (no table), and share the request's
    // query rows through LDS, each wave converting rows of the 16-head tiles.
    const Run run = wave_run(p, xcd_worker(blockIdx.x, gx), gx);
    if (run.lo >= run.hi) return;  // the whole workgroup: no barrier follows
    const int s = wave / p.rows, nb = run.hi - run.lo;
    const int lo = __builtin_amdgcn_readfirstlane(run.lo + s * nb / spw);
    const int hi = __builtin_amdgcn_readfirstlane(run.lo + (s + 1) * nb / spw);
    // (uniform: a scalar branch below, so each path's load waits are known where they join)
    const bool active = __builtin_amdgcn_readfirstlane(wave < spw * p.rows && lo < hi ? 1 : 0) != 0;
    unsigned char* lds = reinterpret_cast<unsigned char*>(pre_dyn);
    __shared__ float wstage[SPIN_MAX_ROWS * 64];  // head weights of each row
    // wave w stages head tile w of every row k: the query loads go out first
    // (the descriptor wait covers them), the first page next, and the
    // conversion then runs while the page is in flight
    // the row's hint first: the descriptor wait below covers it
    const uint32_t hint = hint_fetch(p, run.r * p.rows + row);
    QFull<KT, NS> S;
    constexpr int kRowsMax = WL ? 1 : SPIN_MAX_ROWS;  // WL: one row
#pragma unroll
    for (int k = 0; k < kRowsMax; ++k)
      if (k < p.rows) S.stage_fetch(p, QB, run.r * p.rows + k, wave, k);
    RunCursor db, dd;
    v4u kb[P][PageRegs<KT>::kRegs];
    float sc[P];
    // The conversion runs on each path after the query loads are known to be
    // complete: placed after the two paths join, it made the compiler wait
    // for every load, the first pages' too, and so held up the barrier.
    if (active) {
      db.r = run.r;
      db.N = run.N;
      db.hi = hi;
      db.init(p, lo);  // its wait completes the query loads too
      dd = db;
      first_pages<KT, P, WL>(p, dd, kb, sc, lo, hi);
#pragma unroll
      for (int k = 0; k < kRowsMax; ++k)
        if (k < p.rows) S.stage_put(QB, wave, k, lds, wstage, k);
    } else {
#pragma unroll
      for (int k = 0; k < kRowsMax; ++k)
        if (k < p.rows) S.stage_put(QB, wave, k, lds, wstage, k);
    }
    __syncthreads();
    if (!active) return;
    QFull<KT, NS> Q;
    Q.from_lds(lds, wstage, row);
    page_loop<KT, NS, QB, P, false, WL>(p, db, dd, kb, sc, Q, lo, hi, run.r, row, hint);
  } else {
    int n_ne;
    const ItemTable tb = build_items(p, pre_dyn, tmp, pre_dyn + p.R + 1, &n_ne);
    if (wave >= spw * p.rows) return;  // the idle wave with 3 rows; no barrier follows
    int lo, hi, q_req;
    if (!request_range<1>(p, tb, pre_dyn + p.R + 1, n_ne, stream_id, n_streams, lo, hi, q_req)) {
      const int per = (tb.total + n_streams - 1) / n_streams;
      lo = min(tb.total, stream_id * per);
      hi = min(tb.total, lo + per);
      q_req = -1;
    }
    if (lo >= hi) return;
    TableCursor db;
    db.tb = tb;
    db.b.init(p, tb, lo);
    if (q_req < 0) q_req = __builtin_amdgcn_readfirstlane(db.b.mine.r);
    score_pages<KT, NS, QB, P, Mode == kRunSpan, WL>(p, db, lo, hi, q_req, row);
  }
}

// ---------------------------------------------------------------------------
// Several verifier rows, fp8 keys, at most 64 requests: every wave is a stream
// of its own and scores each page of its run for all ROWS rows, so a page is
// loaded once instead of once per row (half-line loads in the MFMA layout: no
// lane swap, and the kernel is bound by the matrix cores and the VALU, not by
// HBM).  The workgroup stages every row's converted query in LDS; the wave
// walks (row, head tile) steps, each the NS x 4 MFMAs of one head tile over
// the page's 4 sub-tiles, reading that tile's query terms and head weights
// from LDS one step ahead.  A step's MFMAs run beside the previous step's
// epilogue (ReLU and weighted head sum, accumulated per sub-tile in the same
// order as QFull::epi), whose accumulators are complete by then, so the
// matrix cores and the VALU work side by side.  Per accumulator the MFMA
// order (term 0, then 1, ...) and per slot the epilogue order (head tile,
// then head) are those of k_score_wave: the scores are the same bits.
// ---------------------------------------------------------------------------
// Waves per workgroup.  Two query terms: 12, with the 4 rows' staged queries
// (64 KB of LDS) one workgroup per CU and three waves per SIMD (at most 168
// registers), which hide more of each other's stalls than two.  Three terms
// (fp32 queries) do not fit 168 registers: 8 waves, two per SIMD.
template <int NS>
constexpr int rows_waves() { return NS == 2 ? 12 : 8; }

template <int NS, int ROWS>
struct RowsPage {
  const unsigned char* lds;
  const float* ws;
  v8i qa[2][NS];  // query terms of a step (double-buffered)
  v4f wv[2];      // its head weights (4 per lane)
  v4f acc[2][4];  // per sub-tile accumulators of a step (double-buffered)
  float s[4];     // the current row's partial sums per sub-tile

  __device__ __forceinline__ void fetch(int k, int b) {
    const int r = k >> 2, t = k & 3, g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) qa[b][sp] = QFull<0, NS>::lds_part(lds, r, sp, t);
    wv[b] = *reinterpret_cast<const v4f*>(ws + 64 * r + 16 * t + 4 * g);
  }
  __device__ __forceinline__ void mma(const v8i (&kf)[4], int b) {
#pragma unroll
    for (int sp = 0; sp < NS; ++sp)
#pragma unroll
      for (int st = 0; st < 4; ++st)
        acc[b][st] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            qa[b][sp], kf[st], sp == 0 ? v4f{0.0f, 0.0f, 0.0f, 0.0f} : acc[b][st], 0, 0, 0, 127,
            0, 127);
  }
  __device__ __forceinline__ void epi(int k, int b) {
    const bool first = (k & 3) == 0;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      float v = first ? 0.0f : s[st];
#pragma unroll
      for (int i = 0; i < 4; ++i) v = fmaf(wv[b][i], relu(acc[b][st][i]), v);
      s[st] = v;
    }
  }
};

template <int NS, int ROWS>
__device__ __forceinline__ void score_rows_page(const ScoreParams& p, const v8i (&kf)[4], float sc,
                                                const Desc& d, int req, RowsPage<NS, ROWS>& R,
                                                const uint32_t (&hint)[ROWS], int& bad,
                                                CandRun (&rs)[ROWS]) {
  constexpr int S = ROWS * 4;  // steps: (row, head tile)
  R.fetch(0, 0);
#pragma unroll
  for (int k = 0; k < S; ++k) {
    const int b = k & 1;
    R.mma(kf, b);
    if (k > 0) R.epi(k - 1, b ^ 1);
    // (after the epilogue in program order: it reads the buffer's weights)
    if (k + 1 < S) R.fetch(k + 1, b ^ 1);
    // each of the step's 4 NS MFMAs followed by a share of the epilogue's 32
    // VALU instructions
#pragma unroll
    for (int i = 0; i < 4 * NS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, (32 + 4 * NS - 1) / (4 * NS), 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (k > 0 && ((k - 1) & 3) == 3) {  // row (k - 1) / 4 complete
      const int r = (k - 1) >> 2;
      emit_page(p, R.s, sc, d, req * ROWS + r, hint[r], bad, rs[r]);
    }
  }
  R.epi(S - 1, (S - 1) & 1);
  emit_page(p, R.s, sc, d, req * ROWS + ROWS - 1, hint[ROWS - 1], bad, rs[ROWS - 1]);
}


template <int NS, int QB, int ROWS>
__global__ __launch_bounds__(64 * rows_waves<NS>()) void k_score_rows(ScoreParams p) {
  constexpr int P = 2;  // pages in flight per wave
  extern __shared__ int pre_dyn[];
  const int gx = (int)gridDim.x - p.plan_wgs;  // scoring workgroups
  if ((int)blockIdx.x >= gx) {  // the plan role: no barrier, no LDS
    if (threadIdx.x < 256) predict_wg(p.plan, (int)blockIdx.x - gx);
    return;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const Run run = wave_run(p, blockIdx.x, gx);
  if (run.lo >= run.hi) return;  // the whole workgroup: no barrier follows
  const int nb = run.hi - run.lo;
  constexpr int W = rows_waves<NS>();
  const int lo = __builtin_amdgcn_readfirstlane(run.lo + wave * nb / W);
  const int hi = __builtin_amdgcn_readfirstlane(run.lo + (wave + 1) * nb / W);
  const bool active = __builtin_amdgcn_readfirstlane(lo < hi ? 1 : 0) != 0;
  unsigned char* lds = reinterpret_cast<unsigned char*>(pre_dyn);
  __shared__ __align__(16) float wstage[SPIN_MAX_ROWS * 64];  // head weights of each row
  uint32_t hraw[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) hraw[r] = hint_fetch(p, run.r * ROWS + r);
  // wave w < 4 stages head tile w of every row (as k_score_wave)
  QFull<0, NS> S;
  const bool stager = wave < 4;
  if (stager)
#pragma unroll
    for (int k = 0; k < ROWS; ++k) S.stage_fetch(p, QB, run.r * ROWS + k, wave, k);
  RunCursor db, dd;
  v4u kb[P][8];
  float sc[P];
  if (active) {
    db.r = run.r;
    db.N = run.N;
    db.hi = hi;
    db.init(p, lo);  // its wait completes the query loads too
    dd = db;
    first_pages<0, P, false>(p, dd, kb, sc, lo, hi);
    if (stager)
#pragma unroll
      for (int k = 0; k < ROWS; ++k) S.stage_put(QB, wave, k, lds, wstage, k);
  } else if (stager) {
#pragma unroll
    for (int k = 0; k < ROWS; ++k) S.stage_put(QB, wave, k, lds, wstage, k);
  }
  __syncthreads();
  if (!active) return;
  uint32_t hint[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) hint[r] = hint_use(hraw[r]);
  RowsPage<NS, ROWS> R;
  R.lds = lds;
  R.ws = wstage;
  int bad = 0;
  CandRun rs[ROWS];
  for (int it = lo; it < hi; it += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int cur = it + u;
      if (cur >= hi) break;
      // refill: page cur + P - 1 (past the end an idle load of the last page)
      PageRegs<0>::load<false>(p, dd.get(p, min(cur + P - 1, hi - 1)).page,
                               kb[(u + P - 1) % P], sc[(u + P - 1) % P], cur + P - 1 >= hi);
      const Desc d = db.get(p, cur);
      v8i kf[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) kf[st] = PageRegs<0>::operand(kb[u], st);
      score_rows_page<NS, ROWS>(p, kf, sc[u], d, run.r, R, hint, bad, rs);
    }
  }
#pragma unroll
  for (int r = 0; r < ROWS; ++r) run_flush(p, rs[r]);
  if (bad && lane == 0) raise_error(p.err, SPIN_DERR_PAGE);
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
template <int KT, int NS, int QB, bool WL>
static void launch_wave_l(const ScoreParams& p, hipStream_t st) {
  constexpr int P = 2;  // pages in flight per wave
  const int spw = p.rows == 1 ? 4 : (p.rows == 2 ? 2 : 1);
  if (p.R <= 64) {  // teams of workgroups, each wave finds its own run
    const size_t stage = (size_t)p.rows * QFull<KT, NS>::kStageBytes;
    const auto wave = k_score_wave<KT, NS, QB, P, kRunWave, WL>;
    const int g = min(resident_workgroups((const void*)wave, 256, stage), p.R * p.max_blocks);
    if (g >= p.R && lds_fits((const void*)wave, stage)) {
      hipLaunchKernelGGL(wave, dim3(g + p.plan_wgs), dim3(256), stage, st, p);
      return;
    }
  }
  const size_t dyn = sizeof(int) * 2 * (p.R + 1);
  const auto aligned = k_score_wave<KT, NS, QB, P, kRunTable, WL>;
  const int g = min(resident_workgroups((const void*)aligned, 256, dyn), p.R * p.max_blocks);
  if (spw * g >= p.R) {  // a stream per request at least: request-aligned runs
    hipLaunchKernelGGL(aligned, dim3(g + p.plan_wgs), dim3(256), dyn, st, p);
    return;
  }
  const auto span = k_score_wave<KT, NS, QB, P, kRunSpan, WL>;
  const int g2 = min(resident_workgroups((const void*)span, 256, dyn), p.R * p.max_blocks);
  hipLaunchKernelGGL(span, dim3(g2 + p.plan_wgs), dim3(256), dyn, st, p);
}

// k_score_rows for fp8 keys with several rows and at most 64 requests, when
// its workgroups fit; false otherwise.
template <int NS, int QB, int ROWS>
static bool launch_rows_n(const ScoreParams& p, hipStream_t st) {
  const size_t stage = (size_t)ROWS * QFull<0, NS>::kStageBytes;
  const auto k = k_score_rows<NS, QB, ROWS>;
  const int g = min(resident_workgroups((const void*)k, 64 * rows_waves<NS>(), stage),
                    p.R * p.max_blocks);
  if (g < p.R || !lds_fits((const void*)k, stage)) return false;
  hipLaunchKernelGGL(k, dim3(g + p.plan_wgs), dim3(64 * rows_waves<NS>()), stage, st, p);
  return true;
}

template <int KT, int NS, int QB>
static void launch_wave(const ScoreParams& p, hipStream_t st) {
  if (p.rows == 1) {
    launch_wave_l<KT, NS, QB, true>(p, st);
    return;
  }
  if constexpr (KT == 0) {
    if (p.R <= 64) {
      const bool done = p.rows == 2 ? launch_rows_n<NS, QB, 2>(p, st)
                        : p.rows == 3 ? launch_rows_n<NS, QB, 3>(p, st)
                                      : launch_rows_n<NS, QB, 4>(p, st);
      if (done) return;
    }
  }
  launch_wave_l<KT, NS, QB, false>(p, st);
}

bool score_filters(const spin_config& c, const spin_batch&) {
  return c.key_dtype != SPIN_F32;  // the per-wave MFMA kernels
}

hipError_t launch_score(const spin_config& c, const spin_batch& b, const void* q, const float* w,
                        const void* kp, const float* ks, const int32_t* pt, int64_t pt_ld,
                        const int32_t* sel, const int32_t* n_sel, float* z, int64_t z_ld,
                        hipStream_t st, const CandSink* sink, const PredictPlan* plan) {
  ScoreParams p{q, w, kp, ks, pt, pt_ld, sel, n_sel, b.ctx_len, b.q_pos, z, z_ld,
                b.batch, b.n_rows, b.max_blocks, b.n_pages, b.err, CandSink{}};
  if (sink && score_filters(c, b)) p.sink = *sink;
  if (plan) {
    if (!score_filters(c, b)) return hipErrorInvalidValue;  // MFMA kernels only
    p.plan = plan->args;
    p.plan_wgs = plan->wgs;
  }
  if (c.key_dtype == SPIN_FP8_E4M3) {
    if (c.q_dtype == SPIN_BF16) launch_wave<0, 2, 1>(p, st);
    else launch_wave<0, 3, 0>(p, st);
  } else if (c.key_dtype == SPIN_BF16) {
    launch_wave<1, 1, 1>(p, st);
  } else {
    hipLaunchKernelGGL(k_score_f32, dim3(b.max_blocks, b.n_rows, b.batch), dim3(64), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace spin
