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
// MFMA kernels: a workgroup of 4 waves owns a contiguous run of
// (request, selected block) items; wave w owns heads 16w..16w+15 of every
// verifier row, so its query tile stays in registers and each key page is
// read from HBM once for all rows.  A page is staged global -> VGPR ->
// LDS (16-byte chunks XOR-swizzled by slot so the MFMA operand reads are
// bank-conflict free), double-buffered: page i+1 is written to LDS and page
// i+2 is in flight while page i is on the matrix cores.  Each wave reduces
// ReLU(qk) * w over its 16 heads in registers (3-step permlane
// reduce-scatter); the 4 head-tile partials meet in LDS and one wave writes
// the page's 64 scores per row as one 256-byte store.
#include "spin_dev.h"
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
// Key pages: geometry, staging and the swizzled LDS layout.
// KT = 0: fp8 rows of 128 B (8 chunks); KT = 1: bf16 rows of 256 B (16 chunks).
// Chunk c of slot s lives at LDS byte s * row + 16 * (c ^ (s & 7)), so the 8
// lanes of an MFMA operand read (8 slots, same logical chunk) hit 8
// different bank groups.
// ---------------------------------------------------------------------------
template <int KT>
struct KGeo {
  static constexpr int kRow = KT == 0 ? 128 : 256;
  static constexpr int kBytes = 64 * kRow;
  static constexpr int kChunksPerRow = kRow / 16;
  static constexpr int kPerThread = kBytes / 16 / 256;
};

__device__ __forceinline__ int swz(int slot, int chunk, int row_bytes) {
  return slot * row_bytes + 16 * (chunk ^ (slot & 7));
}

#define SPIN_LDS(ptr) ((__attribute__((address_space(3))) void*)(ptr))

// Direct global -> LDS copy of one key page (and its fp8 scales) into a ring
// slot.  Wave w writes LDS bytes [w * kBytes/4, (w+1) * kBytes/4) in 1 KB
// instructions (lane l -> 16 l within each); each lane fetches the global
// chunk that the swizzle places there, so every instruction still reads one
// contiguous 1 KB run of the page.  Returns nothing; completion is tracked
// with vmcnt by the caller (kDmaOps[w] instructions per page for wave w).
template <int KT>
struct Dma {
  using G = KGeo<KT>;
  static constexpr int kPerWave = G::kBytes / 4 / 1024;  // 1 KB instructions per wave
  __device__ static __forceinline__ int ops(int wave) { return kPerWave + (KT == 0 && wave == 0); }
  __device__ static __forceinline__ void issue(const ScoreParams& p, int page, uint8_t* kslot,
                                               float* sslot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint8_t* base = reinterpret_cast<const uint8_t*>(p.kp) + (int64_t)page * G::kBytes;
#pragma unroll
    for (int u = 0; u < kPerWave; ++u) {
      const int lds_off = (wave * kPerWave + u) * 1024;      // this instruction's 1 KB
      const int pos = lds_off + 16 * lane;                    // LDS byte this lane fills
      const int slot = pos / G::kRow, cpos = (pos % G::kRow) / 16;
      const int c = cpos ^ (slot & 7);                        // global chunk stored there
      __builtin_amdgcn_global_load_lds(base + slot * G::kRow + 16 * c, SPIN_LDS(kslot + lds_off),
                                       16, 0, 0);
    }
    if (KT == 0 && wave == 0)
      __builtin_amdgcn_global_load_lds(p.ks + (int64_t)page * 64 + lane, SPIN_LDS(sslot), 4, 0, 0);
  }
};

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt left at their maxima), n <= 63.
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Wait until at most `later` pages' DMA (issued after the page needed now)
// are outstanding for this wave.
template <int KT, int NB>
__device__ __forceinline__ void wait_pages(int later) {
  const int wave = threadIdx.x >> 6;
  const bool w0 = KT == 0 && wave == 0;  // wave 0 also copies the scales
  constexpr int P = Dma<KT>::kPerWave;
#define SPIN_WAIT_CASE(k)                                 \
  case k:                                                 \
    if (w0) wait_vm<(P + 1) * (k)>(); else wait_vm<P * (k)>(); \
    break;
  switch (later < NB - 1 ? later : NB - 1) {
    SPIN_WAIT_CASE(0) SPIN_WAIT_CASE(1) SPIN_WAIT_CASE(2) SPIN_WAIT_CASE(3)
    SPIN_WAIT_CASE(4) SPIN_WAIT_CASE(5) SPIN_WAIT_CASE(6) SPIN_WAIT_CASE(7)
    default: wait_vm<0>();
  }
#undef SPIN_WAIT_CASE
}

// ---------------------------------------------------------------------------
// Query tiles in registers: wave w holds heads 16w .. 16w+15 of NR rows.
// ---------------------------------------------------------------------------
template <int KT, int NS, int NR>
struct QTile;

// fp8 keys: NS E4M3 terms per value, MFMA A-operand layout (lane (m, g):
// head 16w + m, the same dims the key operand holds).
template <int NS, int NR>
struct QTile<0, NS, NR> {
  v8i part[NR][NS];
  float wq[NR][4];  // weights of output heads 16w + 4g + i, over 2^e_head

  __device__ __forceinline__ void load(const ScoreParams& p, int q_bf16, int r) {
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4, w = threadIdx.x >> 6;
#pragma unroll
    for (int row = 0; row < NR; ++row) {
      if (row >= p.rows) break;
      const int64_t qbase = ((int64_t)r * p.rows + row) * 64;
      float x[32];
      load_q32(p.q, q_bf16, (qbase + 16 * w + m) * 128, g, x);
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
        part[row][sp] = v8i{pw[sp][0], pw[sp][1], pw[sp][2], pw[sp][3],
                            pw[sp][4], pw[sp][5], pw[sp][6], pw[sp][7]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ei = __shfl(e, 4 * g + i, 64);
        wq[row][i] = ldexpf(p.w[qbase + 16 * w + 4 * g + i], -ei);
      }
    }
  }

  // partial[row][s]: this lane's ReLU-weighted sum over its 4 heads, sub-tile s
  __device__ __forceinline__ void mul(const uint8_t* kbuf, int rows,
                                      float (&partial)[NR][4]) const {
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int slot = 16 * s + n;
      const v4u a = *reinterpret_cast<const v4u*>(kbuf + swz(slot, g, 128));
      const v4u b = *reinterpret_cast<const v4u*>(kbuf + swz(slot, 4 + g, 128));
      const v8i kf = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w,
                         (int)b.x, (int)b.y, (int)b.z, (int)b.w};
#pragma unroll
      for (int row = 0; row < NR; ++row) {
        if (row >= rows) break;
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int sp = 0; sp < NS; ++sp)
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(part[row][sp], kf, acc, 0, 0, 0,
                                                                 127, 0, 127);
        float t = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) t = fmaf(wq[row][i], relu(acc[i]), t);
        partial[row][s] = t;
      }
    }
  }
};

// bf16 keys: MFMA 16x16x32, lane (n, g): head 16w + n, k-step ks covering
// dims [32 ks + 8 g, +8).
template <int NS, int NR>
struct QTile<1, NS, NR> {
  v4u qa[NR][4];
  float wq[NR][4];

  __device__ __forceinline__ void load(const ScoreParams& p, int, int r) {
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4, w = threadIdx.x >> 6;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);
#pragma unroll
    for (int row = 0; row < NR; ++row) {
      if (row >= p.rows) break;
      const int64_t qbase = ((int64_t)r * p.rows + row) * 64;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qa[row][ks] =
            *reinterpret_cast<const v4u*>(qp + (qbase + 16 * w + n) * 128 + 32 * ks + 8 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) wq[row][i] = p.w[qbase + 16 * w + 4 * g + i];
    }
  }

  __device__ __forceinline__ void mul(const uint8_t* kbuf, int rows,
                                      float (&partial)[NR][4]) const {
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int slot = 16 * s + n;
      v4u kb[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kb[ks] = *reinterpret_cast<const v4u*>(kbuf + swz(slot, 4 * ks + g, 256));
#pragma unroll
      for (int row = 0; row < NR; ++row) {
        if (row >= rows) break;
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, qa[row][ks]),
                                                        __builtin_bit_cast(v8bf, kb[ks]), acc,
                                                        0, 0, 0);
        float t = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) t = fmaf(wq[row][i], relu(acc[i]), t);
        partial[row][s] = t;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// The MFMA score kernel.  NB = ring slots (NB - 1 pages in flight).
// ---------------------------------------------------------------------------
template <int KT, int NR, int NB>
struct ScoreShared {
  uint8_t kbuf[NB][KGeo<KT>::kBytes] __attribute__((aligned(16)));
  float sbuf[NB][64];
  float red[NR][4][64];
  int tmp[32];
};

// Occupancy target: 4 waves per SIMD for one verifier row, fewer for more
// rows (their query tiles need more registers).
template <int NR>
struct WavesPerEU {
  static constexpr int value = NR == 1 ? 4 : (NR == 2 ? 3 : 2);
};

template <int KT, int NS, int NR, int QB, int NB>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(WavesPerEU<NR>::value, 8))) void k_score_mfma(ScoreParams p) {
  __shared__ ScoreShared<KT, NR, NB> sm;
  extern __shared__ int pre_dyn[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const ItemTable tb = build_items(p, pre_dyn, sm.tmp);
  const int per = (tb.total + gridDim.x - 1) / gridDim.x;
  const int lo = min(tb.total, (int)blockIdx.x * per), hi = min(tb.total, lo + per);
  if (lo >= hi) return;
  QTile<KT, NS, NR> Q;
  int q_req = -1;
  DescBatch db, dd;  // cursors of the scoring stream and of the copy stream
  db.init(p, tb, lo);
  dd.init(p, tb, lo);
  // prologue: NB - 1 pages in flight
  for (int i = 0; i < NB - 1 && lo + i < hi; ++i)
    Dma<KT>::issue(p, dd.get(p, tb, lo + i).page, sm.kbuf[i], sm.sbuf[i]);
  for (int it = lo; it < hi; ++it) {
    const int slot = (it - lo) % NB;
    const int ahead = it + NB - 1;
    if (ahead < hi) {
      const int as = (ahead - lo) % NB;
      Dma<KT>::issue(p, dd.get(p, tb, ahead).page, sm.kbuf[as], sm.sbuf[as]);
    }
    const Desc d = db.get(p, tb, it);
    if (d.r != q_req) { Q.load(p, QB, d.r); q_req = d.r; }
    wait_pages<KT, NB>(min(NB - 1, hi - 1 - it));
    __builtin_amdgcn_s_barrier();  // page `it` is in ring slot `slot` for every wave
    float partial[NR][4];
    Q.mul(sm.kbuf[slot], p.rows, partial);
    const float sc = KT == 0 ? sm.sbuf[slot][lane] : 1.0f;
#pragma unroll
    for (int row = 0; row < NR; ++row) {
      if (row >= p.rows) break;
      sm.red[row][wave][lane] = reduce_scatter4(partial[row]);
    }
    __syncthreads();  // partials in `red`; ring slot `slot` may be refilled
    if (wave == (it & 3)) {
      const int s0 = d.j * 64 + lane;
      const bool ok = s0 < d.N && !d.bad;
#pragma unroll
      for (int row = 0; row < NR; ++row) {
        if (row >= p.rows) break;
        const float zs = ((sm.red[row][0][lane] + sm.red[row][1][lane]) + sm.red[row][2][lane]) +
                         sm.red[row][3][lane];
        const float zv = ok ? (KT == 0 ? zs * sc : zs) + 0.0f : 0.0f;
        p.z[((int64_t)d.r * p.rows + row) * p.z_ld + (int64_t)d.k * 64 + lane] = zv;
      }
      if (d.bad && lane == 0) raise_error(p.err, SPIN_DERR_PAGE);
    }
  }
}

// ---------------------------------------------------------------------------
// Single-row MFMA kernel: wave w owns slots 16w .. 16w+15 of every page and
// all 64 heads (the whole query tile in registers), so the head sum finishes
// inside the wave and a page needs one barrier (ring-slot hand-over) only.
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

  // Split the query into NS E4M3 terms per value after a per-head power-of-two
  // scaling (2^e amax in [128, 256)); 2^-e folds into the head weight.
  __device__ __forceinline__ void convert(const ScoreParams& p, int q_bf16, int rowid) {
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
    const int64_t qbase = (int64_t)rowid * 64;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float x[32];
      if (q_bf16) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            x[8 * v + 2 * c] = __uint_as_float(raw[t][v][c] << 16);
            x[8 * v + 2 * c + 1] = __uint_as_float(raw[t][v][c] & 0xFFFF0000u);
          }
      } else {
        load_q32(p.q, q_bf16, (qbase + 16 * t + m) * 128, g, x);
      }
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
        part[sp][t] = v8i{pw[sp][0], pw[sp][1], pw[sp][2], pw[sp][3],
                          pw[sp][4], pw[sp][5], pw[sp][6], pw[sp][7]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ei = __shfl(e, 4 * g + i, 64);
        wq[t][i] = ldexpf(wraw[t][i], -ei);
      }
    }
  }

  // this lane's ReLU-weighted sum over its 16 heads for the 16 slots whose
  // key bytes are in kf (MFMA B operand)
  __device__ __forceinline__ float dot(const v8i& kf) const {
    v4f acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int sp = 0; sp < NS; ++sp)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(part[sp][t], kf, acc[t], 0, 0, 0,
                                                                  127, 0, 127);
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) s = fmaf(wq[t][i], relu(acc[t][i]), s);
    return s;
  }

  // this lane's ReLU-weighted sum over its heads for slot `slot` of the page
  __device__ __forceinline__ float mul(const uint8_t* kbuf, int slot) const {
    const int g = (threadIdx.x & 63) >> 4;
    const v4u a = *reinterpret_cast<const v4u*>(kbuf + swz(slot, g, 128));
    const v4u b = *reinterpret_cast<const v4u*>(kbuf + swz(slot, 4 + g, 128));
    const v8i kf = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    v4f acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int sp = 0; sp < NS; ++sp)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(part[sp][t], kf, acc[t], 0, 0, 0,
                                                                  127, 0, 127);
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) s = fmaf(wq[t][i], relu(acc[t][i]), s);
    return s;
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

  __device__ __forceinline__ float mul(const uint8_t* kbuf, int slot) const {
    const int g = (threadIdx.x & 63) >> 4;
    v4u kb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kb[ks] = *reinterpret_cast<const v4u*>(kbuf + swz(slot, 4 * ks + g, 256));
    v4f acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, qa[t][ks]),
                                                         __builtin_bit_cast(v8bf, kb[ks]), acc[t],
                                                         0, 0, 0);
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) s = fmaf(wq[t][i], relu(acc[t][i]), s);
    return s;
  }
};

template <int KT, int NB>
struct SlotShared {
  uint8_t kbuf[NB][KGeo<KT>::kBytes] __attribute__((aligned(16)));
  float sbuf[NB][64];
  int tmp[32];
};

// G pages per iteration: one barrier, one descriptor step and one wait per
// group, and G x 8 independent MFMAs per wave between barriers.  The ring
// holds NB = G * D pages: one group being scored, D - 1 groups in flight.
template <int KT, int NS, int QB, int G, int D>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(3, 8))) void k_score_slots(ScoreParams p) {
  constexpr int NB = G * D;
  __shared__ SlotShared<KT, NB> sm;
  extern __shared__ int pre_dyn[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4;
  int n_ne;
  const ItemTable tb = build_items(p, pre_dyn, sm.tmp, pre_dyn + p.R + 1, &n_ne);
  int lo, hi, q_req;
  if (!request_range<G>(p, tb, pre_dyn + p.R + 1, n_ne, blockIdx.x, gridDim.x, lo, hi, q_req)) {
    // fewer workgroups than requests: contiguous runs of whole groups
    const int n_groups = (tb.total + G - 1) / G;
    const int per = (n_groups + gridDim.x - 1) / gridDim.x;
    lo = min(tb.total, (int)blockIdx.x * per * G);
    hi = min(tb.total, lo + per * G);
    q_req = -1;
  }
  if (lo >= hi) return;
  QFull<KT, NS> Q;
  // the first request's query loads fly together with the descriptor loads
  if (q_req >= 0) Q.fetch(p, QB, q_req);
  DescBatch db;  // cursor of the scoring stream
  db.init(p, tb, lo);
  if (q_req < 0) {
    q_req = __builtin_amdgcn_readfirstlane(db.mine.r);
    Q.fetch(p, QB, q_req);
  }
  DescBatch dd = db;  // cursor of the copy stream
  for (int i = 0; i < (D - 1) * G && lo + i < hi; ++i)
    Dma<KT>::issue(p, dd.get(p, tb, lo + i).page, sm.kbuf[i], sm.sbuf[i]);
  Q.convert(p, QB, q_req);  // while the first pages are in flight
  const int my_slot = 16 * wave + (lane & 15);  // page slot this lane scores
  int ring = 0;                                 // ring slot of group `it`
  for (int it = lo; it < hi; it += G) {
    const int cnt = min(G, hi - it);
    Desc d[G];
#pragma unroll
    for (int u = 0; u < G; ++u) d[u] = db.get(p, tb, min(it + u, hi - 1));
    const int issued_end = min(hi, it + (D - 1) * G);   // pages [it, issued_end) in flight
    wait_pages<KT, NB>(max(0, issued_end - (it + cnt)));
    __builtin_amdgcn_s_barrier();  // group visible; the previous group is no longer read
    // refill: the group D - 1 ahead goes where the previous group was
    const int ahead = it + (D - 1) * G;
    const int aring = (ring + (D - 1) * G) % NB;
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (ahead + u < hi)
        Dma<KT>::issue(p, dd.get(p, tb, ahead + u).page, sm.kbuf[(aring + u) % NB],
                       sm.sbuf[(aring + u) % NB]);
    float sv[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (u >= cnt) { sv[u] = 0.0f; continue; }
      if (d[u].r != q_req) { Q.load(p, QB, d[u].r); q_req = d[u].r; }  // rows == 1
      sv[u] = Q.mul(sm.kbuf[ring + u], my_slot);
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (u >= cnt) break;
      float s = sv[u];
      s += xor16(s);
      s += xor32(s);
      const float sc = KT == 0 ? sm.sbuf[ring + u][my_slot] : 1.0f;
      if (g == 0) {
        const int gslot = d[u].j * 64 + my_slot;
        const float zv = (gslot < d[u].N && !d[u].bad) ? (KT == 0 ? s * sc : s) + 0.0f : 0.0f;
        p.z[(int64_t)d[u].r * p.z_ld + (int64_t)d[u].k * 64 + my_slot] = zv;
      }
      if (d[u].bad && lane == 0 && wave == 0) raise_error(p.err, SPIN_DERR_PAGE);
    }
    ring = (ring + G) % NB;
  }
}


// ---------------------------------------------------------------------------
// fp8 keys, one verifier row: every wave scores whole pages on its own.
// A wave holds the request's whole query (64 heads, NS E4M3 terms), loads
// each page straight into registers (lane (n, g) holds the key bytes
// [16g, 16g + 16) and [64 + 16g, 64 + 16g + 16) of slots 16s + n, s = 0..3,
// the same dims its query registers hold) with P pages in flight, and runs
// 4 sub-tiles x 4 head tiles x NS MFMAs per page.  A reduce-scatter over the
// lane groups leaves lane l with slot l's total, which it scales and stores.
// No LDS staging and no barriers: waves progress independently.
// ---------------------------------------------------------------------------
template <int NS, int QB, int P, bool Span>
__global__ __launch_bounds__(256) void k_score_wave(ScoreParams p) {
  // Span: a wave's range may cross requests (fewer waves than requests), so
  // the query is reloaded inside the loop; without it (at least one wave per
  // request, ranges aligned to requests) the loop keeps no reload state and
  // the kernel fits two waves per SIMD
  extern __shared__ int pre_dyn[];
  __shared__ int tmp[32];
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int wave_id = blockIdx.x * 4 + (threadIdx.x >> 6), n_waves = gridDim.x * 4;
  int n_ne;
  const ItemTable tb = build_items(p, pre_dyn, tmp, pre_dyn + p.R + 1, &n_ne);
  int lo, hi, q_req;
  if (!request_range<1>(p, tb, pre_dyn + p.R + 1, n_ne, wave_id, n_waves, lo, hi, q_req)) {
    const int per = (tb.total + n_waves - 1) / n_waves;
    lo = min(tb.total, wave_id * per);
    hi = min(tb.total, lo + per);
    q_req = -1;
  }
  if (lo >= hi) return;  // no barrier follows
  QFull<0, NS> Q;
  if (q_req >= 0) Q.fetch(p, QB, q_req);
  DescBatch db;
  db.init(p, tb, lo);
  if (q_req < 0) {
    q_req = __builtin_amdgcn_readfirstlane(db.mine.r);
    Q.fetch(p, QB, q_req);
  }
  DescBatch dd = db;
  const uint8_t* kp = reinterpret_cast<const uint8_t*>(p.kp);
  // lane's byte offsets inside a page: sub-tile s, halves h
  const int off0 = n * 128 + 16 * g;
  v4u kb[P][8];
  float sc[P];
  const auto load_page = [&](int page, v4u (&b)[8], float& s) {
    const uint8_t* base = kp + (int64_t)page * 8192 + off0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      b[2 * t] = *reinterpret_cast<const v4u*>(base + t * 2048);
      b[2 * t + 1] = *reinterpret_cast<const v4u*>(base + t * 2048 + 64);
    }
    s = p.ks[(int64_t)page * 64 + lane];
  };
#pragma unroll
  for (int u = 0; u < P - 1; ++u) load_page(dd.get(p, tb, min(lo + u, hi - 1)).page, kb[u], sc[u]);
  Q.convert(p, QB, q_req);
  uint32_t hint = p.sink.hint ? p.sink.hint[q_req] : 0u;  // one row per request here
  int bad = 0;
  for (int it = lo; it < hi; it += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int cur = it + u;
      if (cur >= hi) break;
      // refill: page cur + P - 1 (the last page again past the end: an L2 hit)
      load_page(dd.get(p, tb, min(cur + P - 1, hi - 1)).page, kb[(u + P - 1) % P],
                sc[(u + P - 1) % P]);
      const Desc d = db.get(p, tb, cur);
      if (Span && d.r != q_req) {
        q_req = d.r;
        Q.load(p, QB, q_req);
        if (p.sink.hint) hint = p.sink.hint[q_req];
      }
      float part[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const v4u a = kb[u][2 * st], b2 = kb[u][2 * st + 1];
        const v8i kf = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w,
                           (int)b2.x, (int)b2.y, (int)b2.z, (int)b2.w};
        part[st] = Q.dot(kf);
      }
      const float tot = reduce_scatter4(part);
      const int slot = d.j * 64 + lane;
      const float zv = (slot < d.N && !d.bad) ? tot * sc[u] + 0.0f : 0.0f;
      p.z[(int64_t)d.r * p.z_ld + (int64_t)d.k * 64 + lane] = zv;
      bad |= d.bad;
      if (p.sink.hint) {  // top-K pre-filter: this block's slots at or above the hint
        const uint32_t key = float_key(zv);
        const bool pass = slot < d.N && key >= hint;
        const uint64_t m = __ballot(pass);
        const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (pass)
          p.sink.cand[(int64_t)d.r * p.sink.cand_ld + (int64_t)d.k * 64 + pos] =
              make_uint2(key, (uint32_t)slot);
        if (lane == 0) p.sink.pcnt[(int64_t)d.r * p.sink.pcnt_ld + d.k] = __popcll(m);
      }
    }
  }
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
template <int KT, int NS, int NR, int QB>
static void launch_mfma(const ScoreParams& p, hipStream_t st) {
  constexpr int NB = KT == 0 ? 6 : 4;
  const auto kern = k_score_mfma<KT, NS, NR, QB, NB>;
  const size_t dyn = sizeof(int) * 2 * (p.R + 1);
  const int g = min(resident_workgroups((const void*)kern, 256, dyn), p.R * p.max_blocks);
  hipLaunchKernelGGL(kern, dim3(g), dim3(256), dyn, st, p);
}

template <int KT, int NS, int QB>
static void launch_slots(const ScoreParams& p, hipStream_t st) {
  constexpr int G = 2, D = KT == 0 ? 3 : 2;
  const auto kern = k_score_slots<KT, NS, QB, G, D>;
  const size_t dyn = sizeof(int) * 2 * (p.R + 1);
  const int g = min(resident_workgroups((const void*)kern, 256, dyn), p.R * p.max_blocks);
  hipLaunchKernelGGL(kern, dim3(g), dim3(256), dyn, st, p);
}

template <int NS, int QB>
static void launch_wave(const ScoreParams& p, hipStream_t st) {
  constexpr int P = 2;  // pages in flight per wave (two waves per SIMD)
  const size_t dyn = sizeof(int) * 2 * (p.R + 1);
  const auto aligned = k_score_wave<NS, QB, P, false>;
  const int g = min(resident_workgroups((const void*)aligned, 256, dyn), p.R * p.max_blocks);
  if (4 * g >= p.R) {  // a wave per request at least: request-aligned ranges
    hipLaunchKernelGGL(aligned, dim3(g), dim3(256), dyn, st, p);
    return;
  }
  const auto span = k_score_wave<NS, QB, P, true>;
  const int g2 = min(resident_workgroups((const void*)span, 256, dyn), p.R * p.max_blocks);
  hipLaunchKernelGGL(span, dim3(g2), dim3(256), dyn, st, p);
}

template <int KT, int NS, int QB>
static void launch_rows(const ScoreParams& p, hipStream_t st) {
  if (p.rows <= 1 && KT == 0) launch_wave<NS, QB>(p, st);
  else if (p.rows <= 1) launch_slots<KT, NS, QB>(p, st);
  else if (p.rows <= 2) launch_mfma<KT, NS, 2, QB>(p, st);
  else launch_mfma<KT, NS, 4, QB>(p, st);
}

bool score_filters(const spin_config& c, const spin_batch& b) {
  return c.key_dtype == SPIN_FP8_E4M3 && b.n_rows == 1;  // the per-wave kernel
}

hipError_t launch_score(const spin_config& c, const spin_batch& b, const void* q, const float* w,
                        const void* kp, const float* ks, const int32_t* pt, int64_t pt_ld,
                        const int32_t* sel, const int32_t* n_sel, float* z, int64_t z_ld,
                        hipStream_t st, const CandSink* sink) {
  ScoreParams p{q, w, kp, ks, pt, pt_ld, sel, n_sel, b.ctx_len, b.q_pos, z, z_ld,
                b.batch, b.n_rows, b.max_blocks, b.n_pages, b.err, CandSink{}};
  if (sink && score_filters(c, b)) p.sink = *sink;
  if (c.key_dtype == SPIN_FP8_E4M3) {
    if (c.q_dtype == SPIN_BF16) launch_rows<0, 2, 1>(p, st);
    else launch_rows<0, 3, 0>(p, st);
  } else if (c.key_dtype == SPIN_BF16) {
    launch_rows<1, 1, 1>(p, st);
  } else {
    hipLaunchKernelGGL(k_score_f32, dim3(b.max_blocks, b.n_rows, b.batch), dim3(64), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace spin
