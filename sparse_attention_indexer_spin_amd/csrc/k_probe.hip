// HBM read probe over KV pages with the fp8 score kernel's access pattern
// (a measurement helper, not a stage of the method): whole 8 KB pages by
// 16-byte non-temporal loads (lane l: bytes (l & 7) 128 + ((l >> 3) & 1) 64
// + (l >> 4) 16 of every KB, as the score kernel's whole-line page loads),
// two pages in flight per wave, each wave a contiguous run of the list.
#include "spin_launch.h"
#include "spin_probe.h"

namespace spin {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void probe_load(const uint8_t* kp, int64_t n_pages, int id,
                                           v4u (&b)[8]) {
  const int lane = threadIdx.x & 63;
  const int64_t page = (id >= 0 && id < n_pages) ? id : 0;
  const uint8_t* base = kp + page * 8192 + (lane & 7) * 128 + ((lane >> 3) & 1) * 64 +
                        (lane >> 4) * 16;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    b[i] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(base + i * 1024));
}

__device__ __forceinline__ uint32_t probe_fold(const v4u (&b)[8], uint32_t acc) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc ^= b[i].x ^ b[i].y ^ b[i].z ^ b[i].w;
  return acc;
}

__global__ __launch_bounds__(256) void k_read_pages(const uint8_t* __restrict__ kp,
                                                    int64_t n_pages,
                                                    const int32_t* __restrict__ ids, int n,
                                                    uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int w = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  const int lo = (int)((int64_t)w * n / SPIN_READ_PROBE_WAVES);
  const int hi = (int)((int64_t)(w + 1) * n / SPIN_READ_PROBE_WAVES);
  uint32_t acc = 0u;
  v4u a[8], b[8];
  int base = lo, mine = 0;  // the ids of items base .. base + 63, one per lane
  const auto id_of = [&](int k) {
    if (k - base >= 64) {
      base = k;
      mine = ids[min(base + lane, n - 1)];
    }
    return __builtin_amdgcn_readlane(mine, k - base);
  };
  if (lo < hi) {
    mine = ids[min(base + lane, n - 1)];
    probe_load(kp, n_pages, id_of(lo), a);
    for (int it = lo; it < hi; it += 2) {
      if (it + 1 < hi) probe_load(kp, n_pages, id_of(it + 1), b);
      acc = probe_fold(a, acc);
      if (it + 1 >= hi) break;
      if (it + 2 < hi) probe_load(kp, n_pages, id_of(it + 2), a);
      acc = probe_fold(b, acc);
    }
  }
  sink[(int64_t)w * 64 + lane] = acc;
}

hipError_t launch_read_pages(const void* kp, int64_t n_pages, const int32_t* ids, int n,
                             uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL(k_read_pages, dim3(SPIN_READ_PROBE_WAVES / 4), dim3(256), 0, st,
                     static_cast<const uint8_t*>(kp), n_pages, ids, n, sink);
  return hipGetLastError();
}

}  // namespace spin
