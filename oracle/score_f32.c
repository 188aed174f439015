/*
 * Exact-fp32 indexer score for the CPU oracle -- TEST INFRASTRUCTURE ONLY.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this file's library (through oracle/score_f32.py); the product path never
 * does.  It shares no code with the HIP library.
 *
 * The indexer score of the paper ("SPIN: Shadow Predictive Indexer for Sparse
 * Attention", Sec. 2; Algorithm 1, the Indexer step) is
 *     z[i] = sum_h w_h * ReLU(q_h . k_i).
 * The pages leave the floating-point evaluation open.  For fp32 keys and fp32
 * queries the exact mode fixes one canonical fp32 evaluation, so that every
 * integer decision downstream (block masks, top-K, exploration) and the EMA
 * state can be compared bit for bit:
 *     for each head h:  s = +0; for c = 0 .. d-1: s = fmaf(q[h][c], k[i][c], s)
 *                       r_h = s > 0 ? s : +0
 *     z = +0; for h = 0 .. n_h-1: z = fmaf(w[h], r_h, z)
 * fmaf is the C99 fused multiply-add: q*k + s with ONE rounding to fp32 (round
 * to nearest, ties to even).  Built with -ffp-contract=off so that nothing
 * else is fused or reassociated.
 */
#include <math.h>
#include <stdint.h>

/* q: [n_h][d] fp32, w: [n_h] fp32, keys: [n][d] fp32 rows, z: [n] fp32 out. */
void oracle_score_f32(const float* q, const float* w, const float* keys, int64_t n, int n_h,
                      int d, float* z) {
  for (int64_t i = 0; i < n; ++i) {
    const float* k = keys + i * (int64_t)d;
    float acc = 0.0f;
    for (int h = 0; h < n_h; ++h) {
      const float* qh = q + (int64_t)h * d;
      float s = 0.0f;
      for (int c = 0; c < d; ++c) s = fmaf(qh[c], k[c], s);
      const float r = s > 0.0f ? s : 0.0f;
      acc = fmaf(w[h], r, acc);
    }
    z[i] = acc + 0.0f; /* -0 -> +0 */
  }
}

/* One fused multiply-add, exposed so the tests can pin fmaf itself. */
float oracle_fmaf(float a, float b, float c) { return fmaf(a, b, c); }
