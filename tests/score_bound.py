"""Rigorous per-slot error bounds for the MFMA indexer scores (test helper).

The score z = scale * sum_h w_h ReLU(q_h . k) is computed on the matrix cores
from exactly decoded keys; what separates the GPU's fp32 value from the fp64
value of the same inputs is, per head h,
  * the query's representation: for fp8 keys each head's query is scaled by a
    power of two 2^e_h (2^e_h amax_h in [128, 256)) and written as a sum of
    E4M3 terms (two for bf16 queries, three for fp32 queries).  After the last
    term the residual is at most half the E4M3 subnormal quantum, 2^-10 in
    scaled units, or for fp32 queries also 2^-12 of the element (three terms
    of four significant bits).  bf16 keys use the bf16 query as it is.
  * the accumulation of n exact products (fp8 x fp8 and bf16 x bf16 products
    are exact in fp32) in fp32 in an unspecified order: at most gamma_n times
    the sum of |products|, gamma_n = n u / (1 - n u); u = 2^-23 covers
    truncating as well as rounding adders;
  * the head sum over 64 heads, each step possibly a separate multiply and
    add: gamma_128 of sum_h w_h |r_h| plus (1 + gamma_128) times the head
    errors (ReLU is 1-Lipschitz);
  * the scale multiply and the store: two more roundings of |z|.
A lost query term (e.g. only the first E4M3 term) breaks this bound by orders
of magnitude; the CPU test of this helper checks that it does.
"""
from __future__ import annotations

import numpy as np

U = 2.0 ** -23


def gamma(n: int, u: float = U) -> float:
    return n * u / (1 - n * u)


def head_exponents(q: np.ndarray) -> np.ndarray:
    """e_h with 2^e_h amax_h in [128, 256) (0 for an all-zero head)."""
    amax = np.abs(q).max(axis=-1)
    e = np.zeros_like(amax, dtype=np.int64)
    nz = amax > 0
    e[nz] = 7 - np.floor(np.log2(amax[nz])).astype(np.int64)
    return e


def score_bound(q: np.ndarray, w: np.ndarray, k: np.ndarray, scale, key_dtype: str,
                q_dtype: str) -> np.ndarray:
    """Per-slot bound on |z_gpu - z_exact|.

    q: [n_h, d] decoded query (fp64), w: [n_h], k: [n, d] decoded keys WITHOUT
    the per-slot scale, scale: [n] (fp8) or None."""
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n_h, d = q.shape
    ak, aq = np.abs(k), np.abs(q)
    absdot = ak @ aq.T                                     # [n, n_h] sum_c |q_c k_c|
    if key_dtype == "fp8":
        n_terms = 2 if q_dtype == "bf16" else 3
        e = head_exponents(q)
        dq = np.broadcast_to((2.0 ** -10 * 2.0 ** (-e))[:, None], q.shape)
        if q_dtype == "f32":
            dq = np.maximum(dq, aq * 2.0 ** -12)
        rep = ak @ dq.T                                    # query representation
        acc = gamma(n_terms * d) * (1 + 2.0 ** -3) * absdot
        ds = rep + acc
    elif key_dtype == "bf16":
        ds = gamma(d) * absdot
    else:
        raise ValueError(key_dtype)
    r = np.maximum(k @ q.T, 0.0)
    z = r @ w
    b = (1 + gamma(128)) * (ds @ w) + gamma(128) * z
    if scale is not None:
        s = np.asarray(scale, dtype=np.float64)
        b, z = b * s, z * s
    return b + 2 * U * np.abs(z) + 1e-30


def check_bound(z_gpu, z_exact, bound):
    """(ok, worst |dz| / bound)."""
    dz = np.abs(np.asarray(z_gpu, dtype=np.float64) - np.asarray(z_exact, dtype=np.float64))
    ratio = dz / bound
    worst = float(ratio.max()) if ratio.size else 0.0
    return worst <= 1.0, worst
