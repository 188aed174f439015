"""CPU checks of the per-slot score bound the GPU parity tests assert
(tests/score_bound.py): it holds for a host model of the fp8 path's query
split, and a query carried by its first E4M3 term alone breaks it by orders
of magnitude, so the bound pins that the query is carried at bf16 precision
(for fp32 queries the bound allows 2^-12 of each element, the precision of
three terms)."""
import numpy as np
import torch

from oracle import spin_oracle as O
from tests.score_bound import check_bound, head_exponents, score_bound


def _e4m3(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to E4M3 (round to nearest even) with torch's cast."""
    return torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).to(
        torch.float32).numpy()


def _split(q: np.ndarray, n_terms: int) -> np.ndarray:
    """Query as the sum of its E4M3 terms after the per-head power-of-two scaling."""
    e = head_exponents(q)
    x = (q * 2.0 ** e[:, None]).astype(np.float32)
    rep = np.zeros_like(x, dtype=np.float64)
    for _ in range(n_terms):
        t = _e4m3(x)
        rep += t
        x = (x - t).astype(np.float32)
    return rep * 2.0 ** (-e[:, None])


def _inputs(q_dtype, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((64, 128)) * rng.uniform(0.1, 10, (64, 1))
    q[3] *= 1e-3                       # a head far below the others
    q[5, :8] *= 1e-4                   # elements far below their head's amax
    if q_dtype == "bf16":
        q = torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    else:
        q = q.astype(np.float32).astype(np.float64)
    codes = rng.integers(0, 256, (300, 128)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x30
    k = O.decode_e4m3(codes)
    scale = rng.uniform(0.001, 0.02, 300)
    w = rng.uniform(0.5, 1.5, 64)
    return q, w, k, scale


def test_bound_holds_for_split_query_and_catches_a_lost_term():
    for q_dtype, n_terms in (("bf16", 2), ("f32", 3)):
        q, w, k, scale = _inputs(q_dtype, 7)
        exact = O.index_scores(q, w, k) * scale
        b = score_bound(q, w, k, scale, "fp8", q_dtype)
        ok, worst = check_bound(O.index_scores(_split(q, n_terms), w, k) * scale, exact, b)
        assert ok, (q_dtype, worst)
        ok, worst = check_bound(O.index_scores(_split(q, 1), w, k) * scale, exact, b)
        assert not ok and worst > (30 if q_dtype == "bf16" else 3), (q_dtype, worst)
    # the bound is far inside the 2e-2 relative contract
    q, w, k, scale = _inputs("bf16", 8)
    exact = O.index_scores(q, w, k) * scale
    rel = score_bound(q, w, k, scale, "fp8", "bf16") / np.maximum(exact, 1e-3 * np.sqrt(
        np.mean(exact ** 2)))
    assert np.median(rel) < 1e-3


def test_bound_holds_for_fp32_accumulation_bf16_keys():
    rng = np.random.default_rng(9)
    q = torch.randn(64, 128, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn(500, 128, dtype=torch.float32).to(torch.bfloat16)
    w = rng.uniform(0.5, 1.5, 64)
    qd, kd = q.to(torch.float64).numpy(), k.to(torch.float64).numpy()
    exact = O.index_scores(qd, w, kd)
    # fp32 products and fp32 sums in one fixed order (a model of the MFMA path)
    dots = (k.float() @ q.float().T).numpy()
    z32 = (np.maximum(dots, 0).astype(np.float32) @ w.astype(np.float32)).astype(np.float32)
    ok, worst = check_bound(z32, exact, score_bound(qd, w, kd, None, "bf16", "bf16"))
    assert ok, worst
