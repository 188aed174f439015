"""The library's host-side budget allocation (spin_budget_allocate, no GPU)
against the oracle's, on random miss curves and running miss rates."""
import numpy as np
import pytest

from oracle import spin_budget as OB


@pytest.fixture(scope="module")
def api():
    import os
    from sparse_attention_indexer_spin_amd import _lib, api as A
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_attention_indexer_spin_amd import build
        build.build()
    return A


@pytest.mark.parametrize("seed", range(25))
def test_minimax_matches_oracle(api, seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 12))
    levels = int(rng.choice([4, 10, 20, 100]))
    target = int(rng.integers(0, levels + 1))
    total = rng.integers(0, 5000, L)
    if seed % 5 == 0:
        total[0] = 0
    cov = np.stack([np.sort(rng.integers(0, t + 1, levels + 1)) for t in total])
    want = OB.allocate_minimax(cov.tolist(), total.tolist(), target, levels)
    got = api.spin_budget_allocate("minimax", levels, target, covered=cov, total=total)
    assert got == want


@pytest.mark.parametrize("seed", range(25))
def test_proportional_matches_oracle(api, seed):
    rng = np.random.default_rng(1000 + seed)
    L = int(rng.integers(1, 12))
    levels = int(rng.choice([4, 10, 20, 100]))
    target = int(rng.integers(0, levels + 1))
    miss = rng.random(L) ** rng.choice([1, 3, 8])
    if seed % 4 == 0:
        miss[:] = miss[0]                                   # ties everywhere
    want = OB.allocate_proportional(miss.tolist(), target, levels)
    got = api.spin_budget_allocate("proportional", levels, target, running_miss=miss)
    assert got == want


def test_allocation_argument_errors(api):
    import ctypes as C
    from sparse_attention_indexer_spin_amd import _lib
    lib = _lib.load()
    out = (C.c_int32 * 2)()
    miss = (C.c_double * 2)(0.5, 0.25)
    assert lib.spin_budget_allocate(1, 2, 30, 10, None, None, miss, out) == 2   # 30 !| 10000
    assert lib.spin_budget_allocate(1, 0, 100, 10, None, None, miss, out) == 2  # no layers
    assert lib.spin_budget_allocate(1, 2, 100, 101, None, None, miss, out) == 2
    assert lib.spin_budget_allocate(0, 2, 100, 10, None, None, None, out) == 1  # needs curves
    assert lib.spin_budget_allocate(7, 2, 100, 10, None, None, miss, out) == 2  # policy
    bad = (C.c_double * 2)(0.5, 1.5)
    assert lib.spin_budget_allocate(1, 2, 100, 10, None, None, bad, out) == 2
    cov = (C.c_int64 * 6)(0, 1, 2, 0, 1, 9)                 # covered > total
    tot = (C.c_int64 * 2)(2, 3)
    assert lib.spin_budget_allocate(0, 2, 2, 1, cov, tot, None, out) == 2
    assert lib.spin_budget_allocate(1, 2, 100, 10, None, None, miss, out) == 0
    # the device update refuses a drift threshold outside [0, 10000] before
    # it touches any buffer
    for drift in (-1, 10001):
        assert lib.spin_budget_update(1, 2, 100, 10, drift, 4, None, None, None, None,
                                      None) == 2
