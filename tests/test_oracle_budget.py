"""Pins of the per-layer budget oracle (oracle/spin_budget.py) against the
hand-worked example in tests/golden/budget_levels_hand.txt, the stage-2
block-selection oracle, monotonicity, and brute force over every allocation."""
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import spin_budget as OB
from oracle import spin_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "budget_levels_hand.txt")


def _golden():
    kv = {}
    for line in open(GOLD):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        kv[k.strip()] = v.split()
    return kv


def test_miss_curve_hand_example():
    g = _golden()
    S = np.array([float(x) for x in g["S"]])
    topk = np.array([int(x) for x in g["topk"]])
    N, K, lv = int(g["n_slots"][0]), int(g["K"][0]), int(g["levels"][0])
    cov0, kp = OB.miss_curve(S, topk, N, K, 0, lv)
    cov2, kp2 = OB.miss_curve(S, topk, N, K, 2000, lv)
    assert cov0 == [int(x) for x in g["covered_explore_0"]]
    assert cov2 == [int(x) for x in g["covered_explore_2000"]]
    assert kp == kp2 == int(g["kprime"][0])


def test_minimax_and_proportional_hand_examples():
    g = _golden()
    cov0 = [int(x) for x in g["covered_explore_0"]]
    assert OB.allocate_minimax([cov0, [0, 6, 6, 6, 6]], [8, 6], 2, 4) == \
        [int(x) for x in g["minimax_levels"]]
    miss = [float(x) for x in g["proportional_misses"]]
    assert OB.allocate_proportional(miss, 50, 100) == \
        [int(x) for x in g["proportional_levels"]]


@pytest.mark.parametrize("seed", range(6))
def test_miss_curve_counts_forced_and_ranked_blocks_of_the_selection(seed):
    """covered[g] = dense top-K slots in the blocks that the stage-2 oracle codes
    forced or ranked when run with that level's budget (an independent path:
    reason codes from select_blocks)."""
    rng = np.random.default_rng(seed)
    N = int(rng.integers(64 * 3, 64 * 40))
    B = O.n_blocks(N)
    S = rng.integers(0, 6, B).astype(np.float64)           # many ties
    K = int(rng.integers(8, 300))
    topk = np.sort(rng.choice(N, min(K, N), replace=False))
    topk = np.concatenate([topk, -np.ones(K - len(topk), dtype=np.int64)])
    levels, ex = 20, int(rng.choice([0, 500, 3000]))
    cov, kp = OB.miss_curve(S, topk, N, K, ex, levels)
    assert kp == int((topk >= 0).sum())
    for gl in range(levels + 1):
        m = OB.level_budget(B, K, gl, levels)
        code = O.select_blocks(S, N, K, 0, ex, step=5, layer=0, req_id=0, seed=1, budget=m)
        keep = np.nonzero((code == O.CODE_FORCED) | (code == O.CODE_RANKED))[0]
        want = int(np.isin(topk[topk >= 0] // 64, keep).sum())
        assert cov[gl] == want, (gl, cov[gl], want)
    assert all(a <= b for a, b in zip(cov, cov[1:]))
    if ex == 0:
        assert cov[levels] == kp                              # every block kept


def _miss(c, t):
    return Fraction(0) if t == 0 else Fraction(t - c, t)


@pytest.mark.parametrize("seed", range(8))
def test_minimax_is_optimal_by_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    L, levels = int(rng.integers(2, 4)), 6
    target = int(rng.integers(1, levels))
    total = [int(rng.integers(0, 20)) for _ in range(L)]
    covered = []
    for t in total:
        steps = np.sort(rng.integers(0, t + 1, levels + 1))  # non-decreasing
        covered.append([int(x) for x in steps])
    got = OB.allocate_minimax(covered, total, target, levels)
    assert sum(got) == L * target and all(0 <= x <= levels for x in got)
    best = min(max(_miss(covered[l][g[l]], total[l]) for l in range(L))
               for g in itertools.product(range(levels + 1), repeat=L) if sum(g) == L * target)
    assert max(_miss(covered[l][got[l]], total[l]) for l in range(L)) == best


def test_minimax_stops_at_the_top_level():
    # every layer at the top level before the target is reached
    assert OB.allocate_minimax([[0, 1, 2], [0, 1, 2]], [2, 2], 5, 2) == [2, 2]


def test_proportional_properties():
    assert OB.allocate_proportional([0.2, 0.2, 0.2, 0.2], 60, 100) == [60] * 4
    # one very hard layer is capped at the top level; the rest share the remainder
    # (140 levels over three equal weights: 46.67 each -> 46, plus one level to
    # each of the two lower layers on the tied fractional parts)
    assert OB.allocate_proportional([0.9, 0.01, 0.01, 0.01], 60, 100) == [100, 47, 47, 46]
    for seed in range(20):
        rng = np.random.default_rng(seed)
        L = int(rng.integers(1, 9))
        miss = rng.random(L) * rng.choice([0.01, 1.0])
        tgt = int(rng.integers(0, 101))
        g = OB.allocate_proportional(miss.tolist(), tgt, 100)
        assert sum(g) == L * tgt and all(0 <= x <= 100 for x in g)
        # harder layers never get fewer levels (up to the one-level rounding)
        order = np.argsort(miss)
        assert all(g[order[i]] <= g[order[i + 1]] + 1 for i in range(L - 1))


# Curves of the drift example (2 layers, 4 levels, K' = 10 each): the miss
# rates at levels 0..4 written out, then the covered counts they come from.
_P1 = ([0, 4, 7, 9, 10], [0, 2, 5, 8, 10])    # miss [1 .6 .3 .1 0], [1 .8 .5 .2 0]
_P2 = ([0, 5, 7, 9, 10], [0, 2, 4, 8, 10])    # miss [1 .5 .3 .1 0], [1 .8 .6 .2 0]
_P3 = ([0, 1, 2, 10, 10], [0, 2, 4, 8, 10])   # miss [1 .9 .8  0 0], [1 .8 .6 .2 0]


def test_budget_policy_drift_gate_minimax_hand_example():
    """Minimax on the hand-worked curves above (greedy raises, ties to the
    lower layer): probe 1 gives [2, 2]; probe 2 alone would give [1, 3] but
    moves no miss rate by more than 0.1, so a 0.15 threshold keeps [2, 2];
    probe 3 moves layer 0 by 0.5 at level 2 and is published: [3, 1].  With
    no threshold every probe is published."""
    gated = OB.BudgetPolicy("minimax", 2, 4, 2, drift_bp=1500)
    every = OB.BudgetPolicy("minimax", 2, 4, 2, drift_bp=0)
    want_gated = [([2, 2], True), ([2, 2], False), ([3, 1], True)]
    want_every = [([2, 2], True), ([1, 3], True), ([3, 1], True)]
    for cov, wg, we in zip((_P1, _P2, _P3), want_gated, want_every):
        assert gated.probe(list(cov), [10, 10]) == wg
        assert every.probe(list(cov), [10, 10]) == we


def test_budget_policy_drift_gate_keeps_the_running_means():
    """Proportional: a gated probe still adds each layer's miss rate at its
    current level to the running sums.  Probe 1 at the target levels [2, 2]
    adds (.3, .5) and publishes shares 4 * (.301, .501) / .802 = (1.50, 2.50)
    -> [1, 2] plus the larger fraction -> [2, 2]; probe 2 adds (.3, .6),
    drifts 0.1 and is not published."""
    pol = OB.BudgetPolicy("proportional", 2, 4, 2, drift_bp=1500)
    assert pol.probe(list(_P1), [10, 10]) == ([2, 2], True)
    assert pol.probe(list(_P2), [10, 10]) == ([2, 2], False)
    assert pol.n_probes == 2
    assert pol.miss_sum == pytest.approx([0.6, 1.1], abs=1e-15)
    assert pol.ref == [OB.miss_rates(c, 10) for c in _P1]


def test_budget_policy_full_threshold_publishes_only_the_first_probe():
    """Miss rates lie in [0, 1], so no drift exceeds a threshold of 10000 bp."""
    rng = np.random.default_rng(3)
    pol = OB.BudgetPolicy("minimax", 3, 8, 5, drift_bp=10000)
    for k in range(6):
        tot = rng.integers(1, 50, 3)
        cov = [np.minimum(np.cumsum(rng.integers(0, 5, 9)), t).tolist() for t in tot]
        for l in range(3):
            cov[l][-1] = int(tot[l])
        levels, published = pol.probe(cov, tot.tolist())
        assert published == (k == 0)
        assert sum(levels) == 15
