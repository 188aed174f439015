"""Plain CPU oracle of SPIN's per-layer block budgets.

TEST INFRASTRUCTURE ONLY: imported by tests/ and the benchmark's CPU leg,
never by the product path.  It shares no code with the HIP library.

Source: the project blog "Sparse Attention Still Has a Dense Problem",
section "Per-layer block budgets": the miss rate of a layer is the share of
the dense indexer's top-K slots that fall into skipped blocks; every P decode
steps a dense probe step scores all blocks and measures each layer's miss
curve (its miss rate at each budget); the budgets are sized per layer so that
the total over all layers stays at the user's target block sparsity, choosing
the allocation that minimises the worst layer's miss rate; the result is
published to a table on the device.  The multi-layer workload of this build
states a second rule: each layer's budget in proportion to its running top-K
miss rate.

Readings where the pages are silent (each is listed in the design doc):
  * A budget is a level g in 0 .. levels: it keeps the budget the block
    selection computes for target sparsity 10000 - (10000 / levels) * g basis
    points (so with 100 levels, g percent of the blocks, at least ceil(K/64)).
  * The miss curve counts the blocks the selection keeps deterministically
    at a level: the forced blocks and the ranked ones (predicted score
    descending, lower block first).  Exploration draws are random and are not
    counted.  Summed over the requests of a layer: covered[g] and the number
    of valid dense top-K slots K'.
  * Minimax: start every layer at level 0 and raise, one level at a time, the
    layer whose current miss rate is the largest (ties: lower layer; layers
    already at the top level are skipped) until the levels sum to
    n_layers * target_level.
  * Proportional: shares T * w_l / sum(w) with w_l = miss_l + 1e-3 and
    T = n_layers * target_level, clamped to [0, levels] (clamped layers are
    fixed and the rest re-shared, until no share leaves the range); integer
    parts, then one more level to the largest fractional parts (ties: lower
    layer) until the sum is T.  The running miss rate of a layer is the mean
    of its miss rates at the levels it ran at, over the probes so far.
  * Drift: the table is re-sized when some layer's miss rate at some level
    moved by more than a threshold since the curves of the last publication
    (BudgetPolicy); a zero threshold re-sizes at every probe.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .spin_oracle import BLOCK, block_budget, n_blocks, rank_desc


def level_sparsity_bp(g: int, levels: int) -> int:
    assert 10000 % levels == 0 and 0 <= g <= levels
    return 10000 - (10000 // levels) * g


def level_budget(B: int, K: int, g: int, levels: int) -> int:
    """Blocks kept at level g (the block selection's budget rule)."""
    return block_budget(B, K, level_sparsity_bp(g, levels))


def miss_curve(S, topk, n_slots: int, K: int, explore_bp: int, levels: int):
    """(covered[0..levels], K') of one request of one layer.

    S: predicted block scores of the probe step; topk: the dense top-K slot
    ids of that step (-1 padded)."""
    B = n_blocks(n_slots)
    c = np.zeros(B, dtype=np.int64)
    kprime = 0
    for i in np.asarray(topk).tolist():
        if i >= 0:
            c[i // BLOCK] += 1
            kprime += 1
    forced = sorted({0, B - 1})
    n_f = len(forced)
    rest = [j for j in range(B) if j not in forced]
    order = rank_desc(np.asarray(S, dtype=np.float64), rest).tolist()
    covered = []
    for g in range(levels + 1):
        m = max(level_budget(B, K, g, levels), n_f)
        n_e = min(m * int(explore_bp) // 10000, m - n_f)
        n_r = m - n_f - n_e
        keep = forced + order[:n_r]
        covered.append(int(c[keep].sum()))
    return covered, kprime


def _miss(cov: int, total: int) -> Fraction:
    return Fraction(0) if total == 0 else Fraction(total - cov, total)


def allocate_minimax(covered, total, target_level: int, levels: int):
    """Levels per layer minimising the largest miss rate (greedy, see above).

    covered: [L][levels + 1] ints, total: [L] ints."""
    L = len(total)
    g = [0] * L
    budget = L * int(target_level)
    while sum(g) < budget:
        best = -1
        for l in range(L):
            if g[l] >= levels:
                continue
            if best < 0 or _miss(covered[l][g[l]], total[l]) > _miss(covered[best][g[best]],
                                                                    total[best]):
                best = l
        if best < 0:
            break
        g[best] += 1
    return g


def allocate_proportional(miss, target_level: int, levels: int):
    """Levels per layer proportional to miss_l + 1e-3 (see above)."""
    L = len(miss)
    T = L * int(target_level)
    w = [float(m) + 1e-3 for m in miss]
    fixed = [None] * L
    while True:
        free = [l for l in range(L) if fixed[l] is None]
        rem = T - sum(v for v in fixed if v is not None)
        ws = sum(w[l] for l in free)
        share = {l: rem * w[l] / ws for l in free} if free else {}
        changed = False
        for l in free:
            if share[l] > levels:
                fixed[l] = levels
                changed = True
            elif share[l] < 0:
                fixed[l] = 0
                changed = True
        if not changed:
            break
    g = [0] * L
    frac = []
    for l in range(L):
        if fixed[l] is not None:
            g[l] = fixed[l]
        else:
            g[l] = int(np.floor(share[l]))
            frac.append((share[l] - g[l], l))
    left = T - sum(g)
    frac.sort(key=lambda x: (-x[0], x[1]))
    for _, l in frac:
        if left <= 0:
            break
        if g[l] < levels:
            g[l] += 1
            left -= 1
    return g


def miss_rates(covered_l, total_l):
    """One layer's miss rate at every level, in binary64: (K' - covered[g]) / K'
    (0 for a layer without top-K slots)."""
    t = int(total_l)
    return [0.0 if t == 0 else float(t - int(c)) / float(t) for c in covered_l]


class BudgetPolicy:
    """The policy across probes (the pages: a background computation re-sizes
    the budgets whenever the miss curves drift and publishes them to a table).

    Reading: at every probe,
      * the proportional rule adds each layer's miss rate at the level it ran
        at to its running sum (the probe count grows by one);
      * the levels are re-sized and published when drift_bp == 0, at the
        first probe, or when some layer's miss rate at some level differs by
        more than drift_bp / 10000 from the curves of the last publication;
        otherwise the table keeps its levels.  The published curves become
        the new reference.
    Minimax re-sizes from the probe's curves, proportional from the running
    means."""

    def __init__(self, policy: str, n_layers: int, levels: int, target_level: int,
                 drift_bp: int = 0):
        assert policy in ("minimax", "proportional") and 0 <= drift_bp <= 10000
        self.policy, self.L, self.levels = policy, int(n_layers), int(levels)
        self.target, self.drift_bp = int(target_level), int(drift_bp)
        self.level_now = [self.target] * self.L
        self.miss_sum = [0.0] * self.L
        self.n_probes = 0
        self.ref = None

    def probe(self, covered, total):
        """covered: [L][levels + 1] ints, total: [L] ints (summed over the
        layer's requests and rows).  Returns (levels, published)."""
        cur = [miss_rates(covered[l], total[l]) for l in range(self.L)]
        if self.policy == "proportional":
            self.n_probes += 1
            for l in range(self.L):
                self.miss_sum[l] += cur[l][self.level_now[l]]
        publish = self.drift_bp == 0 or self.ref is None
        if not publish:
            drift = max(abs(a - b) for l in range(self.L) for a, b in zip(cur[l], self.ref[l]))
            publish = drift > self.drift_bp / 10000
        if publish:
            if self.policy == "minimax":
                self.level_now = allocate_minimax(covered, total, self.target, self.levels)
            else:
                self.level_now = allocate_proportional(
                    [m / self.n_probes for m in self.miss_sum], self.target, self.levels)
            self.ref = cur
        return list(self.level_now), publish
