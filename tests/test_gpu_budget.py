"""Per-layer block budgets on the GPU: the miss-curve kernel and the budget
table fill against the oracle (exact integers), and multi-layer runs with
probes in which every step's outputs, every probe's miss curves and every
re-allocation match a reference driven by the oracle's budget functions."""
import numpy as np
import pytest
import torch

import spin_synth as G
from oracle import spin_budget as OB
from oracle import spin_oracle as O
from tests.gpu_util import DEV, banner, device_keys, make_layer
from tests.harness import build_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_indexer_spin_amd import _lib
    return _lib.load()


def _batch(ctx, rows, mb):
    from sparse_attention_indexer_spin_amd import api as A
    t = lambda x: torch.as_tensor(np.asarray(x), dtype=torch.int32, device=DEV)
    keep = dict(ctx=t(ctx), qpos=t([c + 3 for c in ctx]), step=t([5] * len(ctx)),
                req=t(np.arange(len(ctx))))
    bt = A.batch(ctx_len=keep["ctx"], q_pos=keep["qpos"], step=keep["step"], req_id=keep["req"],
                 n_rows=rows, max_blocks=mb, n_pages=1)
    return bt, keep


@pytest.mark.parametrize("mb,ctx", [(64, [4096, 4000, 130, 64]), (2048, [131072, 70001, 200]),
                                    (4096, [262144, 190000]), (8192, [524288, 300001])])
@pytest.mark.parametrize("levels,explore", [(4, 0), (100, 500), (100, 3000)])
@pytest.mark.parametrize("rows", [1, 2])
def test_miss_curve_parity(mb, ctx, levels, explore, rows):
    banner(f"miss curve mb={mb} levels={levels} explore={explore} rows={rows}")
    from sparse_attention_indexer_spin_amd import api as A
    R, K = len(ctx), 2048 if mb > 64 else 512
    ctx = list(ctx) + [64 * mb + 5]                       # plus one invalid request
    R += 1
    S = G.make_scores((R, rows, mb), seed=7 + mb + rows, ties=True)
    rng = np.random.default_rng(mb + levels + rows)
    topk = -np.ones((R, rows, K), dtype=np.int32)
    for r in range(R - 1):
        for row in range(rows):
            n = int(rng.integers(0, min(K, ctx[r]) + 1))
            topk[r, row, :n] = np.sort(rng.choice(ctx[r], n, replace=False))
    bt, keep = _batch(ctx, rows, mb)
    cfg = A.config(topk=K, sparsity_bp=4000, explore_bp=explore)
    cov = torch.full((R, rows, levels + 1), -3, dtype=torch.int32, device=DEV)
    kp = torch.full((R, rows), -3, dtype=torch.int32, device=DEV)
    A.spin_miss_curve(cfg, bt, S.to(DEV), torch.from_numpy(topk).to(DEV), levels, cov, kp)
    cov, kp = cov.cpu().numpy(), kp.cpu().numpy()
    for r in range(R - 1):
        for row in range(rows):
            want, wk = OB.miss_curve(S[r, row, :O.n_blocks(ctx[r])].numpy(), topk[r, row],
                                     ctx[r], K, explore, levels)
            assert cov[r, row].tolist() == want, (r, row)
            assert kp[r, row] == wk
    assert (cov[R - 1] == 0).all() and (kp[R - 1] == 0).all()


def test_budget_fill_parity():
    banner("budget fill")
    from sparse_attention_indexer_spin_amd import api as A
    ctx = [131072, 70001, 200, 64, 1]
    bt, keep = _batch(ctx, 1, 2048)
    cfg = A.config(topk=2048, sparsity_bp=4000)
    for levels in (4, 100):
        for g in sorted({0, 1, levels // 3, levels - 1, levels}):
            out = torch.full((len(ctx),), -1, dtype=torch.int32, device=DEV)
            A.spin_budget_fill(cfg, bt, torch.tensor([g], dtype=torch.int32, device=DEV), levels,
                               out)
            want = [OB.level_budget(O.n_blocks(c), 2048, g, levels) for c in ctx]
            assert out.cpu().tolist() == want, (levels, g)


@pytest.mark.parametrize("policy,one_stream,drift_bp", [("minimax", False, 0),
                                                        ("proportional", False, 0),
                                                        ("proportional", True, 0),
                                                        ("minimax", True, 300)])
def test_stack_budgets_match_oracle_reference(policy, one_stream, drift_bp):
    """SpinStack with probes every 3 steps, the policy run by the library
    (curves, allocation and budgets on the device, no host round trip),
    against sequential spin_step layers whose budgets come from the oracle:
    oracle miss curves of the same probe outputs, oracle allocation, applied
    from the step after the probe."""
    banner(f"stack budgets {policy} one_stream={one_stream} drift_bp={drift_bp}")
    from sparse_attention_indexer_spin_amd import SpinStack
    L, P, levels, sp = 3, 3, 100, 4000
    w = G.WORKLOADS["fp8_256k_ragged_8l"].scaled(batch=4, layers=L, n_slots=64 * 120 + 9,
                                                 n_slots_min=3000, steps=11, topk=256)
    lis = [build_layer(w, layer=l) for l in range(L)]
    keys = [device_keys(li) for li in lis]
    # the reference miss curves read each step's own block scores from S, so
    # the sequential layers do not predict ahead (the stack's probe steps do
    # not either)
    seq = [make_layer(li, sp, predict_ahead=False) for li in lis]
    stk = [make_layer(li, sp) for li in lis]
    stack = SpinStack(stk, budget_policy=policy, probe_period=P, levels=levels,
                      one_stream=one_stream, budget_drift_bp=drift_bp)
    target = (10000 - sp) // 100
    ref_levels, history = [target] * L, []
    ref = OB.BudgetPolicy(policy, L, levels, target, drift_bp=drift_bp)
    Bs = [O.n_blocks(int(c)) for c in lis[0].ctx]
    for s in range(w.steps):
        probe = s > 0 and s % P == 0
        qs = [li.q[s].to(DEV).contiguous() for li in lis]
        ws = [li.weights.to(DEV) for li in lis]
        for l in range(L):
            bud = [B if probe else OB.level_budget(B, w.topk, ref_levels[l], levels) for B in Bs]
            seq[l].step(qs[l], ws[l], *keys[l],
                        budget=torch.tensor(bud, dtype=torch.int32, device=DEV))
        stack.step(qs, ws, [k[0] for k in keys], [k[1] for k in keys], [k[2] for k in keys])
        torch.cuda.synchronize()
        stack.side.synchronize()
        for l in range(L):
            for a, b in ((seq[l].topk_idx, stk[l].topk_idx), (seq[l].V, stk[l].V),
                         (seq[l].D, stk[l].D), (seq[l].row_code, stk[l].row_code)):
                assert torch.equal(a, b), f"step {s} layer {l}"
        if not probe:
            continue
        cov, tot = [], []
        for l in range(L):
            S, top = seq[l].S.cpu().numpy(), seq[l].topk_idx.cpu().numpy()
            c_l, t_l = np.zeros(levels + 1, dtype=np.int64), 0
            for r in range(w.batch):
                c, k = OB.miss_curve(S[r, 0, :Bs[r]], top[r, 0], int(lis[l].ctx[r]), w.topk,
                                     w.explore_bp, levels)
                c_l += np.asarray(c)
                t_l += k
                assert stk_cov_row(stack, l, r) == c, (s, l, r)
            cov.append(c_l.tolist())
            tot.append(t_l)
        ref_levels, _ = ref.probe(cov, tot)
        assert stack.levels_now() == list(ref_levels), s
        history.append((s, list(ref_levels)))
    assert len(history) >= 2
    for lay in seq + stk:
        assert int(lay.err.item()) == 0


@pytest.mark.parametrize("policy", ["minimax", "proportional"])
@pytest.mark.parametrize("L,rows_total,levels", [(1, 5, 100), (3, 24, 100), (8, 50, 4),
                                                  (70, 7, 100)])
def test_budget_update_matches_oracle(policy, L, rows_total, levels):
    """spin_budget_update through the C ABI on random monotone curves (zero
    totals and ties included), three probes in a row (the proportional rule
    carries its running miss rates in the device state): the levels equal the
    oracle allocation every time."""
    banner(f"budget update {policy} L={L} rows={rows_total} levels={levels}")
    from sparse_attention_indexer_spin_amd import api as A
    rng = np.random.default_rng(L * 7 + rows_total)
    target = levels * 3 // 5
    state = torch.zeros(A.spin_budget_state_bytes(L, levels), dtype=torch.uint8, device=DEV)
    table = torch.full((L,), target, dtype=torch.int32, device=DEV)
    ref = OB.BudgetPolicy(policy, L, levels, target)
    for probe in range(3):
        kp = rng.integers(0, 300, (L, rows_total)).astype(np.int32)
        kp[0, :] = 0 if L > 2 and probe == 1 else kp[0, :]       # a layer with no top-K slots
        inc = rng.integers(0, 3, (L, rows_total, levels + 1))
        cov = np.minimum(np.cumsum(inc, axis=2), kp[:, :, None]).astype(np.int32)
        cov[:, :, -1] = kp                                       # the top level covers all
        A.spin_budget_update(policy, levels, target, torch.from_numpy(cov).to(DEV),
                             torch.from_numpy(kp).to(DEV), state, table)
        torch.cuda.synchronize()
        c_l = cov.astype(np.int64).sum(axis=1)
        t_l = kp.astype(np.int64).sum(axis=1)
        ref_levels, published = ref.probe(c_l.tolist(), t_l.tolist())
        assert published
        assert table.cpu().tolist() == ref_levels, probe
        assert sum(ref_levels) == L * target


@pytest.mark.parametrize("policy", ["minimax", "proportional"])
@pytest.mark.parametrize("L,levels,drift_bp", [(3, 100, 400), (8, 20, 1500), (40, 100, 250)])
def test_budget_update_drift_gate_matches_oracle(policy, L, levels, drift_bp):
    """With a drift threshold: eight probes whose curves move a little (at
    most half the threshold per level since the last large move) or, every
    third probe, a lot; the device publishes exactly when the oracle policy
    does, its level table equals the oracle's after every probe, and the
    running miss rates keep advancing across the probes it does not publish."""
    banner(f"budget drift gate {policy} L={L} levels={levels} drift={drift_bp}")
    from sparse_attention_indexer_spin_amd import api as A
    rng = np.random.default_rng(L * 31 + levels + drift_bp)
    rows_total = 6
    target = levels // 2
    state = torch.zeros(A.spin_budget_state_bytes(L, levels), dtype=torch.uint8, device=DEV)
    table = torch.full((L,), target, dtype=torch.int32, device=DEV)
    ref = OB.BudgetPolicy(policy, L, levels, target, drift_bp=drift_bp)
    tot = rng.integers(1000, 3000, L).astype(np.int64)     # a layer's top-K slots

    def curves():  # monotone from anywhere in [0, K'] up to K' at the top level
        c = np.sort(rng.integers(0, tot[:, None] + 1, (L, levels + 1)), axis=1)
        c[:, -1] = tot
        return c

    summed = curves()
    flags = []
    for probe in range(8):
        if probe % 3 == 2:
            summed = curves()                                # a large move
        else:
            # a small one: every miss rate moves by at most a quarter of the
            # threshold (the raised prefix maximum keeps the curve monotone)
            step = np.floor(tot * drift_bp / 40000.0).astype(np.int64)
            new = np.clip(summed + rng.integers(-1, 2, summed.shape) * step[:, None], 0,
                          tot[:, None])
            new[:, -1] = tot
            summed = np.maximum.accumulate(new, axis=1)
        # one row of each layer carries the layer's curve, the others are empty
        cov = np.zeros((L, rows_total, levels + 1), dtype=np.int32)
        kp = np.zeros((L, rows_total), dtype=np.int32)
        cov[:, 0, :] = summed
        kp[:, 0] = tot
        A.spin_budget_update(policy, levels, target, torch.from_numpy(cov).to(DEV),
                             torch.from_numpy(kp).to(DEV), state, table, drift_bp=drift_bp)
        torch.cuda.synchronize()
        ref_levels, published = ref.probe(summed.tolist(), tot.tolist())
        flags.append(published)
        assert table.cpu().tolist() == ref_levels, probe
    assert flags[0] and not all(flags) and sum(flags) >= 2, flags


def stk_cov_row(stack, l, r):
    return stack.covered[l, r, 0].cpu().tolist()
