"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (one spin_step call per decode step through SpinLayer).

The whole batch runs on the GPU; at every step the oracle checks sampled
requests teacher-forced from the GPU's own state before the step:
  * block masks of every row: bit-exact (oracle predict + select on the
    pre-step V and D);
  * indexer scores: sampled slots of the selected blocks, scored one by one
    by the oracle, within the key dtype's tolerance and within the per-slot
    error bound of tests/score_bound.py;
  * top-K: bit-exact against the oracle's top-K of the GPU's fp32 scores;
  * EMA: V and D after the step bit-exact against the oracle's replay of the
    prefix-valid rows on the pre-step state with the GPU's scores.
"""
import numpy as np
import pytest
import torch

import spin_synth as G
from oracle import spin_oracle as O
from tests.gpu_util import DEV, KEY_TORCH, Q_TORCH, banner, z_close
from tests.score_bound import check_bound, score_bound

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-3, "fp8": 2e-2}
SAMPLE_SLOTS = 384


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_indexer_spin_amd import _lib
    return _lib.load()


def _sample_requests(R: int):
    return sorted({0, 1, R // 2, R - 1})


# More than 64 requests: the score kernel builds its item table in LDS, and
# with ~30 pages per wave its z queue fills and flushes mid-run.
_MANY_REQUESTS = {
    "fp8_72req_64k": lambda: G.WORKLOADS["fp8_128k_b32"].scaled(batch=72, n_slots=65536,
                                                                n_slots_min=40001),
    "bf16_72req_64k": lambda: G.WORKLOADS["bf16_64k_b16"].scaled(batch=72, n_slots=65536,
                                                                 n_slots_min=40001),
}


# every workload at its headline sparsity, and the bench workload at every
# point of the sparsity sweep
CASES = [(n, None) for n in ["fp8_128k_b32", "bf16_64k_b16", "fp8_128k_b32_mtp4",
                             "fp8_256k_ragged_8l", "fp8_72req_64k", "bf16_72req_64k"]] + \
    [("fp8_128k_b32", sp) for sp in (0, 2000, 3000, 5000)]


@pytest.mark.parametrize("name,sparsity", CASES)
def test_full_size_sampled_parity(name, sparsity):
    from sparse_attention_indexer_spin_amd import SpinLayer
    w = _MANY_REQUESTS[name]() if name in _MANY_REQUESTS else G.WORKLOADS[name]
    n_steps = 3
    sp = w.sparsity_bp[0] if sparsity is None else sparsity  # headline: 40 %
    banner(f"full size {name} sparsity_bp={sp}")
    layer = 0
    ctx = G.context_lengths(w)
    keys = G.make_keys(w, layer, DEV, ctx)
    W = G.make_weights(w, layer, DEV)
    pos, acc = G.make_schedule(w, ctx, n_steps)
    q = G.cast_queries(w, G.make_queries(w, layer, keys, pos, DEV)).contiguous()
    lay = SpinLayer(batch=w.batch, max_blocks=w.max_blocks, d_cap=G.d_capacity(w, n_steps),
                    topk=w.topk, sparsity_bp=sp, n_rows=w.rows, explore_bp=w.explore_bp,
                    ema_alpha=w.alpha, combine=w.combine, key_dtype=KEY_TORCH[w.key_dtype],
                    q_dtype=Q_TORCH[w.q_dtype], layer=layer, device=DEV)
    lay.set_requests(ctx.to(DEV), pos[0].to(DEV))
    lay.reset()
    acc_dev = acc.to(DEV)
    pt = keys.page_table.cpu().numpy()
    rng = np.random.default_rng(1234)
    worst_bound = 0.0
    for s in range(n_steps):
        torch.cuda.synchronize()
        V0, D0 = lay.V.cpu().numpy().copy(), lay.D.cpu().numpy().copy()
        t_before = lay.step_ctr.cpu().numpy().copy()
        qpos_before = lay.q_pos.cpu().numpy().copy()
        nv = acc[s].numpy() if w.rows > 1 else np.ones(w.batch, dtype=np.int64)
        lay.step(q[s], W, keys.pages, keys.scale, keys.page_table,
                 n_valid=acc_dev[s] if w.rows > 1 else None)
        torch.cuda.synchronize()
        assert int(lay.err.item()) == 0
        code = lay.row_code.cpu().numpy()
        sel, n_sel = lay.sel.cpu().numpy(), lay.n_sel.cpu().numpy()
        z = lay.z.cpu().numpy()
        top = lay.topk_idx.cpu().numpy()
        V1, D1 = lay.V.cpu().numpy(), lay.D.cpu().numpy()
        q_host = q[s].cpu()
        for r in _sample_requests(w.batch):
            N = int(ctx[r])
            B = O.n_blocks(N)
            qp = int(qpos_before[r])
            assert qp == int(pos[s, r])
            # stage 1-2: masks of every row, then their union
            rows_codes = []
            for row in range(w.rows):
                S = O.predict_block_scores(V0[r], D0[r], N, qp + row, w.combine)
                c = O.select_blocks(S, N, w.topk, sp, w.explore_bp, int(t_before[r]), layer, r,
                                    G.PHILOX_SEED)
                assert np.array_equal(code[r, row, :B], c), (name, s, r, row)
                rows_codes.append(c)
            blocks = O.union_blocks(rows_codes)
            assert n_sel[r] == len(blocks) and np.array_equal(sel[r, :n_sel[r]], blocks)
            if sp == 0 or s == 0:
                assert len(blocks) == B          # 0 % sparsity and the warm-up are dense
            slots = O.union_slots(blocks, N)
            comp = np.searchsorted(blocks, slots // 64) * 64 + slots % 64
            # stage 3a: sampled slots scored one by one
            pick = np.sort(rng.choice(slots.size, size=min(SAMPLE_SLOTS, slots.size),
                                      replace=False))
            ps = slots[pick]
            phys = torch.from_numpy(pt[r][ps // 64]).long().to(DEV)
            off = torch.from_numpy(ps % 64).to(DEV)
            raw = keys.pages[phys, off].cpu()
            if w.key_dtype == "fp8":
                k = O.decode_e4m3(raw.numpy())
                sc = keys.scale[phys, off].cpu().numpy().astype(np.float64)
            else:
                k = O.decode_bf16(raw.view(torch.int16).numpy().astype(np.uint16))
                sc = None
            qr = q_host[r]
            qn = qr.view(torch.int16).numpy().astype(np.uint16) if qr.dtype == torch.bfloat16 \
                else qr.numpy()
            qd = O.decode_q(qn, w.q_dtype)
            for row in range(w.rows):
                wr = W[r, row].cpu().numpy()
                want = O.index_scores(qd[row], wr, k if sc is None else k * sc[:, None])
                got = z[r, row, comp[pick]]
                ok, worst = z_close(got, want, TOL[w.key_dtype])
                assert ok, (name, s, r, row, worst)
                ok, worst = check_bound(got, want,
                                        score_bound(qd[row], wr, k, sc, w.key_dtype, w.q_dtype))
                assert ok, ("bound", name, s, r, row, worst)
                worst_bound = max(worst_bound, worst)
                # stage 3b: top-K of the GPU's fp32 scores over the whole domain
                want_top = O.topk_slots(z[r, row, comp], slots, w.topk)
                assert np.array_equal(top[r, row], want_top), (name, s, r, row)
            # stage 4: EMA replay of the prefix-valid rows on the pre-step state
            Vr, Dr = V0[r].copy(), D0[r].copy()
            O.ema_update(Vr, Dr, z[r][:, comp], slots, qp, int(nv[r]), w.alpha)
            assert np.array_equal(V1[r], Vr), (name, s, r)
            assert np.array_equal(D1[r], Dr), (name, s, r)
    banner(f"full size {name} sparsity_bp={sp}: requests {_sample_requests(w.batch)} x "
           f"{n_steps} steps checked; worst |dz| / bound = {worst_bound:.3f}")


@pytest.mark.parametrize("one_stream", [False, True])
def test_full_size_stack_with_budgets(one_stream):
    """The 8-layer ragged workload at full size through SpinStack with per-layer
    budgets (proportional rule, a probe every 2 steps): every step bit-identical
    to sequential spin_step layers given the same budgets; the probe's miss
    curves of sampled requests equal the oracle's; the allocation equals the
    oracle's on the summed curves."""
    from oracle import spin_budget as OB
    from sparse_attention_indexer_spin_amd import SpinLayer, SpinStack
    banner(f"full size stack + budgets fp8_256k_ragged_8l one_stream={one_stream}")
    w = G.WORKLOADS["fp8_256k_ragged_8l"]
    n_steps, sp, P, levels = 5, w.sparsity_bp[0], 2, 100
    ctx = G.context_lengths(w)
    pos, _ = G.make_schedule(w, ctx, n_steps)
    keys, W, Q = [], [], []
    for l in range(w.layers):
        k = G.make_keys(w, l, DEV, ctx)
        keys.append(k)
        W.append(G.make_weights(w, l, DEV))
        Q.append(G.cast_queries(w, G.make_queries(w, l, k, pos, DEV)).contiguous())

    def layers():
        out = []
        for l in range(w.layers):
            lay = SpinLayer(batch=w.batch, max_blocks=w.max_blocks,
                            d_cap=G.d_capacity(w, n_steps), topk=w.topk, sparsity_bp=sp,
                            explore_bp=w.explore_bp, ema_alpha=w.alpha, layer=l, device=DEV)
            lay.set_requests(ctx.to(DEV), pos[0].to(DEV))
            lay.reset()
            out.append(lay)
        return out

    seq, stk = layers(), layers()
    stack = SpinStack(stk, budget_policy="proportional", probe_period=P, levels=levels,
                      one_stream=one_stream)
    target = (10000 - sp) // 100
    Bs = [O.n_blocks(int(c)) for c in ctx]
    levels_now = [target] * w.layers
    checked = False
    for s in range(n_steps):
        probe = s > 0 and s % P == 0
        for l in range(w.layers):
            bud = [B if probe else OB.level_budget(B, w.topk, levels_now[l], levels) for B in Bs]
            seq[l].step(Q[l][s], W[l], keys[l].pages, keys[l].scale, keys[l].page_table,
                        budget=torch.tensor(bud, dtype=torch.int32, device=DEV))
        stack.step([Q[l][s] for l in range(w.layers)], W, [k.pages for k in keys],
                   [k.scale for k in keys], [k.page_table for k in keys])
        torch.cuda.synchronize()
        stack.side.synchronize()
        for l in range(w.layers):
            for a, b in ((seq[l].topk_idx, stk[l].topk_idx), (seq[l].V, stk[l].V),
                         (seq[l].D, stk[l].D), (seq[l].sel, stk[l].sel)):
                assert torch.equal(a, b), f"step {s} layer {l}"
        if not probe:
            continue
        cov = stack.covered.cpu().numpy()
        kp = stack.kprime.cpu().numpy()
        if not checked:
            for l in (0, w.layers - 1):
                S, top = stk[l].S.cpu().numpy(), stk[l].topk_idx.cpu().numpy()
                for r in _sample_requests(w.batch):
                    want, wk = OB.miss_curve(S[r, 0, :Bs[r]], top[r, 0], int(ctx[r]), w.topk,
                                             w.explore_bp, levels)
                    assert cov[l, r, 0].tolist() == want and kp[l, r, 0] == wk, (s, l, r)
            checked = True
        tot = kp.astype(np.int64).sum(axis=(1, 2))
        c = cov.astype(np.int64).sum(axis=(1, 2))
        miss = [0.0 if tot[l] == 0 else float(tot[l] - c[l][levels_now[l]]) / float(tot[l])
                for l in range(w.layers)]
        if s == P:
            want_levels = OB.allocate_proportional(miss, target, levels)
            assert stack.levels_now() == list(want_levels)
        levels_now = stack.levels_now()
    assert checked
    for lay in seq + stk:
        assert int(lay.err.item()) == 0
