"""The design variants of spin_config.flags on the GPU against the oracle:
block pooling (max / top-4 / mean) stage by stage, and every variant closed
loop on integer-valued inputs, where all stages must match bit for bit."""
import numpy as np
import pytest
import torch

import spin_synth as G
from oracle import spin_oracle as O
from tests.gpu_util import DEV, banner, device_keys, make_layer
from tests.harness import build_layer, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_indexer_spin_amd import _lib
    return _lib.load()


@pytest.mark.parametrize("pooling", ["top4", "mean"])
@pytest.mark.parametrize("rows", [1, 3, 4])
@pytest.mark.parametrize("combine", ["max", "sum"])
def test_predict_pooling_parity(pooling, rows, combine):
    banner(f"predict pooling={pooling} rows={rows} combine={combine}")
    from sparse_attention_indexer_spin_amd import api as A
    ctx = [4096, 4000, 130, 66, 3, 1]
    mb = 64
    qpos = [c + 7 for c in ctx]
    V, D = G.make_ema_state(len(ctx), 64 * mb, 4096 + 64, seed=23, ties=True, zero_frac=0.2)
    t = lambda x: torch.as_tensor(np.asarray(x), dtype=torch.int32, device=DEV)
    keep = [t(ctx), t(qpos), t([3] * len(ctx)), t(np.arange(len(ctx)))]
    bt = A.batch(ctx_len=keep[0], q_pos=keep[1], step=keep[2], req_id=keep[3], n_rows=rows,
                 max_blocks=mb, n_pages=1)
    cfg = A.config(topk=512, sparsity_bp=4000, combine=combine, pooling=pooling)
    S = torch.full((len(ctx), rows, mb), -7.0, device=DEV)
    vmax = torch.full((len(ctx), mb), 1e30, device=DEV)    # must be ignored by these poolings
    A.spin_predict_blocks(cfg, bt, V.to(DEV), D.to(DEV), S, v_max=vmax)
    S = S.cpu().numpy()
    for r, N in enumerate(ctx):
        B = O.n_blocks(N)
        for row in range(rows):
            want = O.predict_block_scores(V[r].numpy(), D[r].numpy(), N, qpos[r] + row, combine,
                                          pooling=pooling)
            assert np.array_equal(S[r, row, :B], want), (r, row)
            assert (S[r, row, B:] == -7.0).all()


CLOSED = {
    "f32": G.WORKLOADS["tiny_f32_4k"].scaled(batch=2, n_slots=4096 + 100, n_slots_min=4000,
                                             steps=6),
    "fp8": G.WORKLOADS["fp8_128k_b32"].scaled(batch=3, n_slots=8192, n_slots_min=6000, steps=6,
                                              topk=512),
    "fp8_mtp": G.WORKLOADS["fp8_128k_b32_mtp4"].scaled(batch=3, n_slots=6000, n_slots_min=4500,
                                                       steps=6, topk=256),
}
VARIANTS = [
    ("f32", dict(pooling="mean")),
    ("fp8", dict(pooling="top4")),
    ("fp8", dict(pooling="mean")),
    ("fp8_mtp", dict(mtp_row0_mask=True)),
    ("fp8_mtp", dict(mtp_row0_update=True)),
    ("fp8_mtp", dict(explore_per_row=True)),
    ("fp8_mtp", dict(pooling="top4", mtp_row0_mask=True, mtp_row0_update=True,
                     explore_per_row=True)),
    # exploration policies (Sec. 4.6, "Staleness mitigation")
    ("fp8", dict(explore="age")),
    ("fp8", dict(explore="staleness")),
    ("fp8_mtp", dict(explore="staleness")),
    ("f32", dict(explore="age")),
    # block reductions (Sec. 4.6, "Block reduction")
    ("fp8", dict(reduction="A2")),
    ("fp8_mtp", dict(reduction="A2", pooling="top4")),
    ("f32", dict(reduction="A2", pooling="mean")),
    ("fp8", dict(reduction="A0")),
    ("fp8_mtp", dict(reduction="A0", explore="age")),
    ("f32", dict(reduction="A0", explore="staleness")),
]


@pytest.mark.parametrize("name,variants", VARIANTS)
@pytest.mark.parametrize("deferred", [False, True])
def test_variants_closed_loop_exact(name, variants, deferred):
    banner(f"variants closed loop {name} {variants} deferred={deferred}")
    w = CLOSED[name]
    li = build_layer(w, integer=True)
    sp = w.sparsity_bp[0]
    ref, st = run_oracle(li, w.steps, sp, **variants)
    lay = make_layer(li, sp, **variants)
    pages, scale, pt = device_keys(li)
    W = li.weights.to(DEV)
    for s in range(w.steps):
        q = li.q[s].to(DEV).contiguous()
        nv = li.accept[s].to(DEV)
        if deferred:
            lay.step(q, W, pages, scale, pt, n_valid=nv, defer_ema=True)
            lay.commit(nv)
        else:
            lay.step(q, W, pages, scale, pt, n_valid=nv)
        code = lay.row_code.cpu().numpy()
        sel, n_sel = lay.sel.cpu().numpy(), lay.n_sel.cpu().numpy()
        top = lay.topk_idx.cpu().numpy()
        for r in range(w.batch):
            x = ref[s][r]
            B = O.n_blocks(int(li.ctx[r]))
            assert np.array_equal(code[r, :, :B], x["codes"]), (s, r)
            assert n_sel[r] == len(x["sel"]) and np.array_equal(sel[r, :n_sel[r]], x["sel"])
            assert np.array_equal(top[r], x["topk"]), (s, r)
    Vg, Dg = lay.V.cpu().numpy(), lay.D.cpu().numpy()
    obs = lay.last_obs.cpu().numpy()
    for r in range(w.batch):
        N = int(li.ctx[r])
        assert np.array_equal(Vg[r, :N], st[r].V[:N])
        dl = min(Dg.shape[1], st[r].D.shape[0])
        assert np.array_equal(Dg[r, :dl], st[r].D[:dl])
        B = O.n_blocks(N)
        assert np.array_equal(obs[r, :B], st[r].last_obs[:B])
    assert int(lay.err.item()) == 0


def _bt(ctx, qpos, step, rows, mb):
    from sparse_attention_indexer_spin_amd import api as A
    t = lambda x: torch.as_tensor(np.asarray(x), dtype=torch.int32, device=DEV)
    keep = [t(ctx), t(qpos), t(step), t(np.arange(len(ctx)) * 3 + 1)]
    bt = A.batch(ctx_len=keep[0], q_pos=keep[1], step=keep[2], req_id=keep[3], n_rows=rows,
                 max_blocks=mb, n_pages=1)
    return bt, keep


@pytest.mark.parametrize("policy", ["age", "staleness"])
@pytest.mark.parametrize("rows,mb,ctx", [(1, 64, [4096, 4000, 130, 64, 1]),
                                         (4, 64, [4096, 2000, 65]),
                                         (1, 1000, [64000, 40001]),
                                         (3, 2048, [131072, 99999]),
                                         (1, 8192, [524288, 300001])])
def test_exploration_policy_select_parity(policy, rows, mb, ctx):
    """spin_select_blocks under the age and staleness policies: codes, the
    union and the updated last-observed steps bit-exact against the oracle,
    on scores and observation histories with many ties."""
    banner(f"select explore={policy} rows={rows} mb={mb}")
    from sparse_attention_indexer_spin_amd import api as A
    R, t = len(ctx), 37
    S = G.make_scores((R, rows, mb), seed=61, ties=True)
    g = torch.Generator().manual_seed(62)
    obs = torch.randint(0, 30, (R, mb), generator=g, dtype=torch.int32)
    bt, keep = _bt(ctx, [c + 3 for c in ctx], [t] * R, rows, mb)
    cfg = A.config(topk=2048 if mb > 64 else 512, sparsity_bp=4000, explore_bp=1000,
                   explore=policy)
    code = torch.full((R, rows, mb), 9, dtype=torch.uint8, device=DEV)
    sel = torch.full((R, mb), -5, dtype=torch.int32, device=DEV)
    n_sel = torch.zeros(R, dtype=torch.int32, device=DEV)
    obs_d = obs.to(DEV)
    A.spin_select_blocks(cfg, bt, S.to(DEV), code, sel, n_sel, last_obs=obs_d)
    code, sel, n_sel = code.cpu().numpy(), sel.cpu().numpy(), n_sel.cpu().numpy()
    obs_g = obs_d.cpu().numpy()
    for r, N in enumerate(ctx):
        B = O.n_blocks(N)
        rc = []
        for row in range(rows):
            want = O.select_blocks(S[r, row, :B].numpy(), N, cfg.topk, 4000, 1000, t, 0,
                                   r * 3 + 1, cfg.seed, explore=policy,
                                   last_obs=obs[r, :B].numpy())
            assert np.array_equal(code[r, row, :B], want), (r, row)
            rc.append(want)
        u = O.union_blocks(rc)
        assert n_sel[r] == len(u) and np.array_equal(sel[r, :len(u)], u)
        o = obs[r].numpy().copy()
        o[u] = t
        assert np.array_equal(obs_g[r], o), r


@pytest.mark.parametrize("rows", [1, 2, 4])
@pytest.mark.parametrize("combine", ["max", "sum"])
def test_a2_predict_and_ema_parity(rows, combine):
    """Block reduction A2 stage by stage: block scores from block-level V / D,
    and the block-level EMA from pooled scores with rows replayed in order --
    including query positions whose rows cross a 64-slot block boundary, so
    two blocks' updates meet on one block offset."""
    banner(f"A2 predict + EMA rows={rows} combine={combine}")
    from sparse_attention_indexer_spin_amd import api as A
    ctx = [4096, 4000, 130, 66, 1, 8191]
    qpos = [4096 + 62, 4000 + 5, 130 + 61, 66 + 63, 1 + 10, 8191 + 1]   # near boundaries
    R, mb = len(ctx), 128
    V, D = G.make_ema_state(R, 64 * mb, 8192 + 64, seed=71, ties=True, zero_frac=0.2)
    for pooling in ("max", "top4", "mean"):
        bt, keep = _bt(ctx, qpos, [3] * R, rows, mb)
        cfg = A.config(topk=512, sparsity_bp=4000, combine=combine, pooling=pooling,
                       reduction="A2", ema_alpha=0.9)
        S = torch.full((R, rows, mb), -7.0, device=DEV)
        A.spin_predict_blocks(cfg, bt, V.to(DEV), D.to(DEV), S)
        S = S.cpu().numpy()
        for r, N in enumerate(ctx):
            B = O.n_blocks(N)
            for row in range(rows):
                want = O.predict_block_scores_a2(V[r].numpy(), D[r].numpy(), N, qpos[r] + row,
                                                 combine)
                assert np.array_equal(S[r, row, :B], want), (pooling, r, row)
        sel, n_sel = G.make_selection(R, torch.tensor([O.n_blocks(c) for c in ctx]), mb, 0.5,
                                      seed=72)
        zin = G.make_scores((R, rows, 64 * mb), seed=73)
        g = torch.Generator().manual_seed(74)
        n_valid = torch.randint(1, rows + 1, (R,), generator=g, dtype=torch.int32)
        Vd, Dd = V.to(DEV), D.to(DEV)
        A.spin_ema_update(cfg, bt, zin.to(DEV), sel.to(DEV), n_sel.to(DEV), Vd, Dd,
                          n_valid=n_valid.to(DEV))
        Vg, Dg = Vd.cpu().numpy(), Dd.cpu().numpy()
        for r, N in enumerate(ctx):
            blocks = sel[r, :int(n_sel[r])].numpy()
            slots = O.union_slots(blocks, N)
            comp = np.searchsorted(blocks, slots // 64) * 64 + slots % 64
            v, d = V[r].numpy().copy(), D[r].numpy().copy()
            O.ema_update_a2(v, d, zin[r].numpy()[:, comp], blocks, N, qpos[r], int(n_valid[r]),
                            0.9, pooling)
            assert np.array_equal(Vg[r], v), (pooling, r)
            assert np.array_equal(Dg[r], d), (pooling, r)
        assert int(keep[0].numel()) == R
