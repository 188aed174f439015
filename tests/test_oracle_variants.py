"""Pins of the oracle's design variants (the paper's ablations): block pooling
(Sec. 4.6), row-0 mask sharing, row-0 EMA update and per-row exploration draws
(Sec. 4.5 and Q11 of the readings)."""
import os

import numpy as np
import pytest

from oracle import spin_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "pooling_hand.txt")


def _golden():
    kv = {}
    for line in open(GOLD):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        kv[k.strip()] = [float(x) for x in v.split()]
    return kv


def test_pooling_hand_example():
    g = _golden()
    N = int(g["n_slots"][0])
    V = np.zeros(N, dtype=np.float32)
    V[:64] = np.arange(64, dtype=np.float32) / 8
    V[64:66] = g["block1_values"]
    D = np.zeros(N + 8, dtype=np.float32)
    for pool in ("max", "top4", "mean"):
        S = O.predict_block_scores(V, D, N, N + 1, "max", pooling=pool)
        assert S.tolist() == g[pool], pool


@pytest.mark.parametrize("seed", range(10))
def test_pooling_against_fp64_definitions(seed):
    """top4 and mean are the fp64 means of their definition up to fp32
    rounding of the sums; max is unchanged by the variant machinery."""
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 64 * 9))
    V = (rng.random(N + 70) * rng.choice([1.0, 100.0])).astype(np.float32)
    D = (rng.random(N + 70) * 3).astype(np.float32)
    q = N + 2
    zhat = np.maximum(V[:N], D[q - np.arange(N)]).astype(np.float64)
    Smax = O.predict_block_scores(V, D, N, q, "max")
    S4 = O.predict_block_scores(V, D, N, q, "max", pooling="top4")
    Sm = O.predict_block_scores(V, D, N, q, "max", pooling="mean")
    for j in range(O.n_blocks(N)):
        blk = zhat[64 * j:min(64 * j + 64, N)]
        assert Smax[j] == np.float32(blk.max())
        want4 = np.sort(blk)[::-1][:4].mean()
        assert abs(S4[j] - want4) <= 4e-7 * want4 + 1e-30
        assert abs(Sm[j] - blk.mean()) <= 4e-6 * blk.mean() + 1e-30
        assert Sm[j] <= Smax[j] and S4[j] <= Smax[j] and S4[j] >= Sm[j] - 1e-6 * Smax[j]


def _step_inputs(rows=3, seed=0):
    rng = np.random.default_rng(seed)
    N, K = 64 * 40 + 17, 256
    B = O.n_blocks(N)
    pages = rng.integers(-3, 4, size=(B, 64, 128)).astype(np.float32)
    st = O.RequestState(N + 64, N + 64 + 4 * 8)
    st.V[:N] = rng.integers(0, 5, N).astype(np.float32)
    st.D[:N + 40] = rng.integers(0, 5, N + 40).astype(np.float32)
    st.t = 3
    q = rng.integers(-2, 3, size=(rows, 64, 128)).astype(np.float32)
    w = np.ones((rows, 64), dtype=np.float32)
    return dict(q=q, q_dtype="f32", w=w, pages=pages, page_table_row=np.arange(B),
                key_dtype="f32", scale=None, n_slots=N, q_pos=N, K=K, sparsity_bp=6000,
                explore_bp=2000, alpha=0.5, layer=2, req_id=5, seed=99), st


def _copy(st):
    c = O.RequestState(len(st.V), len(st.D))
    c.V[:], c.D[:], c.t = st.V, st.D, st.t
    return c


def test_row0_mask_scores_row0_blocks_only():
    kw, st = _step_inputs()
    res = O.spin_step(_copy(st), mtp_row0_mask=True, **kw)
    want = np.nonzero(res["codes"][0] != O.CODE_SKIP)[0]
    assert np.array_equal(res["sel"], want)
    full = O.spin_step(_copy(st), **kw)
    assert set(want.tolist()) <= set(full["sel"].tolist())


def test_row0_update_is_the_single_row_update():
    kw, st = _step_inputs()
    a, b = _copy(st), _copy(st)
    res = O.spin_step(a, mtp_row0_update=True, n_valid=3, **kw)
    O.ema_update(b.V, b.D, res["z32"][:1], res["slots"], kw["q_pos"], 1, kw["alpha"])
    assert np.array_equal(a.V, b.V) and np.array_equal(a.D, b.D)
    c = _copy(st)
    O.spin_step(c, n_valid=3, **kw)
    assert not np.array_equal(a.D, c.D)                # the prefix-valid replay differs


def test_per_row_exploration_draws():
    kw, st = _step_inputs()
    shared = O.spin_step(_copy(st), **kw)
    per = O.spin_step(_copy(st), explore_per_row=True, **kw)
    ex_sh = [set(np.nonzero(c == O.CODE_EXPLORED)[0]) for c in shared["codes"]]
    ex_pr = [set(np.nonzero(c == O.CODE_EXPLORED)[0]) for c in per["codes"]]
    assert ex_pr[0] == ex_sh[0]                        # row 0 keeps the shared counter
    assert ex_pr[1] != ex_pr[0] or ex_pr[2] != ex_pr[0]
    # row r's draw: the smallest priorities of the counter with the row in its layer word
    B = O.n_blocks(kw["n_slots"])
    for r in (1, 2):
        pri = O.block_priority(B, st.t, kw["layer"] + 65536 * r, kw["req_id"], kw["seed"])
        pool = [j for j in range(B) if per["codes"][r][j] in (O.CODE_SKIP, O.CODE_EXPLORED)]
        order = sorted(pool, key=lambda j: (int(pri[j]), j))
        assert ex_pr[r] == set(order[:len(ex_pr[r])])


# ---------------------------------------------------------------------------
# exploration policies and block reductions (Sec. 4.6): hand examples and
# properties
# ---------------------------------------------------------------------------
def _hand():
    from tests.conftest import read_golden
    return read_golden("variants_hand.txt")


def _g(g, key, dtype=float):
    return np.array(g[key], dtype=dtype)


@pytest.mark.parametrize("policy", ["age", "staleness"])
def test_exploration_policies_hand(policy):
    g = _hand()
    S = _g(g, "explore_S:", np.float32)
    obs = _g(g, "explore_last_obs:", np.int64)
    codes = O.select_blocks(S, 512, 64, 0, 4000, 6, 0, 0, 0, budget=5, explore=policy,
                            last_obs=obs)
    assert codes.tolist() == _g(g, f"explore_{policy}_codes:", int).tolist()


def test_exploration_policies_properties():
    rng = np.random.default_rng(3)
    for trial in range(30):
        B = int(rng.integers(3, 200))
        S = rng.random(B).astype(np.float32) * 10
        obs = rng.integers(0, 20, B)
        t = 25
        for policy in ("random", "age", "staleness"):
            c = O.select_blocks(S, 64 * B, 64, 4000, 2000, t, 1, 2, 3, explore=policy,
                                last_obs=obs)
            expl = np.nonzero(c == O.CODE_EXPLORED)[0]
            pool = np.nonzero(c == O.CODE_SKIP)[0]
            m = O.block_budget(B, 64, 4000)
            assert (c != 0).sum() == max(m, 2 if B > 1 else 1)
            if policy == "age" and len(expl) and len(pool):
                # every explored block is at least as old as every one left out
                assert obs[expl].max() <= obs[pool].min()
            if policy == "staleness" and len(expl) and len(pool):
                sc = S * (t - obs).astype(np.float32)
                assert sc[expl].min() >= sc[pool].max()


@pytest.mark.parametrize("gamma", [0, 5000])
def test_a0_hand_example(gamma):
    g = _hand()
    z = np.zeros(320, dtype=np.float32)
    z[_g(g, "a0_slots:", int)] = _g(g, "a0_values:", np.float32)
    codes = O.a0_select(z, 320, 3, gamma, 5, 0, 0, 0)
    assert codes.tolist() == _g(g, f"a0_codes_gamma{gamma}:", int).tolist()


def test_a0_properties():
    rng = np.random.default_rng(4)
    for trial in range(30):
        N = int(rng.integers(65, 64 * 50))
        B = O.n_blocks(N)
        z = rng.random(N).astype(np.float32)
        K = int(rng.integers(1, 300))
        c = O.a0_select(z, N, K, 0, 3, 0, 0, 0)
        # the expanded blocks are exactly those holding a top-K slot (fp64 argsort)
        top = np.argsort(-z.astype(np.float64), kind="stable")[:K]
        want = set((top // 64).tolist()) | {0, B - 1}
        assert set(np.nonzero(c)[0].tolist()) == want
        # K >= N: every block
        assert (O.a0_select(z, N, N, 0, 3, 0, 0, 0) != 0).all()
        # the warm-up step is dense
        assert (O.a0_select(z, N, K, 0, 0, 0, 0, 0) == O.CODE_DENSE).all()


def test_a2_hand_example():
    g = _hand()
    Vb = np.zeros(8, dtype=np.float32)
    Db = np.zeros(8, dtype=np.float32)
    z = np.zeros((2, 128), dtype=np.float32)      # blocks 0 and 2, compact
    z[0, 5], z[0, 64 + 9] = 4.0, 2.0
    z[0, 6] = 1.0
    z[1, 63] = 8.0
    O.ema_update_a2(Vb, Db, z[:1], [0, 2], 192, 200, 1, 0.5)
    assert Vb[:3].tolist() == _g(g, "a2_Vb_after_row0:").tolist()
    Vb[:] = 0
    Db[:] = 0
    O.ema_update_a2(Vb, Db, z, [0, 2], 192, 200, 2, 0.5)
    assert Vb[:3].tolist() == _g(g, "a2_Vb_after_row1:").tolist()
    assert Db[:4].tolist() == _g(g, "a2_Db_after_row1:").tolist()
    S = O.predict_block_scores_a2(Vb, Db, 192, 202)
    assert S.tolist() == _g(g, "a2_S_next:").tolist()


def test_a2_properties():
    """Unselected blocks keep their state; row order matters; pooling follows
    pool_block on the block's valid slots."""
    rng = np.random.default_rng(5)
    N = 64 * 7 + 5
    sel = np.array([0, 3, 7])
    n = 64 * 2 + 5
    z = rng.random((2, n)).astype(np.float32) * 4
    Vb0 = rng.random(16).astype(np.float32)
    Db0 = rng.random(16).astype(np.float32)
    V1, D1 = Vb0.copy(), Db0.copy()
    O.ema_update_a2(V1, D1, z, sel, N, 500, 2, 0.9)
    keep = np.setdiff1d(np.arange(8), sel)
    assert np.array_equal(V1[keep], Vb0[keep])
    V2, D2 = Vb0.copy(), Db0.copy()
    O.ema_update_a2(V2, D2, z[::-1].copy(), sel, N, 500, 2, 0.9)
    assert not np.array_equal(D1, D2)              # the rows' offsets differ
    zb = O.pool_scores(z[0], sel, N, "top4")
    assert zb[2] == O.pool_block(z[0, 128:133], "top4")


@pytest.mark.parametrize("reduction,explore", [("A1", "age"), ("A1", "staleness"),
                                               ("A0", "random"), ("A2", "random"),
                                               ("A2", "age")])
def test_variant_pipeline_records_observations(reduction, explore):
    """A closed loop of every variant: the warm-up step observes every block at
    t = 0, and after each step the scored union carries that step."""
    rng = np.random.default_rng(6)
    N, K, rows = 64 * 30 + 7, 16, 2
    q = rng.integers(-3, 4, (rows, 64, 128)).astype(np.float32)
    w = np.ones((rows, 64), dtype=np.float32)
    pages = rng.integers(-3, 4, (31, 64, 128)).astype(np.float32)
    st = O.RequestState(64 * 31, N + 64)
    for t in range(4):
        res = O.spin_step(st, q=q, q_dtype="f32", w=w, pages=pages, page_table_row=np.arange(31),
                          key_dtype="f32", scale=None, n_slots=N, q_pos=N + 2 * t, K=K,
                          sparsity_bp=5000, explore_bp=1000, alpha=0.9, layer=0, req_id=0,
                          seed=7, explore=explore, reduction=reduction)
        assert (st.last_obs[res["sel"]] == t).all()
        if t == 0:
            assert len(res["sel"]) == O.n_blocks(N)
        else:
            assert len(res["sel"]) < O.n_blocks(N)
