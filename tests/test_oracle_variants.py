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
