"""Pins for the CPU oracle: each check ties an oracle function to something
other than itself (hand-worked values from the method's definition, closed
forms, invariants, or an independent library routine).  CPU only."""
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import spin_oracle as O
from tests.conftest import ROOT, read_golden

# ---------------------------------------------------------------------------
# Philox4x32-10
# ---------------------------------------------------------------------------
PIN_SRC = os.path.join(ROOT, "tests", "pins", "philox_rocrand_pin.cpp")


@pytest.fixture(scope="session")
def rocrand_philox(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND pin")
    exe = str(tmp_path_factory.mktemp("pin") / "philox_pin")
    subprocess.run([hipcc, "-O1", "-o", exe, PIN_SRC], check=True,
                   capture_output=True, cwd=str(tmp_path_factory.getbasetemp()))

    def run(ctrs, keys):
        lines = "".join("%x %x %x %x %x %x\n" % (*c, *k) for c, k in zip(ctrs, keys))
        out = subprocess.run([exe], input=lines, capture_output=True, text=True, check=True)
        return [tuple(int(x, 16) for x in ln.split()) for ln in out.stdout.strip().splitlines()]
    return run


def test_philox_published_kat():
    g = read_golden("philox_kat.txt")
    vals = [int(x, 16) for x in g["00000000"]]
    # line layout: c1 c2 c3 k0 k1 x0 x1 x2 x3 after the first token (c0)
    ctr = (0, vals[0], vals[1], vals[2])
    key = (vals[3], vals[4])
    got = [int(x) for x in O.philox4x32_10(ctr, key)]
    assert got == vals[5:9]


def test_philox_matches_rocrand(rocrand_philox):
    rng = np.random.default_rng(1)
    ctrs = [tuple(int(x) for x in rng.integers(0, 2**32, 4)) for _ in range(200)]
    ctrs = [(c[0], c[1] & 0x3FFFFFFF, c[2], c[3]) for c in ctrs]
    keys = [tuple(int(x) for x in rng.integers(0, 2**32, 2)) for _ in range(200)]
    ref = rocrand_philox(ctrs, keys)
    for c, k, r in zip(ctrs, keys, ref):
        assert tuple(int(x) for x in O.philox4x32_10(c, k)) == r


def test_block_priority_vectorised_matches_rocrand(rocrand_philox):
    seed = 0x1234_5678_5350_494E
    pri = O.block_priority(300, 17, 3, 11, seed)
    ref = rocrand_philox([(j, 17, 3, 11) for j in range(300)],
                         [(seed & 0xFFFFFFFF, seed >> 32)] * 300)
    assert [int(p) for p in pri] == [r[0] for r in ref]


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------
def test_decode_e4m3_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # closed-form spot values of the format
    assert O.decode_e4m3([0x38])[0] == 1.0
    assert O.decode_e4m3([0x7E])[0] == 448.0
    assert O.decode_e4m3([0x01])[0] == 2.0 ** -9
    assert O.decode_e4m3([0xC0])[0] == -2.0


def test_decode_bf16_vs_torch():
    rng = np.random.default_rng(2)
    x = torch.from_numpy(rng.standard_normal(1000).astype(np.float32) * 100).to(torch.bfloat16)
    codes = x.view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(O.decode_bf16(codes), x.to(torch.float64).numpy())


# ---------------------------------------------------------------------------
# stage 1: predicted block scores
# ---------------------------------------------------------------------------
def test_predict_hand_example():
    g = read_golden("predict_hand.txt")
    b, N, q = int(g["b"][0]), int(g["N"][0]), int(g["q"][0])
    V = np.array(g["V"], dtype=np.float32)
    D = np.array(g["D"], dtype=np.float32)
    assert np.array_equal(O.predict_block_scores(V, D, N, q, "max", b),
                          np.array(g["S_max"], dtype=np.float32))
    assert np.array_equal(O.predict_block_scores(V, D, N, q, "sum", b),
                          np.array(g["S_sum"], dtype=np.float32))


def _sliding_max_numpy(D, q, N, b):
    # block j reads offsets q-i for i in [jb, min((j+1)b, N)); via numpy's
    # sliding-window view over the reversed offset axis
    from numpy.lib.stride_tricks import sliding_window_view
    rev = D[q - np.arange(N)]                         # rev[i] = D[q - i]
    pad = np.concatenate([rev, np.full((-N) % b, -np.inf, dtype=np.float32)])
    return sliding_window_view(pad, b)[::b].max(axis=1)


@pytest.mark.parametrize("N", [4096, 4000, 65, 64, 1])
def test_predict_special_cases(N):
    rng = np.random.default_rng(N)
    q = N + 3
    V = rng.random(N + 64).astype(np.float32) * 5
    D = rng.random(q + 8).astype(np.float32) * 5
    B = O.n_blocks(N)
    zeros_v, zeros_d = np.zeros_like(V), np.zeros_like(D)
    # V = 0: S is a windowed max of D (clamped at 0)
    S = O.predict_block_scores(zeros_v, D, N, q)
    assert np.array_equal(S, np.maximum(_sliding_max_numpy(D, q, N, 64), 0).astype(np.float32))
    # D = 0: S is the block max of V over valid slots
    S = O.predict_block_scores(V, zeros_d, N, q)
    vb = np.concatenate([V[:N], np.zeros((-N) % 64, np.float32)]).reshape(B, 64).max(1)
    assert np.array_equal(S, vb)
    # max combine decomposes: S = max(blockmax V, windowmax D)
    S = O.predict_block_scores(V, D, N, q)
    vb = np.concatenate([V[:N], np.full((-N) % 64, -np.inf, np.float32)]).reshape(B, 64).max(1)
    assert np.array_equal(S, np.maximum(vb, _sliding_max_numpy(D, q, N, 64)))


# ---------------------------------------------------------------------------
# stage 2: budget and selection
# ---------------------------------------------------------------------------
def test_budget_closed_forms():
    with open(os.path.join(ROOT, "tests", "golden", "budget_hand.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    for r in rows:
        B, K, rho, m = int(r[0]), int(r[1]), int(r[2]), int(r[3])
        n_e = int(r[-1])
        assert O.block_budget(B, K, rho) == m, r
        n_f = 2 if B > 1 else 1
        m_kept = max(m, n_f)                       # forced blocks are always retained
        assert min(m_kept * 500 // 10000, m_kept - n_f) == n_e


def test_select_hand_example():
    g = read_golden("select_hand.txt")
    S = np.array(g["S"], dtype=np.float32)
    code = O.select_blocks(S, int(g["N"][0]), int(g["K"][0]), int(g["rho_bp"][0]),
                           int(g["gamma_bp"][0]), step=3, layer=0, req_id=0, seed=0x5350494E)
    assert sorted(np.nonzero(code == O.CODE_FORCED)[0]) == [int(x) for x in g["forced"]]
    assert sorted(np.nonzero(code == O.CODE_RANKED)[0]) == sorted(int(x) for x in g["ranked"])
    explored = np.nonzero(code == O.CODE_EXPLORED)[0]
    assert len(explored) == 1 and int(explored[0]) in [int(x) for x in g["pool"]]


def test_select_exploration_pick_vs_rocrand(rocrand_philox):
    g = read_golden("select_hand.txt")
    S = np.array(g["S"], dtype=np.float32)
    seed = 0x5350494E
    pool = [int(x) for x in g["pool"]]
    for t in range(1, 40):
        code = O.select_blocks(S, 640, 64, 3000, 1500, step=t, layer=2, req_id=5, seed=seed)
        pri = rocrand_philox([(j, t, 2, 5) for j in pool], [(seed, 0)] * len(pool))
        want = min(zip([p[0] for p in pri], pool))[1]
        assert int(np.nonzero(code == O.CODE_EXPLORED)[0][0]) == want


@pytest.mark.parametrize("B,K,rho,gamma", [(64, 512, 4000, 500), (1024, 2048, 4000, 500),
                                           (333, 2048, 5000, 2000), (2048, 2048, 0, 500),
                                           (7, 64, 9000, 5000), (1, 512, 4000, 500),
                                           (2, 64, 9900, 500)])
def test_select_invariants(B, K, rho, gamma):
    rng = np.random.default_rng(B + rho)
    N = B * 64 - 17 if B > 1 else 30
    for t in range(0, 6):
        S = np.round(rng.random(B) * 8).astype(np.float32)        # many ties
        code = O.select_blocks(S, N, K, rho, gamma, step=t, layer=1, req_id=9, seed=77)
        if t == 0:
            assert (code == O.CODE_DENSE).all()
            continue
        m = max(O.block_budget(B, K, rho), len({0, B - 1}))
        assert int((code != 0).sum()) == m                       # |M| = m
        assert code[0] == O.CODE_FORCED and code[B - 1] == O.CODE_FORCED
        ranked = np.nonzero(code == O.CODE_RANKED)[0]
        others = np.nonzero((code == O.CODE_SKIP) | (code == O.CODE_EXPLORED))[0]
        # every ranked block beats every unranked non-forced block under (S desc, j asc)
        for r_ in ranked:
            for o in others:
                assert (S[r_] > S[o]) or (S[r_] == S[o] and r_ < o)
        n_f = len({0, B - 1})
        assert int((code == O.CODE_EXPLORED).sum()) == min(m * gamma // 10000, m - n_f)
        if rho == 0:
            assert (code != 0).all()


def test_exploration_is_uniform():
    """Exploration draws are uniform over the pool (chi-square at 0.1 %)."""
    B, n = 200, 4000
    S = np.zeros(B, dtype=np.float32)
    S[:100] = 1.0
    m = O.block_budget(B, 64, 4000)          # ceil(0.6 * 200) = 120
    n_e = m * 1000 // 10000                  # 12
    n_r = m - 2 - n_e                        # 106: blocks 1..99 then 100..106 (lower index wins ties)
    pool = np.arange(n_r + 1, B - 1)         # 107..198
    counts = np.zeros(B)
    for t in range(1, n + 1):
        code = O.select_blocks(S, B * 64, 64, 4000, 1000, step=t, layer=0, req_id=1, seed=5)
        assert (code[1:n_r + 1] == O.CODE_RANKED).all()
        counts += code == O.CODE_EXPLORED
    assert counts[: n_r + 1].sum() == 0 and counts[B - 1] == 0
    obs = counts[pool]
    exp = n * n_e / len(pool)
    chi2 = ((obs - exp) ** 2 / exp).sum()
    from scipy.stats import chi2 as c2
    assert chi2 < c2.ppf(0.999, len(pool) - 1)


# ---------------------------------------------------------------------------
# stage 3: indexer score and top-K
# ---------------------------------------------------------------------------
def test_score_hand_example():
    g = read_golden("score_hand.txt")
    q = np.array(g["q"], dtype=np.float64).reshape(2, 2)
    w = np.array(g["w"], dtype=np.float64)
    k = np.array(g["k"], dtype=np.float64).reshape(3, 2)
    assert np.array_equal(O.index_scores(q, w, k), np.array(g["z"], dtype=np.float64))


def test_score_single_head_is_relu_dot():
    rng = np.random.default_rng(3)
    q = rng.integers(-5, 6, (1, 128))
    k = rng.integers(-5, 6, (50, 128))
    want = [max(int(np.dot(q[0], ki)), 0) for ki in k]      # textbook dot product
    assert np.array_equal(O.index_scores(q, [1.0], k), np.array(want, dtype=np.float64))


def test_score_structure():
    rng = np.random.default_rng(4)
    q = rng.integers(-3, 4, (64, 128)).astype(np.float64)
    k = rng.integers(-4, 5, (100, 128)).astype(np.float64)
    w1 = rng.integers(1, 4, 64) * 0.5
    w2 = rng.integers(1, 4, 64) * 0.25
    z1, z2 = O.index_scores(q, w1, k), O.index_scores(q, w2, k)
    assert np.array_equal(O.index_scores(q, w1 + w2, k), z1 + z2)        # linear in w
    perm = rng.permutation(64)
    assert np.array_equal(O.index_scores(q[perm], w1[perm], k), z1)      # head order free
    # a head whose query is negated contributes ReLU(-x) instead of ReLU(x)
    q2 = q.copy()
    q2[5] *= -1
    d = k @ q[5]
    assert np.array_equal(O.index_scores(q2, w1, k) - z1,
                          w1[5] * (np.maximum(-d, 0) - np.maximum(d, 0)))


# --- exact fp32 mode: the canonical fp32 order (oracle/score_f32.c) -------
def _round_f32(x: Fraction) -> float:
    """Round an exact rational to the nearest fp32 (ties to even), written
    from the definition of IEEE-754 binary32 (24-bit significand, emin -126,
    subnormal quantum 2^-149); no float arithmetic is involved."""
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * quantum
    assert v < Fraction(2) ** 128, "overflow"
    return sign * float(v)           # v is an fp32 value: exact in a Python float


def _exact_chain_z(q, w, k):
    """z of one slot in the canonical order, each fma rounded from the exact
    rational a*b + c (the definition of a fused multiply-add)."""
    z = Fraction(0)
    for h in range(q.shape[0]):
        s = Fraction(0)
        for c in range(q.shape[1]):
            s = Fraction(_round_f32(Fraction(float(q[h, c])) * Fraction(float(k[c])) + s))
        r = s if s > 0 else Fraction(0)
        z = Fraction(_round_f32(Fraction(float(w[h])) * r + z))
    return np.float32(float(z))


def test_fmaf_rounds_once():
    from oracle.score_f32 import fmaf
    a = np.float32(1 + 2.0 ** -12)
    # a*a = 1 + 2^-11 + 2^-24 is halfway between two fp32 neighbours; a tiny
    # addend decides the direction.  A product and sum rounded to fp64 first
    # would lose it and round the tie to even instead.
    up, down = np.float32(1 + 2.0 ** -11 + 2.0 ** -23), np.float32(1 + 2.0 ** -11)
    assert fmaf(a, a, np.float32(2.0 ** -60)) == up
    assert fmaf(a, a, np.float32(-(2.0 ** -60))) == down
    assert np.float32(np.float64(a) * np.float64(a) + 2.0 ** -60) == down  # double rounding
    rng = np.random.default_rng(11)
    for _ in range(300):
        x, y, c = (np.float32(v) for v in rng.standard_normal(3) * 2.0 ** rng.integers(-8, 8, 3))
        want = _round_f32(Fraction(float(x)) * Fraction(float(y)) + Fraction(float(c)))
        assert fmaf(x, y, c) == np.float32(want)


def test_exact_f32_score_matches_rational_chain():
    """Gaussian inputs of the tiny workload's shape: the C oracle's canonical
    fp32 chain equals the chain evaluated with exact rationals and rounded per
    the fp32 definition, bit for bit."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((64, 128)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, 64).astype(np.float32)
    k = rng.standard_normal((6, 128)).astype(np.float32)
    z = O.index_scores_exact_f32(q, w, k)
    for i in range(k.shape[0]):
        assert z[i] == _exact_chain_z(q, w, k[i]), i


def test_exact_f32_score_hand_and_integer_inputs():
    g = read_golden("score_hand.txt")
    q = np.array(g["q"], dtype=np.float32).reshape(2, 2)
    w = np.array(g["w"], dtype=np.float32)
    k = np.array(g["k"], dtype=np.float32).reshape(3, 2)
    assert np.array_equal(O.index_scores_exact_f32(q, w, k), np.array(g["z"], dtype=np.float32))
    # small integers: every partial sum is exact in fp32, so the chain equals
    # the fp64 definition exactly
    rng = np.random.default_rng(13)
    q = rng.integers(-4, 5, (64, 128)).astype(np.float32)
    k = rng.integers(-4, 5, (200, 128)).astype(np.float32)
    w = (rng.integers(1, 5, 64) * 0.5).astype(np.float32)
    assert np.array_equal(O.index_scores_exact_f32(q, w, k),
                          O.index_scores(q, w, k).astype(np.float32))


def test_exact_f32_score_within_fp32_error_bound():
    """|z32 - z| within the standard bound for recursive summation with fma
    (gamma_n = n u / (1 - n u), u = 2^-24): per head gamma_128 sum_c |q_c k_c|,
    then the head sum adds gamma_64 sum_h w_h |r_h| and scales the head errors
    by (1 + gamma_64)."""
    rng = np.random.default_rng(14)
    q = rng.standard_normal((64, 128)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, 64).astype(np.float32)
    k = rng.standard_normal((500, 128)).astype(np.float32)
    u = 2.0 ** -24
    g = lambda n: n * u / (1 - n * u)
    qd, kd, wd = q.astype(np.float64), k.astype(np.float64), w.astype(np.float64)
    z64 = O.index_scores(qd, wd, kd)
    absdot = np.abs(kd) @ np.abs(qd).T                      # [n, n_h]
    r = np.maximum(kd @ qd.T, 0)
    bound = (1 + g(64)) * g(128) * (absdot @ wd) + g(64) * (r @ wd)
    err = np.abs(O.index_scores_exact_f32(q, w, k).astype(np.float64) - z64)
    assert np.all(err <= bound)
    assert err.max() > 0                    # the fp32 chain is not the fp64 value


def test_fp8_scale_pulls_out_of_relu():
    rng = np.random.default_rng(5)
    pages = rng.integers(0, 256, (3, 64, 128)).astype(np.uint8)
    pages[(pages & 0x7F) == 0x7F] = 0x10          # no NaN codes
    scale = np.ones((3, 64), dtype=np.float32)
    pt = np.array([2, 0, 1])
    slots = np.arange(0, 190)
    k1 = O.gather_keys(pages, pt, slots, "fp8", scale)
    k4 = O.gather_keys(pages, pt, slots, "fp8", scale * 4)
    q = rng.integers(-3, 4, (64, 128)).astype(np.float64)
    w = np.ones(64)
    assert np.array_equal(O.index_scores(q, w, k4), 4 * O.index_scores(q, w, k1))
    # the page table is honoured: slot 64 lives on physical page pt[1] = 0, row 0
    assert np.array_equal(k1[64], O.decode_e4m3(pages[0, 0]))


def test_topk_hand_example():
    g = read_golden("topk_hand.txt")
    z = np.array(g["z"], dtype=np.float32)
    slots = np.arange(8)
    assert list(O.topk_slots(z, slots, 4)) == [int(x) for x in g["K4"]]
    assert list(O.topk_slots(z, slots, 5)) == [int(x) for x in g["K5"]]
    assert list(O.topk_slots(z, slots, 10)) == [int(x) for x in g["K10"]]


def test_topk_distinct_matches_argpartition():
    rng = np.random.default_rng(6)
    z = rng.permutation(50000).astype(np.float32)
    slots = np.sort(rng.choice(200000, 50000, replace=False))
    want = np.sort(slots[np.argpartition(-z, 2048)[:2048]])
    assert np.array_equal(O.topk_slots(z, slots, 2048), want)


def test_topk_signed_zero_ties():
    z = np.array([-0.0, 0.0, -0.0, 1.0], dtype=np.float32)
    assert list(O.topk_slots(z, np.arange(4), 2)) == [0, 3]


# ---------------------------------------------------------------------------
# stage 4: EMA
# ---------------------------------------------------------------------------
def test_ema_hand_example():
    g = read_golden("ema_hand.txt")
    V = np.zeros(16, np.float32)
    D = np.zeros(16, np.float32)
    O.ema_update(V, D, np.array([[4.0]], np.float32), [7], 10, 1, float(g["alpha"][0]))
    O.ema_update(V, D, np.array([[8.0]], np.float32), [7], 11, 1, float(g["alpha"][0]))
    assert V[7] == float(g["V7"][0])
    assert D[3] == float(g["D3"][0]) and D[4] == float(g["D4"][0])
    assert np.count_nonzero(V) == 1 and np.count_nonzero(D) == 2


def test_ema_closed_form():
    """Constant observation z: V_n = (1 - a^n) z (exact arithmetic) within a few ulp per step."""
    V = np.zeros(4, np.float32)
    D = np.zeros(64, np.float32)
    z = np.float32(37.25)
    for n in range(1, 61):
        O.ema_update(V, D, np.array([[z]], np.float32), [2], 10, 1, 0.9)
        b = np.float64(np.float32(1.0) - np.float32(0.9))
        a = 1.0 - b
        exact = (1.0 - a ** n) * np.float64(z)
        assert abs(V[2] - exact) <= 4 * n * np.spacing(np.float32(exact))
    # beta is 1 - alpha rounded in fp32
    assert np.float32(1.0) - np.float32(0.9) == np.float32(0.100000024)


def test_ema_replay_order_and_prefix():
    rng = np.random.default_rng(7)
    slots = np.arange(64, 128)
    z = rng.random((2, 64)).astype(np.float32) * 10
    base_v = rng.random(256).astype(np.float32)
    base_d = rng.random(256).astype(np.float32)
    V1, D1 = base_v.copy(), base_d.copy()
    O.ema_update(V1, D1, z, slots, 150, 2, 0.9)
    V2, D2 = base_v.copy(), base_d.copy()
    O.ema_update(V2, D2, z[::-1].copy(), slots, 150, 2, 0.9)
    assert not np.array_equal(V1, V2)                 # row order matters
    V3, D3 = base_v.copy(), base_d.copy()
    O.ema_update(V3, D3, z, slots, 150, 1, 0.9)       # L = 1 == row 0 only
    V4, D4 = base_v.copy(), base_d.copy()
    O.ema_update(V4, D4, z[:1], slots, 150, 1, 0.9)
    assert np.array_equal(V3, V4) and np.array_equal(D3, D4)
    untouched = np.setdiff1d(np.arange(256), slots)
    assert np.array_equal(V1[untouched], base_v[untouched])   # unobserved slots unchanged
    touched_d = np.union1d(150 - slots, 151 - slots)
    assert np.array_equal(np.delete(D1, touched_d), np.delete(base_d, touched_d))
