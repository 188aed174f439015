"""Whole-step invariants of the CPU oracle (SPIN paper Algorithm 1 with the
prose that follows it, Sec. 3.2.1 and Sec. 3.2.2).  CPU only."""
import copy

import numpy as np
import pytest

import spin_synth as G
from oracle import spin_oracle as O
from tests.harness import build_layer, run_oracle

SMALL_F32 = G.WORKLOADS["tiny_f32_4k"].scaled(steps=6)
SMALL_FP8 = G.WORKLOADS["fp8_128k_b32"].scaled(batch=2, n_slots=4096 + 200, n_slots_min=4096 + 200,
                                               topk=512, steps=6)
SMALL_MTP = G.WORKLOADS["fp8_128k_b32_mtp4"].scaled(batch=2, n_slots=3000, n_slots_min=3000,
                                                    topk=256, steps=8)


@pytest.fixture(scope="module")
def f32_layer():
    return build_layer(SMALL_F32)


@pytest.fixture(scope="module")
def fp8_layer():
    return build_layer(SMALL_FP8)


def dense_topk(li, s, r, rows=1):
    """Top-K of the dense indexer over every slot (no SPIN)."""
    w = li.w
    N = int(li.ctx[r])
    slots = np.arange(N)
    keys = O.gather_keys(li.np_pages(), li.keys.page_table.numpy()[r], slots, w.key_dtype,
                         None if li.keys.scale is None else li.keys.scale.numpy())
    qd = O.decode_q(li.np_q(s)[r], w.q_dtype)
    z = O.canon32(O.index_scores(qd[0], li.weights[r, 0].numpy(), keys))
    return O.topk_slots(z, slots, w.topk), z


def test_first_step_is_dense(fp8_layer):
    res, _ = run_oracle(fp8_layer, 1, 4000)
    for r, x in res[0].items():
        assert (x["codes"] == O.CODE_DENSE).all()
        assert np.array_equal(x["topk"][0], dense_topk(fp8_layer, 0, r)[0])


@pytest.mark.parametrize("which", ["f32", "fp8"])
def test_zero_sparsity_equals_dense_topk(which, f32_layer, fp8_layer):
    li = f32_layer if which == "f32" else fp8_layer
    res, _ = run_oracle(li, li.w.steps, 0)
    for s in range(li.w.steps):
        for r, x in res[s].items():
            assert (x["codes"] != O.CODE_SKIP).all()
            assert np.array_equal(x["topk"][0], dense_topk(li, s, r)[0])


def test_sparse_topk_is_masked_dense_topk(fp8_layer):
    """Miss-rate protocol identity (Sec. 4.1): sparse top-K = top-K of the dense
    scores after the block mask is applied."""
    li = fp8_layer
    res, _ = run_oracle(li, li.w.steps, 4000)
    for s in range(1, li.w.steps):
        for r, x in res[s].items():
            top, z = dense_topk(li, s, r)
            masked = np.full_like(z, -np.inf)
            masked[x["slots"]] = z[x["slots"]]
            keep = np.isfinite(masked)
            want = O.topk_slots(masked[keep], np.nonzero(keep)[0], li.w.topk)
            assert np.array_equal(x["topk"][0], want)
            B = O.n_blocks(int(li.ctx[r]))
            assert len(x["sel"]) == O.block_budget(B, li.w.topk, 4000)


def test_checkpoint_resume_is_bit_identical(f32_layer):
    li = f32_layer
    res_a, st_a = run_oracle(li, 3, 4000)
    snap = copy.deepcopy(st_a)
    # continue from the snapshot with the remaining steps
    li2 = copy.copy(li)
    li2.pos, li2.accept, li2.q = li.pos[3:], li.accept[3:], li.q[3:]
    res_b, st_b = run_oracle(li2, 3, 4000, states=snap)
    res_full, st_full = run_oracle(li, 6, 4000)
    for s in range(3):
        for r in res_b[s]:
            assert np.array_equal(res_b[s][r]["topk"], res_full[s + 3][r]["topk"])
    for r in st_b:
        assert np.array_equal(st_b[r].V, st_full[r].V) and np.array_equal(st_b[r].D, st_full[r].D)


def test_integer_inputs_give_exact_fp32_scores():
    w = SMALL_FP8.scaled(steps=3)
    li = build_layer(w, integer=True)
    res, _ = run_oracle(li, 3, 4000)
    for s in range(3):
        for r, x in res[s].items():
            assert np.array_equal(x["z64"], x["z32"].astype(np.float64))


def test_mtp_union_and_deferred_replay():
    li = build_layer(SMALL_MTP)
    res, states = run_oracle(li, SMALL_MTP.steps, 4000)
    for s in range(1, SMALL_MTP.steps):
        for r, x in res[s].items():
            union = O.union_blocks(x["codes"])
            assert np.array_equal(union, x["sel"])
            for row in range(4):                     # each row's own mask is inside the union
                assert set(np.nonzero(x["codes"][row])[0]) <= set(x["sel"])
            B = O.n_blocks(int(li.ctx[r]))
            m = O.block_budget(B, SMALL_MTP.topk, 4000)
            assert all(int((x["codes"][row] != 0).sum()) == m for row in range(4))
            assert m <= len(x["sel"]) <= B
    # the generator and the oracle are deterministic: two builds give identical results
    one = SMALL_MTP.scaled(rows=1, accept_probs=None)
    li1 = build_layer(one)
    r1, _ = run_oracle(li1, 3, 4000)
    li1b = build_layer(one)
    r2, _ = run_oracle(li1b, 3, 4000)
    for s in range(3):
        for r in r1[s]:
            assert np.array_equal(r1[s][r]["topk"], r2[s][r]["topk"])
