"""SPIN_PREDICT_AHEAD: the EMA update of a step also predicts the next step's
block scores, which that step then uses instead of predicting.  A layer with
the flag must step bit for bit like one without (masks, block lists, top-K,
V, D, the V maxima, counters and last-observed steps), and after every step
its S must equal spin_predict_blocks on the state it left, at the next
position.  Cases cover both EMA kernels (beside the top-K and on their own,
f32 keys), contexts that end inside a block and on a block boundary (then a
block past the last holds the offset of the slot beyond the context),
acceptance 0 / 1, every pooling, the sum combine, the V maxima and the
exploration policies that read S."""
import numpy as np
import pytest
import torch

import spin_synth as G
from tests.gpu_util import DEV, banner, device_keys, make_layer
from tests.harness import build_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_indexer_spin_amd import _lib
    return _lib.load()


def _w(name):
    if name == "f32":
        return G.WORKLOADS["tiny_f32_4k"].scaled(batch=3, n_slots=64 * 40 + 5, n_slots_min=300,
                                                 steps=8, topk=128)
    if name == "bf16":
        return G.WORKLOADS["bf16_64k_b16"].scaled(batch=3, n_slots=64 * 90, n_slots_min=64 * 20,
                                                  steps=7, topk=256)
    if name == "fp8_edge":  # every context a multiple of 64
        return G.WORKLOADS["fp8_128k_b32"].scaled(batch=4, n_slots=64 * 150, n_slots_min=64 * 150,
                                                  steps=7, topk=256)
    return G.WORKLOADS["fp8_128k_b32"].scaled(batch=5, n_slots=64 * 200 + 37, n_slots_min=900,
                                              steps=8, topk=256)


CASES = [
    ("fp8", {}, False),
    ("fp8", {}, True),                           # acceptance 0 / 1 per request
    ("fp8_edge", {}, False),
    ("fp8", dict(vmax_cache=True), False),
    ("fp8", dict(pooling="top4"), False),
    ("fp8", dict(pooling="mean", combine="sum"), False),
    ("fp8", dict(explore="staleness"), False),
    ("fp8", dict(explore="age", mtp_row0_update=True), True),
    ("bf16", {}, False),
    ("f32", dict(combine="sum"), False),
    ("f32", dict(pooling="top4"), True),
]


@pytest.mark.parametrize("name,variants,accept", CASES)
def test_predict_ahead_steps_like_plain_steps(name, variants, accept):
    banner(f"predict ahead {name} {variants} accept={accept}")
    from sparse_attention_indexer_spin_amd import api as A
    w = _w(name)
    li = build_layer(w, integer=(name == "f32"))
    sp = 4000
    ahead = make_layer(li, sp, predict_ahead=True, **variants)
    plain = make_layer(li, sp, predict_ahead=False, **variants)
    pages, scale, pt = device_keys(li)
    W = li.weights.to(DEV)
    rng = np.random.default_rng(7)
    S2 = torch.empty_like(ahead.S)
    for s in range(w.steps):
        q = li.q[s].to(DEV).contiguous()
        nv = torch.as_tensor(rng.integers(0, 2, w.batch), dtype=torch.int32, device=DEV) \
            if accept else None
        ahead.step(q, W, pages, scale, pt, n_valid=nv)
        plain.step(q, W, pages, scale, pt, n_valid=nv)
        torch.cuda.synchronize()
        for a, b, what in ((ahead.topk_idx, plain.topk_idx, "top-K"),
                           (ahead.row_code, plain.row_code, "codes"),
                           (ahead.sel, plain.sel, "sel"), (ahead.n_sel, plain.n_sel, "n_sel"),
                           (ahead.V, plain.V, "V"), (ahead.D, plain.D, "D"),
                           (ahead.q_pos, plain.q_pos, "q_pos"),
                           (ahead.step_ctr, plain.step_ctr, "step"),
                           (ahead.last_obs, plain.last_obs, "last_obs")):
            assert torch.equal(a, b), f"{what} differs at step {s}"
        if ahead.v_max is not None:
            assert torch.equal(ahead.v_max, plain.v_max), f"V maxima differ at step {s}"
        # S now holds the next step's scores: the standalone prediction there
        S2.fill_(-7.0)
        A.spin_predict_blocks(ahead.cfg, ahead.batch(pages.shape[0]), ahead.V, ahead.D, S2,
                              v_max=ahead.v_max)
        torch.cuda.synchronize()
        B = [-(-int(c) // 64) for c in li.ctx]
        Sa, Sb = ahead.S.cpu(), S2.cpu()
        for r in range(w.batch):
            assert torch.equal(Sa[r, 0, :B[r]], Sb[r, 0, :B[r]]), f"S step {s} request {r}"
        tag = ahead.s_tag.cpu().numpy()
        assert (tag[:, 0] == ahead.step_ctr.cpu().numpy()).all()
        assert (tag[:, 1] == ahead.q_pos.cpu().numpy()).all()
    assert int(ahead.err.item()) == 0 and int(plain.err.item()) == 0


def test_tags_go_stale_when_the_requests_change():
    """After set_requests (new positions) the next step predicts for itself."""
    banner("predict ahead: new requests")
    w = _w("fp8")
    li = build_layer(w)
    ahead = make_layer(li, 4000, predict_ahead=True)
    plain = make_layer(li, 4000, predict_ahead=False)
    pages, scale, pt = device_keys(li)
    W = li.weights.to(DEV)
    for s in range(w.steps):
        if s == 4:  # the requests jump ahead by 3 positions between steps
            for lay in (ahead, plain):
                lay.set_requests(li.ctx.to(DEV), lay.q_pos + 3)
        q = li.q[s].to(DEV).contiguous()
        ahead.step(q, W, pages, scale, pt)
        plain.step(q, W, pages, scale, pt)
        torch.cuda.synchronize()
        assert torch.equal(ahead.topk_idx, plain.topk_idx), s
        assert torch.equal(ahead.V, plain.V) and torch.equal(ahead.D, plain.D), s
