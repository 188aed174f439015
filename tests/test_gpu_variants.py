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
    for r in range(w.batch):
        N = int(li.ctx[r])
        assert np.array_equal(Vg[r, :N], st[r].V[:N])
        dl = min(Dg.shape[1], st[r].D.shape[0])
        assert np.array_equal(Dg[r, :dl], st[r].D[:dl])
    assert int(lay.err.item()) == 0
