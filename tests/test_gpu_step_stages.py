"""Inside spin_step, predict and select (+ union) must leave S, row codes and
block lists bit-identical to spin_predict_blocks followed by
spin_select_blocks on the same state, for every block capacity the selection
is instantiated for (up to 8,192 blocks), with short contexts in a large
capacity, budgets, several verifier rows and an invalid request."""
import numpy as np
import pytest
import torch

import spin_synth as G
from tests.gpu_util import DEV, banner, make_layer
from tests.harness import build_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_indexer_spin_amd import _lib
    return _lib.load()


CASES = [
    # rows, requests, longest / shortest context, block capacity (None: fit), bad request
    (1, 5, 64 * 300 + 17, 100, None, None),
    (4, 5, 64 * 300 + 17, 100, None, None),
    (2, 3, 20000, 3000, 4096, 1),
    (1, 2, 70000, 60000, 8192, None),
    (3, 4, 9000, 64, 1024, 2),
]


@pytest.mark.parametrize("rows,R,n_max,n_min,mb,bad", CASES)
def test_step_predict_select_matches_stages(rows, R, n_max, n_min, mb, bad):
    banner(f"step predict+select rows={rows} R={R} N={n_min}..{n_max} mb={mb} bad={bad}")
    from sparse_attention_indexer_spin_amd import SpinLayer, api as A
    name = "fp8_128k_b32_mtp4" if rows > 1 else "fp8_128k_b32"
    w = G.WORKLOADS[name].scaled(batch=R, rows=rows, n_slots=n_max, n_slots_min=n_min, steps=5,
                                 topk=256)
    li = build_layer(w)
    cap = mb or w.max_blocks
    # (S after the step is the step's own prediction: without predicting ahead)
    lay = SpinLayer(batch=R, max_blocks=cap, d_cap=G.d_capacity(w, w.steps), topk=w.topk,
                    sparsity_bp=4000, n_rows=rows, explore_bp=w.explore_bp, ema_alpha=w.alpha,
                    key_dtype=torch.uint8, q_dtype=torch.bfloat16, device=DEV,
                    predict_ahead=False)
    ctx = li.ctx.clone()
    if bad is not None:
        ctx[bad] = 64 * cap + 1                   # beyond the block capacity
    lay.set_requests(ctx.to(DEV), li.pos[0].to(DEV))
    lay.reset()
    pages, scale = li.keys.pages.to(DEV), li.keys.scale.to(DEV)
    pt = torch.zeros(R, cap, dtype=torch.int32)
    pt[:, :li.keys.page_table.shape[1]] = li.keys.page_table
    pt = pt.to(DEV)
    budget = torch.tensor([0] + [max(1, int(c) // 64 // 3) for c in li.ctx[1:]],
                          dtype=torch.int32, device=DEV)
    for s in range(w.steps):
        bud = budget if s >= 2 else None
        bt = lay.batch(pages.shape[0])
        S2, code2 = lay.S.clone(), lay.row_code.clone()
        sel2, nsel2 = lay.sel.clone(), lay.n_sel.clone()
        A.spin_predict_blocks(lay.cfg, bt, lay.V, lay.D, S2)
        A.spin_select_blocks(lay.cfg, bt, S2, code2, sel2, nsel2, budget=bud)
        lay.step(li.q[s].to(DEV).contiguous(), li.weights.to(DEV), pages, scale, pt,
                 n_valid=li.accept[s].to(DEV) if rows > 1 else None, budget=bud)
        torch.cuda.synchronize()
        assert torch.equal(lay.S, S2), f"S differs at step {s}"
        assert torch.equal(lay.row_code, code2), f"row codes differ at step {s}"
        assert torch.equal(lay.n_sel, nsel2), f"n_sel differs at step {s}"
        assert torch.equal(lay.sel, sel2), f"block lists differ at step {s}"
    err = int(lay.err.item())
    if bad is None:
        assert err == 0
    else:
        # the context past capacity also puts q_pos before its end (bit 2)
        assert err & 1 and int(lay.n_sel[bad].item()) == 0
