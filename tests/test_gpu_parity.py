"""GPU parity of the HIP path against the CPU oracle, stage by stage on shared
generator inputs, closed-loop on integer-valued inputs (every score exact in
fp32, so every stage must match bit for bit), and the error paths.

Bars: bit-exact for masks, exploration draws, block lists, top-K index sets
and EMA state.  Indexer scores: fp32 keys with fp32 queries (the exact mode)
bit-exact against the oracle's canonical fp32 order; bf16 and fp8 keys within
1e-3 and 2e-2 relative to max(|z|, 1e-3 rms(z)) (the contract) and, tighter,
within the per-slot error bound of tests/score_bound.py (the query's E4M3
terms and fp32 accumulation), which a lost query term breaks."""
import numpy as np
import pytest
import torch

import spin_synth as G
from oracle import spin_oracle as O
from tests.gpu_util import DEV, banner, device_keys, make_layer, np_bits, z_close
from tests.harness import build_layer, run_oracle
from tests.score_bound import check_bound, score_bound

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-3, "fp8": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_indexer_spin_amd import _lib
    return _lib.load()


def api():
    from sparse_attention_indexer_spin_amd import api as A
    return A


def _batch(ctx, qpos, step, rows, max_blocks, n_pages=1, req=None):
    A = api()
    R = len(ctx)
    t = lambda x: torch.as_tensor(np.asarray(x), dtype=torch.int32, device=DEV)
    keep = dict(ctx=t(ctx), qpos=t(qpos), step=t(step),
                req=t(np.arange(R) if req is None else req), err=torch.zeros(1, dtype=torch.int32,
                                                                              device=DEV))
    bt = A.batch(ctx_len=keep["ctx"], q_pos=keep["qpos"], step=keep["step"], req_id=keep["req"],
                 n_rows=rows, max_blocks=max_blocks, n_pages=n_pages, err=keep["err"])
    return bt, keep


# ---------------------------------------------------------------------------
# stage 1: predict
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("rows", [1, 2, 3, 4])
@pytest.mark.parametrize("combine", ["max", "sum"])
def test_predict_parity(rows, combine):
    banner(f"predict rows={rows} combine={combine}")
    A = api()
    ctx = [4096, 4000, 130, 64, 1]
    mb = 64
    qpos = [c + 7 for c in ctx]
    V, D = G.make_ema_state(len(ctx), 64 * mb, 4096 + 64, seed=11, ties=True, zero_frac=0.2)
    bt, keep = _batch(ctx, qpos, [3] * len(ctx), rows, mb)
    cfg = A.config(topk=512, sparsity_bp=4000, combine=combine)
    S = torch.full((len(ctx), rows, mb), -7.0, device=DEV)
    A.spin_predict_blocks(cfg, bt, V.to(DEV), D.to(DEV), S)
    S = S.cpu().numpy()
    for r, N in enumerate(ctx):
        B = O.n_blocks(N)
        for row in range(rows):
            want = O.predict_block_scores(V[r].numpy(), D[r].numpy(), N, qpos[r] + row, combine)
            assert np.array_equal(S[r, row, :B], want), (r, row)
            assert (S[r, row, B:] == -7.0).all()
    assert int(keep["err"].item()) == 0


def _signed_state(ctx, mb, d_cap, seed):
    """V of mixed sign (every third request all negative) with V = 0 past each
    context end, D non-negative, and the V block maxima over all 64 slots."""
    V, D = G.make_ema_state(len(ctx), 64 * mb, d_cap, seed=seed, ties=True, zero_frac=0.2)
    for r, N in enumerate(ctx):
        if r % 3 == 0:
            V[r] = -V[r] - 1.0
        V[r, N:] = 0.0
    vmax = V.view(len(ctx), mb, 64).amax(dim=2)
    return V, D, vmax


@pytest.mark.parametrize("rows", [1, 2, 3, 4])
@pytest.mark.parametrize("combine", ["max", "sum"])
def test_predict_parity_vmax(rows, combine):
    """With the V block maxima (max combine: one float per block instead of 64
    V values, the last block read in full) S still equals the oracle's."""
    banner(f"predict vmax rows={rows} combine={combine}")
    A = api()
    ctx = [4096, 4000, 130, 64, 1, 4095]
    mb = 64
    qpos = [c + 7 for c in ctx]
    V, D, vmax = _signed_state(ctx, mb, 4096 + 64, seed=31)
    bt, keep = _batch(ctx, qpos, [3] * len(ctx), rows, mb)
    cfg = A.config(topk=512, sparsity_bp=4000, combine=combine)
    S = torch.full((len(ctx), rows, mb), -7.0, device=DEV)
    A.spin_predict_blocks(cfg, bt, V.to(DEV), D.to(DEV), S, v_max=vmax.to(DEV))
    S = S.cpu().numpy()
    for r, N in enumerate(ctx):
        B = O.n_blocks(N)
        for row in range(rows):
            want = O.predict_block_scores(V[r].numpy(), D[r].numpy(), N, qpos[r] + row, combine)
            assert np.array_equal(S[r, row, :B], want), (r, row)
    assert int(keep["err"].item()) == 0


@pytest.mark.parametrize("rows", [1, 4])
def test_ema_keeps_vmax(rows):
    """The EMA update refreshes the block maxima of the blocks it updates: after
    it, every block's entry equals the max of V over its 64 slots."""
    banner(f"ema vmax rows={rows}")
    A = api()
    ctx = [131072, 9000, 4096 + 33, 64, 1]
    R, mb = len(ctx), 2048
    V, D, vmax = _signed_state(ctx, mb, 131072 + 64, seed=41)
    sel, n_sel = G.make_selection(R, torch.tensor([O.n_blocks(c) for c in ctx]), mb, 0.5, seed=6)
    zin = G.make_scores((R, rows, 64 * mb), seed=42, signed=True)
    g = torch.Generator().manual_seed(7)
    n_valid = torch.randint(1, rows + 1, (R,), generator=g, dtype=torch.int32)
    bt, keep = _batch(ctx, [c + 11 for c in ctx], [4] * R, rows, mb)
    cfg = A.config(topk=2048, sparsity_bp=4000, ema_alpha=0.9)
    Vd, Dd, Md = V.to(DEV), D.to(DEV), vmax.to(DEV)
    A.spin_ema_update(cfg, bt, zin.to(DEV), sel.to(DEV), n_sel.to(DEV), Vd, Dd,
                      n_valid=n_valid.to(DEV), v_max=Md)
    want = Vd.view(R, mb, 64).amax(dim=2)
    assert torch.equal(Md, want)
    assert not torch.equal(Md, vmax.to(DEV))  # the update did move some maxima
    assert int(keep["err"].item()) == 0


# ---------------------------------------------------------------------------
# stage 2: select (+ union)
# ---------------------------------------------------------------------------
# block capacities from 1 to 8,192: every blocks-per-thread instantiation of
# the selection, full and ragged contexts, 1-4 rows
@pytest.mark.parametrize("rows,mb,ctx", [(1, 64, [4096, 4000, 130, 64, 1]),
                                         (4, 64, [4096, 2000, 65]),
                                         (1, 1, [64, 1, 30]),
                                         (2, 100, [6400, 6000, 129]),
                                         (1, 250, [16000, 15999, 4000]),
                                         (3, 500, [32000, 31000, 64 * 7]),
                                         (1, 1000, [64000, 40001]),
                                         (1, 2048, [131072, 131000, 70001, 200]),
                                         (4, 2048, [131072, 99999]),
                                         (1, 4096, [262144, 70000]),
                                         (2, 8192, [524288, 300001])])
@pytest.mark.parametrize("step", [0, 1, 9])
def test_select_parity(rows, mb, ctx, step):
    banner(f"select rows={rows} mb={mb} step={step}")
    A = api()
    R = len(ctx)
    S = G.make_scores((R, rows, mb), seed=100 + step, ties=True)
    budget = torch.tensor([0] + [max(1, O.n_blocks(c) // 3) for c in ctx[1:]], dtype=torch.int32)
    for use_budget in (False, True):
        for sp, ex in ((4000, 500), (0, 500), (5000, 3000)):
            bt, keep = _batch(ctx, [c + 3 for c in ctx], [step] * R, rows, mb,
                              req=np.arange(R) * 7 + 1)
            cfg = A.config(topk=2048 if mb > 64 else 512, sparsity_bp=sp, explore_bp=ex,
                           layer=3, seed=0x1234_5678_5350_494E)
            code = torch.full((R, rows, mb), 9, dtype=torch.uint8, device=DEV)
            sel = torch.full((R, mb), -5, dtype=torch.int32, device=DEV)
            n_sel = torch.zeros(R, dtype=torch.int32, device=DEV)
            A.spin_select_blocks(cfg, bt, S.to(DEV), code, sel, n_sel,
                                 budget=budget.to(DEV) if use_budget else None)
            code, sel, n_sel = code.cpu().numpy(), sel.cpu().numpy(), n_sel.cpu().numpy()
            for r, N in enumerate(ctx):
                B = O.n_blocks(N)
                rows_codes = []
                for row in range(rows):
                    want = O.select_blocks(S[r, row, :B].numpy(), N, cfg.topk, sp, ex, step, 3,
                                           r * 7 + 1, 0x1234_5678_5350_494E,
                                           int(budget[r]) if use_budget else None)
                    assert np.array_equal(code[r, row, :B], want), (r, row, sp, use_budget)
                    rows_codes.append(want)
                u = O.union_blocks(rows_codes)
                assert n_sel[r] == len(u)
                assert np.array_equal(sel[r, :len(u)], u)
                assert (sel[r, len(u):] == -1).all()


# ---------------------------------------------------------------------------
# stage 3a: indexer score
# ---------------------------------------------------------------------------
def _small(key, q, rows=1, integer=False, N=(4096 + 200, 3000)):
    base = G.WORKLOADS["fp8_128k_b32"].scaled(batch=len(N), n_slots=max(N), n_slots_min=min(N),
                                              rows=rows, key_dtype=key, q_dtype=q, steps=3,
                                              topk=512)
    w = base
    li = build_layer(w, integer=integer)
    return li


@pytest.mark.parametrize("key,q", [("f32", "f32"), ("bf16", "bf16"), ("fp8", "bf16"),
                                   ("fp8", "f32")])
@pytest.mark.parametrize("integer", [False, True])
@pytest.mark.parametrize("rows", [1, 2, 3, 4])
def test_score_parity(key, q, integer, rows):
    banner(f"score key={key} q={q} integer={integer} rows={rows}")
    A = api()
    li = _small(key, q, rows=rows, integer=integer)
    w = li.w
    R, mb = w.batch, w.max_blocks
    sel, n_sel = G.make_selection(R, torch.tensor([O.n_blocks(int(c)) for c in li.ctx]), mb,
                                  0.5, seed=5)
    pages, scale, pt = device_keys(li)
    bt, keep = _batch(li.ctx.numpy(), li.pos[0].numpy(), [1] * R, rows, mb, n_pages=pages.shape[0])
    cfg = A.config(topk=512, sparsity_bp=4000, key_dtype=pages.dtype,
                   q_dtype=torch.bfloat16 if q == "bf16" else torch.float32)
    z = torch.full((R, rows, 64 * mb), -3.0, device=DEV)
    qd = li.q[1].to(DEV).contiguous()
    A.spin_sparse_index_score(cfg, bt, qd, li.weights.to(DEV), pages, scale, pt, sel.to(DEV),
                              n_sel.to(DEV), z)
    z = z.cpu().numpy()
    np_pages = li.np_pages()
    np_scale = None if li.keys.scale is None else li.keys.scale.numpy()
    for r in range(R):
        N = int(li.ctx[r])
        blocks = sel[r, :int(n_sel[r])].numpy()
        slots = O.union_slots(blocks, N)
        keys = O.gather_keys(np_pages, li.keys.page_table[r].numpy(), slots, key, np_scale)
        qr = O.decode_q(li.np_q(1)[r], q)
        comp = (np.searchsorted(blocks, slots // 64) * 64 + slots % 64)
        if key == "fp8":
            phys = li.keys.page_table[r].numpy()[slots // 64]
            sc = np_scale[phys, slots % 64].astype(np.float64)
            unscaled = O.gather_keys(np_pages, li.keys.page_table[r].numpy(), slots, key,
                                     np.ones_like(np_scale))
        for row in range(rows):
            want = O.index_scores(qr[row], li.weights[r, row].numpy(), keys)
            got = z[r, row, comp]
            if integer:
                assert np.array_equal(got.astype(np.float64), want), (r, row)
            elif key == "f32":   # the exact mode: the canonical fp32 order, bit for bit
                exact = O.index_scores_exact_f32(qr[row], li.weights[r, row].numpy(), keys)
                assert np.array_equal(got, exact), (r, row)
            else:
                ok, worst = z_close(got, want, TOL[key])
                assert ok, (r, row, worst)
                if key == "fp8":
                    b = score_bound(qr[row], li.weights[r, row].numpy(), unscaled, sc, key, q)
                else:
                    b = score_bound(qr[row], li.weights[r, row].numpy(), keys, None, key, q)
                ok, worst = check_bound(got, want, b)
                assert ok, ("bound", r, row, worst)
            # slots past the context end of a scored block read as 0
            tail = np.setdiff1d(np.arange(len(blocks) * 64), comp)
            assert (z[r, row, tail] == 0).all()
    assert int(keep["err"].item()) == 0


@pytest.mark.parametrize("rows", [1, 3])
def test_score_parity_more_requests_than_waves(rows):
    """3,000 short requests: more requests than the fp8 kernel has waves, so a
    wave's range crosses requests and the query is reloaded inside the loop
    (with several rows, the per-row-wave kernel's path for many requests)."""
    banner(f"score: more requests than waves, rows={rows}")
    A = api()
    li = _small("fp8", "bf16", rows=rows, N=tuple(64 + (r * 37) % 200 for r in range(3000)))
    w = li.w
    R, mb = w.batch, w.max_blocks
    sel, n_sel = G.make_selection(R, torch.tensor([O.n_blocks(int(c)) for c in li.ctx]), mb,
                                  0.5, seed=7)
    pages, scale, pt = device_keys(li)
    bt, keep = _batch(li.ctx.numpy(), li.pos[0].numpy(), [1] * R, rows, mb,
                      n_pages=pages.shape[0])
    cfg = A.config(topk=512, sparsity_bp=4000, key_dtype=pages.dtype, q_dtype=torch.bfloat16)
    z = torch.full((R, rows, 64 * mb), -3.0, device=DEV)
    A.spin_sparse_index_score(cfg, bt, li.q[1].to(DEV).contiguous(), li.weights.to(DEV), pages,
                              scale, pt, sel.to(DEV), n_sel.to(DEV), z)
    z = z.cpu().numpy()
    np_pages, np_scale = li.np_pages(), li.keys.scale.numpy()
    q_all = li.np_q(1)
    for r in range(0, R, 7 if rows > 1 else 1):
        N = int(li.ctx[r])
        blocks = sel[r, :int(n_sel[r])].numpy()
        slots = O.union_slots(blocks, N)
        keys = O.gather_keys(np_pages, li.keys.page_table[r].numpy(), slots, "fp8", np_scale)
        comp = np.searchsorted(blocks, slots // 64) * 64 + slots % 64
        phys = li.keys.page_table[r].numpy()[slots // 64]
        unscaled = O.gather_keys(np_pages, li.keys.page_table[r].numpy(), slots, "fp8",
                                 np.ones_like(np_scale))
        for row in range(rows):
            qd = O.decode_q(q_all[r], "bf16")[row]
            want = O.index_scores(qd, li.weights[r, row].numpy(), keys)
            ok, worst = z_close(z[r, row, comp], want, TOL["fp8"])
            assert ok, (r, row, worst)
            b = score_bound(qd, li.weights[r, row].numpy(), unscaled,
                            np_scale[phys, slots % 64].astype(np.float64), "fp8", "bf16")
            ok, worst = check_bound(z[r, row, comp], want, b)
            assert ok, ("bound", r, row, worst)
    assert int(keep["err"].item()) == 0


@pytest.mark.parametrize("rows", [2, 4])
def test_score_rows_kernels_agree(rows):
    """Several verifier rows: the kernel that scores a page for all rows in one
    wave (at most 64 requests) and the one with a wave per row (used past 64
    requests) make the same arithmetic in the same order, so the first 40
    requests of a 70-request batch score the same bits either way."""
    banner(f"score: all-rows and per-row-wave kernels agree, rows={rows}")
    A = api()
    li = _small("fp8", "bf16", rows=rows, N=tuple(700 + (r * 997) % 9000 for r in range(70)))
    w = li.w
    R, mb = w.batch, w.max_blocks
    sel, n_sel = G.make_selection(R, torch.tensor([O.n_blocks(int(c)) for c in li.ctx]), mb,
                                  0.5, seed=11)
    pages, scale, pt = device_keys(li)
    q, wts = li.q[1].to(DEV).contiguous(), li.weights.to(DEV)
    cfg = A.config(topk=512, sparsity_bp=4000, key_dtype=pages.dtype, q_dtype=torch.bfloat16)
    zs = []
    for n in (R, 40):
        bt, keep = _batch(li.ctx.numpy()[:n], li.pos[0].numpy()[:n], [1] * n, rows, mb,
                          n_pages=pages.shape[0])
        z = torch.full((n, rows, 64 * mb), -3.0, device=DEV)
        A.spin_sparse_index_score(cfg, bt, q[:n].contiguous(), wts[:n].contiguous(), pages, scale,
                                  pt[:n].contiguous(), sel[:n].to(DEV).contiguous(),
                                  n_sel[:n].to(DEV).contiguous(), z)
        torch.cuda.synchronize()
        assert int(keep["err"].item()) == 0
        zs.append(z[:40].cpu())
    assert torch.equal(zs[0], zs[1])


# ---------------------------------------------------------------------------
# stage 3b: top-K
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("K", [64, 512, 2048, 100000])
@pytest.mark.parametrize("ties", [False, True])
def test_topk_parity(K, ties):
    """Exact for any threshold hint: zeroed workspace (everything passes the
    filter), the hint the previous call left (fast path), and a hint above
    every key (nothing passes: fallback)."""
    banner(f"topk K={K} ties={ties}")
    A = api()
    ctx = [131072, 70001, 4096 + 5, 64]
    R, mb, rows = len(ctx), 2048, 2
    sel, n_sel = G.make_selection(R, torch.tensor([O.n_blocks(c) for c in ctx]), mb, 0.6, seed=9)
    zin = G.make_scores((R, rows, 64 * mb), seed=K + ties, ties=ties, signed=True)
    bt, keep = _batch(ctx, [c + 1 for c in ctx], [2] * R, rows, mb)
    Kc = min(K, 8192)
    cfg = A.config(topk=Kc, sparsity_bp=4000)
    ws = torch.zeros(A.workspace_bytes(cfg, R, rows, mb), dtype=torch.uint8, device=DEV)
    want = {}
    for r, N in enumerate(ctx):
        blocks = sel[r, :int(n_sel[r])].numpy()
        slots = O.union_slots(blocks, N)
        comp = np.searchsorted(blocks, slots // 64) * 64 + slots % 64
        for row in range(rows):
            want[r, row] = O.topk_slots(zin[r, row].numpy()[comp], slots, Kc)
    zd, seld, nsd = zin.to(DEV), sel.to(DEV), n_sel.to(DEV)
    for attempt in ("zero hint", "carried hint", "carried hint again", "hint above all"):
        if attempt == "hint above all":
            ws[: 4 * R * rows] = 0xFF
        out = torch.full((R, rows, Kc), -9, dtype=torch.int32, device=DEV)
        A.spin_topk(cfg, bt, zd, seld, nsd, out, workspace=ws)
        out = out.cpu().numpy()
        for r in range(R):
            for row in range(rows):
                assert np.array_equal(out[r, row], want[r, row]), (attempt, r, row)


def test_topk_tracks_drifting_scores():
    """Scores that drift from call to call (as in decoding): every call exact."""
    banner("topk drift")
    A = api()
    ctx = [131072, 90000]
    R, mb, rows = 2, 2048, 1
    sel, n_sel = G.make_selection(R, torch.tensor([O.n_blocks(c) for c in ctx]), mb, 0.6, seed=3)
    cfg = A.config(topk=2048, sparsity_bp=4000)
    ws = torch.zeros(A.workspace_bytes(cfg, R, rows, mb), dtype=torch.uint8, device=DEV)
    bt, keep = _batch(ctx, [c + 1 for c in ctx], [2] * R, rows, mb)
    base = G.make_scores((R, rows, 64 * mb), seed=77)
    for step in range(8):
        zin = base * (1.0 + 0.15 * step) + G.make_scores((R, rows, 64 * mb), seed=step) * 0.3
        out = torch.full((R, rows, 2048), -9, dtype=torch.int32, device=DEV)
        A.spin_topk(cfg, bt, zin.to(DEV), sel.to(DEV), n_sel.to(DEV), out, workspace=ws)
        out = out.cpu().numpy()
        for r, N in enumerate(ctx):
            blocks = sel[r, :int(n_sel[r])].numpy()
            slots = O.union_slots(blocks, N)
            comp = np.searchsorted(blocks, slots // 64) * 64 + slots % 64
            assert np.array_equal(out[r, 0], O.topk_slots(zin[r, 0].numpy()[comp], slots, 2048))


# ---------------------------------------------------------------------------
# stage 4: EMA with deferred replay
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("rows", [1, 4])
def test_ema_parity(rows):
    banner(f"ema rows={rows}")
    A = api()
    ctx = [131072, 9000, 4096 + 33, 64, 1]
    R, mb = len(ctx), 2048
    d_cap = 131072 + 64
    sel, n_sel = G.make_selection(R, torch.tensor([O.n_blocks(c) for c in ctx]), mb, 0.5, seed=4)
    V, D = G.make_ema_state(R, 64 * mb, d_cap, seed=21)
    zin = G.make_scores((R, rows, 64 * mb), seed=22)
    qpos = [c + 11 for c in ctx]
    g = torch.Generator().manual_seed(5)
    n_valid = torch.randint(1, rows + 1, (R,), generator=g, dtype=torch.int32)
    bt, keep = _batch(ctx, qpos, [4] * R, rows, mb)
    cfg = A.config(topk=2048, sparsity_bp=4000, ema_alpha=0.9)
    Vd, Dd = V.to(DEV), D.to(DEV)
    A.spin_ema_update(cfg, bt, zin.to(DEV), sel.to(DEV), n_sel.to(DEV), Vd, Dd,
                      n_valid=n_valid.to(DEV))
    Vg, Dg = Vd.cpu().numpy(), Dd.cpu().numpy()
    for r, N in enumerate(ctx):
        blocks = sel[r, :int(n_sel[r])].numpy()
        slots = O.union_slots(blocks, N)
        comp = np.searchsorted(blocks, slots // 64) * 64 + slots % 64
        v, d = V[r].numpy().copy(), D[r].numpy().copy()
        O.ema_update(v, d, zin[r].numpy()[:, comp], slots, qpos[r], int(n_valid[r]), 0.9)
        assert np.array_equal(Vg[r], v), r
        assert np.array_equal(Dg[r], d), r
    assert int(keep["err"].item()) == 0


# ---------------------------------------------------------------------------
# closed loop on integer-valued inputs: every stage bit-exact, every step
# ---------------------------------------------------------------------------
CLOSED = {
    "f32": G.WORKLOADS["tiny_f32_4k"].scaled(batch=2, n_slots=4096 + 100, n_slots_min=4000,
                                             steps=8),
    "bf16": G.WORKLOADS["bf16_64k_b16"].scaled(batch=3, n_slots=8192 + 64, n_slots_min=5000,
                                               steps=8, topk=512),
    "fp8": G.WORKLOADS["fp8_128k_b32"].scaled(batch=3, n_slots=8192, n_slots_min=6000, steps=8,
                                              topk=512),
    "fp8_mtp": G.WORKLOADS["fp8_128k_b32_mtp4"].scaled(batch=3, n_slots=6000, n_slots_min=4500,
                                                       steps=8, topk=256),
}


@pytest.mark.parametrize("name,vmax", [(n, False) for n in CLOSED] + [("fp8", True),
                                                                      ("fp8_mtp", True)])
@pytest.mark.parametrize("deferred", [False, True])
def test_closed_loop_exact(name, vmax, deferred):
    """vmax: the layer keeps the V block maxima and predict reads them."""
    banner(f"closed loop {name} vmax={vmax} deferred={deferred}")
    w = CLOSED[name]
    li = build_layer(w, integer=True)
    sp = w.sparsity_bp[0]
    ref, _ = run_oracle(li, w.steps, sp)
    lay = make_layer(li, sp, vmax_cache=vmax)
    pages, scale, pt = device_keys(li)
    W = li.weights.to(DEV)
    for s in range(w.steps):
        assert torch.equal(lay.q_pos.cpu(), li.pos[s].to(torch.int32))
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
    _, st = run_oracle(li, w.steps, sp)
    Vg, Dg = lay.V.cpu().numpy(), lay.D.cpu().numpy()
    for r in range(w.batch):
        N = int(li.ctx[r])
        assert np.array_equal(Vg[r, :N], st[r].V[:N])
        dl = min(Dg.shape[1], st[r].D.shape[0])
        assert np.array_equal(Dg[r, :dl], st[r].D[:dl])
    assert int(lay.err.item()) == 0


# ---------------------------------------------------------------------------
# realistic inputs, closed loop on the tiny fp32 workload: exact mode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("combine", ["sum", "max"])
def test_tiny_f32_closed_loop_exact(combine):
    """The tiny workload on its own Gaussian inputs (fp32 keys and queries,
    the exact mode): every one of its 32 steps equals the closed-loop oracle
    bit for bit -- block masks and exploration draws, the scored union, every
    score, top-K, and V and D after the step.  combine "sum" is the
    workload's rule as written, "max" the paper's Eq. 1."""
    banner(f"tiny f32 closed loop exact combine={combine}")
    w = G.WORKLOADS["tiny_f32_4k"]
    li = build_layer(w)
    ref, states = run_oracle(li, w.steps, w.sparsity_bp[0], combine=combine,
                             keep_state_history=True)
    lay = make_layer(li, w.sparsity_bp[0], combine=combine)
    pages, scale, pt = device_keys(li)
    W = li.weights.to(DEV)
    N = int(li.ctx[0])
    B = O.n_blocks(N)
    n_explored = 0
    for s in range(w.steps):
        lay.step(li.q[s].to(DEV).contiguous(), W, pages, scale, pt)
        x = ref[s][0]
        code = lay.row_code.cpu().numpy()[0, :, :B]
        assert np.array_equal(code, x["codes"]), s
        n_explored += int((code == O.CODE_EXPLORED).sum())
        n_sel = int(lay.n_sel[0])
        assert n_sel == len(x["sel"]) and np.array_equal(lay.sel.cpu().numpy()[0, :n_sel],
                                                           x["sel"]), s
        comp = np.searchsorted(x["sel"], x["slots"] // 64) * 64 + x["slots"] % 64
        assert np.array_equal(lay.z.cpu().numpy()[0][:, comp], x["z32"]), s
        assert np.array_equal(lay.topk_idx.cpu().numpy()[0], x["topk"]), s
        V, D = x["state_after"]
        assert np.array_equal(lay.V.cpu().numpy()[0, :N], V[:N]), s
        dl = min(lay.D.shape[1], D.shape[0])
        assert np.array_equal(lay.D.cpu().numpy()[0, :dl], D[:dl]), s
    assert n_explored > 0
    assert int(lay.err.item()) == 0


# ---------------------------------------------------------------------------
# error paths and determinism
# ---------------------------------------------------------------------------
def test_device_error_word_and_skip():
    banner("device error paths")
    w = CLOSED["fp8"]
    li = build_layer(w, integer=True)
    lay = make_layer(li, 4000)
    pages, scale, pt = device_keys(li)
    ctx = li.ctx.clone()
    ctx[1] = 64 * w.max_blocks + 1               # context beyond capacity
    qpos = li.pos[0].clone()
    qpos[2] = int(ctx[2]) - 5                    # query before the context end
    lay.set_requests(ctx.to(DEV), qpos.to(DEV))
    lay.step(li.q[0].to(DEV).contiguous(), li.weights.to(DEV), pages, scale, pt)
    err = int(lay.err.item())
    assert err & 1 and err & 2
    assert (lay.topk_idx[1:].cpu() == -1).all()
    assert lay.n_sel[1:].cpu().tolist() == [0, 0]
    # a page id outside the pool
    lay2 = make_layer(li, 4000)
    bad_pt = pt.clone()
    bad_pt[0, 3] = pages.shape[0] + 10
    lay2.step(li.q[0].to(DEV).contiguous(), li.weights.to(DEV), pages, scale, bad_pt)
    assert int(lay2.err.item()) & 4


def test_repeat_runs_bit_identical():
    banner("determinism")
    w = CLOSED["fp8_mtp"]
    li = build_layer(w)
    outs = []
    for _ in range(2):
        lay = make_layer(li, 4000)
        pages, scale, pt = device_keys(li)
        for s in range(4):
            lay.step(li.q[s].to(DEV).contiguous(), li.weights.to(DEV), pages, scale, pt,
                     n_valid=li.accept[s].to(DEV))
        outs.append([t.cpu().clone() for t in (lay.z, lay.topk_idx, lay.V, lay.D, lay.row_code)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
