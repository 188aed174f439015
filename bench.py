"""Benchmark of the SPIN decode step on one MI355X.

Workload (default): 32 requests x 131,072 compressed slots (~512K tokens at 4x
compression, 2,048 blocks of 64), fp8 E4M3 keys with per-slot fp32 scales,
bf16 queries, 64 heads x 128 dims, top-K 2048, 40 % target block sparsity with
a 5 % exploration share, EMA decay 0.9.  A "step" is one pass of the whole hot
path: predict -> select -> sparse indexer score -> top-K -> EMA -> advance,
each launched through the C ABI on the current stream, inputs resident in HBM.

Prints one JSON line.  `value` = indexer keys scored per second of whole-step
time (one spin_step call per step).  By default (`--cache rotate`) the bench
steps 8 independent copies of the workload (own key pages, EMA state and
buffers; the same data) round robin back to back, as the layers of a model
run: when a copy steps again, the other copies have streamed 7 x its pages
(~2.4 GB) and 7 x its ~51 MB of EMA state and step buffers through the L2s and
the 256 MB MALL, so its pages and its state come from HBM, and no host sync or
event sits between steps.  (The page loads are non-temporal; with 4 copies
the state of all copies, ~205 MB, stays in the MALL, which a model with tens
of layers does not allow.)  The two other protocols are
reported beside it: `cold` times each step alone after a 1 GiB read (adds the
event and launch latency of an isolated step), `warm` steps one copy back to
back (the MALL keeps part of the previous step's pages).  `roofline` is the
score kernel's algorithmic HBM bytes per launch / its mean launch duration
(the stage launched round robin over the copies between two HIP events on
the step's stream, on the last timed step's selection) against 8 TB/s, with
`traffic` taken from the committed FETCH_SIZE/WRITE_SIZE summary when it was
measured on the current kernel source.  `cpu_baseline` times the CPU oracle
on whole requests of the same workload for about 10 s.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import spin_synth as G  # noqa: E402

HBM_PEAK_GBS = 8000.0
FP8_MFMA_PEAK_TFLOPS = 5000.0  # dense fp8 MFMA, MI355X


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="fp8_128k_b32")
    ap.add_argument("--sparsity-bp", type=int, default=None)
    ap.add_argument("--sweep", action="store_true",
                    help="--stack: time the workload's sparsity sweep and fit t = a(1-rho) + c")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the fixed-cost section (the sparsity sweep with its fits)")
    ap.add_argument("--sweep-runs", type=int, default=3)
    ap.add_argument("--stage-reps", type=int, default=20)
    ap.add_argument("--runs", type=int, default=3,
                    help="rotate: timed runs of the steps (each from a reset) and of the stage "
                         "loop; the line reports their median and spread")
    ap.add_argument("--cache", choices=["rotate", "cold", "warm"], default="rotate",
                    help="rotate: step --copies independent copies of the workload round robin "
                         "back to back (each step's pages were evicted by the others, as between "
                         "the layers of a model); cold: a 1 GiB read before every timed step and "
                         "stage launch, each timed alone; warm: one copy back to back")
    ap.add_argument("--copies", type=int, default=8,
                    help="rotate: copies of the workload; at 8 the other copies' EMA state and "
                         "buffers (~360 MB) also evict a copy's own from the 256 MB MALL")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-max-requests", type=int, default=32)
    ap.add_argument("--stack", action="store_true",
                    help="multi-layer workloads: time whole decode steps of every layer, one "
                         "spin_step per layer on one stream and the spin_stack schedule (plans "
                         "on a side stream)")
    ap.add_argument("--budget-policy", choices=["none", "proportional", "minimax"],
                    default="proportional",
                    help="--stack: per-layer block budgets re-sized from a dense probe every "
                         "--probe-period steps (the multi-layer workload states the "
                         "proportional rule), timed beside the uniform runs")
    ap.add_argument("--probe-period", type=int, default=8)
    ap.add_argument("--budget-drift-bp", type=int, default=0,
                    help="--stack with budgets: re-size the levels only when a layer's miss "
                         "curve moved by more than this many basis points since the last "
                         "re-sizing (0: at every probe)")
    ap.add_argument("--stack-layers", type=int, default=8,
                    help="--stack on a one-layer workload: that many independent layers of it")
    ap.add_argument("--miss-eval", action="store_true",
                    help="top-K miss rate (share of the dense top-K slots outside the scored "
                         "blocks) of the method's design variants, closed loop on the workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run three plain 1 GiB device-to-device copies (the reference "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


class Inputs:
    """Synthetic workload resident on the GPU."""

    def __init__(self, w: G.Workload, n_steps: int, dev="cuda"):
        self.w = w
        self.ctx = G.context_lengths(w)
        self.keys = G.make_keys(w, 0, dev, self.ctx)
        self.weights = G.make_weights(w, 0, dev)
        self.pos, self.accept = G.make_schedule(w, self.ctx, n_steps)
        q = G.make_queries(w, 0, self.keys, self.pos, dev)
        self.q = G.cast_queries(w, q).contiguous()
        del q
        self.accept_dev = self.accept.to(dev)
        torch.cuda.synchronize()


def algorithmic_score_bytes(w: G.Workload, slots: float, n_blocks_sel: float):
    """Bytes the score stage must move per launch (skipped blocks not counted):
    each scored slot's key (+ scale) once, its z once per verifier row, the
    block list and page-table entries, and every row's query and weights."""
    kb = {"fp8": 128 + 4, "bf16": 256, "f32": 512}[w.key_dtype]
    qb = {"bf16": 2, "f32": 4}[w.q_dtype]
    per_slot = kb + 4 * w.rows                        # key (+ scale) + z writes
    per_block = 8                                     # sel entry + page-table entry
    per_req = w.rows * 64 * (128 * qb + 4)            # q and w
    return slots * per_slot + n_blocks_sel * per_block + w.batch * per_req


class Evictor:
    """Reads a 1 GiB buffer: afterwards the L2s and the 256 MB MALL hold clean,
    unrelated lines, as after the other layers of a model ran."""

    def __init__(self, dev="cuda"):
        self.buf = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device=dev)

    def __call__(self):
        self.buf.sum()


# Untimed calls before a stage is timed back to back.  When the load changes
# (say from latency-bound launches to the HBM-bound score kernel) the chip's
# power management takes ~15-20 ms to settle: the score launch then runs
# ~60.5 us for two rounds over the copies, 63-71 us for the next ~20 rounds
# and ~60.5 us again from ~15 ms on.  Timing starts after the transient.
WARM_MS = 25.0


def _timed_us(fn, reps: int, stream, evict=None, warm_log=None) -> float:
    """Mean duration of `fn` over `reps` launches (HIP events on `stream`):
    back to back, after untimed calls for WARM_MS of device time (and at
    least reps / 4 of them), or each one after `evict` (outside its events),
    after reps / 4 untimed calls.  `warm_log` (a list) receives the number
    of untimed calls, which locates the timed launches in a kernel trace."""
    n, t_end = 0, time.perf_counter() + (WARM_MS * 1e-3 if evict is None else 0.0)
    while n < max(1, reps // 4) or time.perf_counter() < t_end:
        fn()
        n += 1
        if n % 4 == 0:  # keep the host within a few calls of the device
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    if warm_log is not None:
        warm_log.append(n)
    if evict is None:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        evict()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / reps * 1e3


def run_gpu(inp: Inputs, sparsity_bp: int, steps: int, warmup: int, stage_reps: int = 0,
            evict=None):
    """Time `steps` decode steps (one spin_step call each) after `warmup` untimed
    ones; with stage_reps > 0, then time each stage alone on the last step's inputs.
    With `evict`, every timed step and stage launch runs after it (cold caches)."""
    from sparse_attention_indexer_spin_amd import SpinLayer, api
    w = inp.w
    lay = SpinLayer(batch=w.batch, max_blocks=w.max_blocks, d_cap=G.d_capacity(w, steps + warmup),
                    topk=w.topk, sparsity_bp=sparsity_bp, n_rows=w.rows,
                    explore_bp=w.explore_bp, ema_alpha=w.alpha, combine=w.combine,
                    key_dtype={"fp8": torch.uint8, "bf16": torch.bfloat16,
                               "f32": torch.float32}[w.key_dtype],
                    q_dtype=torch.bfloat16 if w.q_dtype == "bf16" else torch.float32)
    lay.set_requests(inp.ctx.cuda(), inp.pos[0].cuda())
    lay.reset()
    pages, scale, pt = inp.keys.pages, inp.keys.scale, inp.keys.page_table
    bt = lay.batch(pages.shape[0])
    stream = torch.cuda.current_stream()
    nv = [inp.accept_dev[s] if w.rows > 1 else None for s in range(warmup + steps)]
    ios = [lay.make_io(inp.q[s], inp.weights, pages, scale, pt, n_valid=nv[s])
           for s in range(warmup + steps)]
    for s in range(warmup):
        api.spin_step(lay.cfg, bt, ios[s])
    torch.cuda.synchronize()
    if evict is None:
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for s in range(warmup, warmup + steps):
            api.spin_step(lay.cfg, bt, ios[s])
        t1.record(stream)
        torch.cuda.synchronize()
        total_ms = t0.elapsed_time(t1)
    else:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for k, s in enumerate(range(warmup, warmup + steps)):
            evict()
            ev[k][0].record(stream)
            api.spin_step(lay.cfg, bt, ios[s])
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        total_ms = sum(a.elapsed_time(b) for a, b in ev)
    assert int(lay.err.item()) == 0, f"device error word {int(lay.err.item())}"
    n_sel = lay.n_sel.cpu().numpy().astype(np.int64)
    ctx = lay.ctx_len.cpu().numpy().astype(np.int64)
    # scored keys per step: the valid slots of the selected blocks of every row
    keys = int(np.minimum(n_sel * 64, ctx).sum()) * w.rows
    out = dict(total_ms=total_ms, ms_per_step=total_ms / steps, keys_per_step=keys,
               n_sel=int(n_sel.sum()))
    if stage_reps:
        # the last step's inputs: its selection is in lay.sel / lay.n_sel
        q = inp.q[warmup + steps - 1]
        last_nv = nv[-1]
        st = {
            "predict": lambda: api.spin_predict_blocks(lay.cfg, bt, lay.V, lay.D, lay.S,
                                                       v_max=lay.v_max),
            "select": lambda: api.spin_select_blocks(lay.cfg, bt, lay.S, lay.row_code, lay.sel,
                                                     lay.n_sel),
            "score": lambda: api.spin_sparse_index_score(lay.cfg, bt, q, inp.weights, pages,
                                                         scale, pt, lay.sel, lay.n_sel, lay.z),
            "topk": lambda: api.spin_topk(lay.cfg, bt, lay.z, lay.sel, lay.n_sel, lay.topk_idx,
                                          lay.workspace),
            "ema": lambda: api.spin_ema_update(lay.cfg, bt, lay.z, lay.sel, lay.n_sel, lay.V,
                                               lay.D, n_valid=last_nv, v_max=lay.v_max),
        }
        out["stage_us"] = {k: _timed_us(f, stage_reps, stream, evict) for k, f in st.items()}
        assert int(lay.err.item()) == 0, f"device error word {int(lay.err.item())}"
    return out


class StackInputs:
    """Per-layer synthetic inputs of a multi-layer workload, resident on the GPU."""

    def __init__(self, w: G.Workload, n_steps: int, dev="cuda"):
        self.w = w
        self.ctx = G.context_lengths(w)
        self.pos, self.accept = G.make_schedule(w, self.ctx, n_steps)
        self.keys, self.weights, self.q = [], [], []
        for l in range(w.layers):
            k = G.make_keys(w, l, dev, self.ctx)
            self.keys.append(k)
            self.weights.append(G.make_weights(w, l, dev))
            q = G.make_queries(w, l, k, self.pos, dev)
            self.q.append(G.cast_queries(w, q).contiguous())
            del q
        torch.cuda.synchronize()


def run_stack(inp: StackInputs, sparsity_bp: int, steps: int, warmup: int, evict=None,
              policy: str = "none", probe_period: int = 8,
              modes=("seq", "stack", "ema_stream", "one_stream"), drift_bp: int = 0):
    """Whole decode steps of every layer: (a) one spin_step per layer in layer
    order on the current stream, (b) one spin_stack_step (plans on a side
    stream).  Each mode on its own layer states from the same reset; each timed
    step after `evict` when given.  Both modes must agree bit for bit."""
    from sparse_attention_indexer_spin_amd import SpinLayer, SpinStack
    w = inp.w

    def layers():
        out = []
        for l in range(w.layers):
            lay = SpinLayer(batch=w.batch, max_blocks=w.max_blocks,
                            d_cap=G.d_capacity(w, steps + warmup), topk=w.topk,
                            sparsity_bp=sparsity_bp, n_rows=w.rows, explore_bp=w.explore_bp,
                            ema_alpha=w.alpha, combine=w.combine, key_dtype=torch.uint8,
                            q_dtype=torch.bfloat16, layer=l)
            lay.set_requests(inp.ctx.cuda(), inp.pos[0].cuda())
            lay.reset()
            out.append(lay)
        return out

    pages = [k.pages for k in inp.keys]
    scales = [k.scale for k in inp.keys]
    pts = [k.page_table for k in inp.keys]
    stream = torch.cuda.current_stream()

    def timed(step_fn, join=None):
        """Mean step time; `join` (if given) orders the main stream after work
        the step left on other streams, before the last end event."""
        for s in range(warmup):
            step_fn(s)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for k, s in enumerate(range(warmup, warmup + steps)):
            if evict is not None:
                evict()
            ev[k][0].record(stream)
            step_fn(s)
            if join is not None and (evict is not None or k == steps - 1):
                join()
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / steps

    seq, ms_seq = None, None
    if "seq" in modes:
        seq = layers()

        def seq_step(s):
            for l, lay in enumerate(seq):
                lay.step(inp.q[l][s], inp.weights[l], pages[l], scales[l], pts[l])

        ms_seq = timed(seq_step)
    def run_stack_mode(ema_stream, one_stream=False):
        lays = layers()
        stack = SpinStack(lays, ema_stream=ema_stream, one_stream=one_stream)

        def stack_step(s):
            if evict is not None:
                # the plans may not start before the timed region (they would
                # run beside the eviction read): order the side stream after main
                stack.inputs_changed()
            stack.step([inp.q[l][s] for l in range(w.layers)], inp.weights, pages, scales, pts)

        ms = timed(stack_step, join=stack.join)
        torch.cuda.synchronize()
        return ms, lays

    ms_stack, stk_layers = run_stack_mode(False)
    ms_stack_ema_stream, lays_ema_stream = (run_stack_mode(True) if "ema_stream" in modes
                                            else (None, None))
    ms_one_stream, lays_one_stream = (run_stack_mode(False, one_stream=True)
                                      if "one_stream" in modes else (None, None))
    budget = None
    if policy != "none":
        # the same schedule with per-layer budgets and dense probe steps; the
        # effective sparsity counts every selected block of every step
        bud_layers = layers()
        bstack = SpinStack(bud_layers, budget_policy=policy, probe_period=probe_period,
                           budget_drift_bp=drift_bp)
        sel_blocks = []

        def budget_step(s):
            if evict is not None:
                bstack.inputs_changed()
            bstack.step([inp.q[l][s] for l in range(w.layers)], inp.weights, pages, scales, pts)

        for s in range(warmup):
            budget_step(s)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for k, s in enumerate(range(warmup, warmup + steps)):
            if evict is not None:
                evict()
            ev[k][0].record(stream)
            budget_step(s)
            if evict is not None or k == steps - 1:
                bstack.join()
            ev[k][1].record(stream)
            sel_blocks.append(torch.stack([lay.n_sel for lay in bud_layers]).sum())
        torch.cuda.synchronize()
        ms_budget = sum(a.elapsed_time(b) for a, b in ev) / steps
        total_blocks = w.layers * int(sum(-(-int(c) // 64) for c in inp.ctx))
        chosen = float(torch.stack(sel_blocks).sum().item()) / steps
        budget = {"policy": policy, "probe_period": probe_period, "drift_bp": drift_bp,
                  "us_per_step": ms_budget * 1e3,
                  "us_per_step_layer": ms_budget * 1e3 / w.layers,
                  "effective_block_sparsity": 1.0 - chosen / total_blocks,
                  "levels_after_last_probe": bstack.levels_now(),
                  "probe_steps": [t for t in range(1, warmup + steps) if t % probe_period == 0]}
        for lay in bud_layers:
            assert int(lay.err.item()) == 0
    for other in (seq, lays_ema_stream, lays_one_stream):
        if other is None:
            continue
        for a, b in zip(other, stk_layers):
            assert torch.equal(a.topk_idx, b.topk_idx) and torch.equal(a.V, b.V), \
                "stack and sequential steps disagree"
            assert int(a.err.item()) == 0
    for b in stk_layers:
        assert int(b.err.item()) == 0
    keys = 0
    ctx = inp.ctx.numpy().astype(np.int64)
    n_sel = 0
    for lay in stk_layers:
        ns = lay.n_sel.cpu().numpy().astype(np.int64)
        keys += int(np.minimum(ns * 64, ctx).sum()) * w.rows
        n_sel += int(ns.sum())
    # the score launches of all layers round robin on their last selections
    # (each layer's pages evicted by the others', as in the stack), for the roofline
    from sparse_attention_indexer_spin_amd import api
    last = warmup + steps - 1
    bts = [lay.batch(pages[l].shape[0]) for l, lay in enumerate(stk_layers)]

    def score_round():
        for l, lay in enumerate(stk_layers):
            api.spin_sparse_index_score(lay.cfg, bts[l], inp.q[l][last], inp.weights[l],
                                        pages[l], scales[l], pts[l], lay.sel, lay.n_sel, lay.z)

    score_us = _timed_us(score_round, 5, stream, evict) / w.layers
    keys0 = keys // w.layers
    n_sel0 = n_sel // w.layers
    return dict(ms_seq=ms_seq, ms_stack=ms_stack, ms_stack_ema_stream=ms_stack_ema_stream,
                ms_one_stream=ms_one_stream,
                keys_per_step=keys, n_sel=n_sel,
                score_us_layer0=score_us, keys_layer0=keys0, n_sel_layer0=n_sel0,
                budget=budget)


def run_rotate(inp: Inputs, sparsity_bp: int, steps: int, warmup: int, stage_reps: int,
               copies: int, runs: int = 3):
    """`copies` independent copies of the workload -- own key pages (same data),
    EMA state and buffers -- stepped round robin back to back, as the layers of
    a model run: by the time a copy steps again, the others have streamed
    (copies - 1) x its pages and state through the L2s and the 256 MB MALL, and no host
    sync or event sits between two steps.  Per-step time = total / (steps x
    copies), the median over `runs` runs, each from a reset.  Stage timing
    likewise: each stage launched round robin over the copies, reps x copies
    launches between two events, the median over `runs` loops."""
    from sparse_attention_indexer_spin_amd import SpinLayer, api
    w = inp.w
    pages = [inp.keys.pages] + [inp.keys.pages.clone() for _ in range(copies - 1)]
    scales = [inp.keys.scale] + [None if inp.keys.scale is None else inp.keys.scale.clone()
                                 for _ in range(copies - 1)]
    pt = inp.keys.page_table
    lays = []
    for c in range(copies):
        lay = SpinLayer(batch=w.batch, max_blocks=w.max_blocks,
                        d_cap=G.d_capacity(w, steps + warmup), topk=w.topk,
                        sparsity_bp=sparsity_bp, n_rows=w.rows, explore_bp=w.explore_bp,
                        ema_alpha=w.alpha, combine=w.combine,
                        key_dtype={"fp8": torch.uint8, "bf16": torch.bfloat16,
                                   "f32": torch.float32}[w.key_dtype],
                        q_dtype=torch.bfloat16 if w.q_dtype == "bf16" else torch.float32)
        lay.set_requests(inp.ctx.cuda(), inp.pos[0].cuda())
        lay.reset()
        lays.append(lay)
    bts = [lay.batch(pages[c].shape[0]) for c, lay in enumerate(lays)]
    nv = [inp.accept_dev[s] if w.rows > 1 else None for s in range(warmup + steps)]
    ios = [[lay.make_io(inp.q[s], inp.weights, pages[c], scales[c], pt, n_valid=nv[s])
            for s in range(warmup + steps)] for c, lay in enumerate(lays)]
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    run_ms = []
    for run in range(runs):
        if run:
            for lay in lays:
                lay.set_requests(inp.ctx.cuda(), inp.pos[0].cuda())
                lay.reset()
        for s in range(warmup):
            for c in range(copies):
                api.spin_step(lays[c].cfg, bts[c], ios[c][s])
        torch.cuda.synchronize()
        t0.record(stream)
        for s in range(warmup, warmup + steps):
            for c in range(copies):
                api.spin_step(lays[c].cfg, bts[c], ios[c][s])
        t1.record(stream)
        torch.cuda.synchronize()
        run_ms.append(t0.elapsed_time(t1))
    total_ms = float(np.median(run_ms))
    for lay in lays:
        assert int(lay.err.item()) == 0, f"device error word {int(lay.err.item())}"
    for lay in lays[1:]:
        assert torch.equal(lay.topk_idx, lays[0].topk_idx), "copies disagree"
    n_sel = lays[0].n_sel.cpu().numpy().astype(np.int64)
    ctx = lays[0].ctx_len.cpu().numpy().astype(np.int64)
    keys = int(np.minimum(n_sel * 64, ctx).sum()) * w.rows
    out = dict(total_ms=total_ms, ms_per_step=total_ms / (steps * copies), keys_per_step=keys,
               n_sel=int(n_sel.sum()),
               ms_per_step_runs=[t / (steps * copies) for t in run_ms])
    # the same copies as the layers of one model through the multi-layer
    # schedule (plans on a side stream), from fresh state: per-layer step time
    from sparse_attention_indexer_spin_amd import SpinStack
    slays = []
    for c in range(copies):
        lay = SpinLayer(batch=w.batch, max_blocks=w.max_blocks,
                        d_cap=G.d_capacity(w, steps + warmup), topk=w.topk,
                        sparsity_bp=sparsity_bp, n_rows=w.rows, explore_bp=w.explore_bp,
                        ema_alpha=w.alpha, combine=w.combine,
                        key_dtype={"fp8": torch.uint8, "bf16": torch.bfloat16,
                                   "f32": torch.float32}[w.key_dtype],
                        q_dtype=torch.bfloat16 if w.q_dtype == "bf16" else torch.float32)
        lay.set_requests(inp.ctx.cuda(), inp.pos[0].cuda())
        lay.reset()
        slays.append(lay)
    stack = SpinStack(slays)
    if w.rows == 1:
        for s in range(warmup):
            stack.step([inp.q[s]] * copies, [inp.weights] * copies, pages, scales, [pt] * copies)
        torch.cuda.synchronize()
        t0.record(stream)
        for s in range(warmup, warmup + steps):
            stack.step([inp.q[s]] * copies, [inp.weights] * copies, pages, scales, [pt] * copies)
        t1.record(stream)
        torch.cuda.synchronize()
        for lay in slays:
            assert torch.equal(lay.topk_idx, lays[0].topk_idx), "stack and spin_step disagree"
        out["stack_ms_per_step"] = t0.elapsed_time(t1) / (steps * copies)
    del slays, stack
    if w.rows == 1:
        # the round of spin_steps over the copies captured in one HIP graph (as
        # a model captures its layers' decode step) and replayed
        gl = []
        for c in range(copies):
            lay = SpinLayer(batch=w.batch, max_blocks=w.max_blocks,
                            d_cap=G.d_capacity(w, steps + warmup + 1), topk=w.topk,
                            sparsity_bp=sparsity_bp, n_rows=1, explore_bp=w.explore_bp,
                            ema_alpha=w.alpha, combine=w.combine,
                            key_dtype={"fp8": torch.uint8, "bf16": torch.bfloat16,
                                       "f32": torch.float32}[w.key_dtype],
                            q_dtype=torch.bfloat16 if w.q_dtype == "bf16" else torch.float32)
            lay.set_requests(inp.ctx.cuda(), inp.pos[0].cuda())
            lay.reset()
            gl.append(lay)
        for s in range(warmup):
            for c in range(copies):
                gl[c].step(inp.q[s], inp.weights, pages[c], scales[c], pt)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for c in range(copies):
                gl[c].step(inp.q[warmup], inp.weights, pages[c], scales[c], pt)
        torch.cuda.synchronize()
        t0.record(stream)
        for s in range(steps):
            graph.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        for lay in gl:
            assert int(lay.err.item()) == 0, f"device error word {int(lay.err.item())}"
        out["graph_ms_per_step"] = t0.elapsed_time(t1) / (steps * copies)
        del graph, gl
    if stage_reps:
        q = inp.q[warmup + steps - 1]
        last_nv = nv[-1]

        def per_copy(make):
            fns = [make(c, lays[c], bts[c]) for c in range(copies)]
            return lambda: [f() for f in fns]

        # the score stages first, on the last step's own selection and query: the
        # candidate filter then compares against the hint that step's top-K left
        # (after the predict and select stages the selection is the next step's,
        # the hint no longer fits it and the candidate count is not a step's)
        st = {
            # the kernel spin_step runs (it also filters the top-K candidates)
            "score": per_copy(lambda c, lay, bt: lambda: api.spin_sparse_index_score(
                lay.cfg, bt, q, inp.weights, pages[c], scales[c], pt, lay.sel, lay.n_sel,
                lay.z, workspace=lay.workspace)),
            "score_no_filter": per_copy(lambda c, lay, bt: lambda: api.spin_sparse_index_score(
                lay.cfg, bt, q, inp.weights, pages[c], scales[c], pt, lay.sel, lay.n_sel,
                lay.z)),
            "topk": per_copy(lambda c, lay, bt: lambda: api.spin_topk(
                lay.cfg, bt, lay.z, lay.sel, lay.n_sel, lay.topk_idx, lay.workspace)),
            "ema": per_copy(lambda c, lay, bt: lambda: api.spin_ema_update(
                lay.cfg, bt, lay.z, lay.sel, lay.n_sel, lay.V, lay.D, n_valid=last_nv,
                v_max=lay.v_max)),
            "predict": per_copy(lambda c, lay, bt: lambda: api.spin_predict_blocks(
                lay.cfg, bt, lay.V, lay.D, lay.S, v_max=lay.v_max)),
            "select": per_copy(lambda c, lay, bt: lambda: api.spin_select_blocks(
                lay.cfg, bt, lay.S, lay.row_code, lay.sel, lay.n_sel)),
        }
        # the score launch's pages (the last step's selection), for the HBM
        # read probe timed beside the stages
        probe_ids = []
        for lay in lays:
            kk = torch.arange(w.max_blocks, device=lay.sel.device)
            mask = kk[None, :] < lay.n_sel.long()[:, None]
            probe_ids.append(pt.long().gather(1, lay.sel.long().clamp(min=0))[mask]
                             .to(torch.int32).contiguous())
        # every loop starts from the state the last step left (its selection,
        # the top-K hints and candidates in the workspace): the predict and
        # select stages of a loop leave the next step's selection behind
        snap = [(lay.sel.clone(), lay.n_sel.clone(),
                 None if lay.workspace is None else lay.workspace.clone()) for lay in lays]

        def stage_loop():
            for lay, (s_sel, s_n, s_ws) in zip(lays, snap):
                lay.sel.copy_(s_sel)
                lay.n_sel.copy_(s_n)
                if s_ws is not None:
                    lay.workspace.copy_(s_ws)
            return {k: _timed_us(f, stage_reps, stream, warm_log=warm[k]) / copies
                    for k, f in st.items()}

        warm = {k: [] for k in st}
        loops = [stage_loop() for _ in range(max(1, runs))]
        del snap
        # untimed calls (rounds over the copies) before each loop's timed ones
        out["stage_warm_rounds"] = warm
        if w.key_dtype == "fp8":
            # a plain read of the same pages with the score kernel's loads
            # (include/spin_probe.h): the practical ceiling of the score launch
            from sparse_attention_indexer_spin_amd import _lib as LIB
            sink = torch.zeros(LIB.SPIN_READ_PROBE_SINK_WORDS, dtype=torch.int32,
                               device=pages[0].device)
            probe = per_copy(lambda c, lay, bt: lambda: api.spin_read_pages(
                pages[c], probe_ids[c], sink))
            pr = [_timed_us(probe, stage_reps, stream) / copies for _ in range(max(1, runs))]
            out["page_read_us"] = float(np.median(pr))
            out["page_read_us_spread"] = [min(pr), max(pr)]
            out["page_read_bytes"] = 8192.0 * sum(int(x.numel()) for x in probe_ids) / copies
        out["stage_us"] = {k: float(np.median([lp[k] for lp in loops])) for k in st}
        out["stage_us_spread"] = {k: [min(lp[k] for lp in loops), max(lp[k] for lp in loops)]
                                  for k in st}
        for lay in lays:
            assert int(lay.err.item()) == 0, f"device error word {int(lay.err.item())}"
    return out


def _copies_of(inp: Inputs, copies: int):
    pages = [inp.keys.pages] + [inp.keys.pages.clone() for _ in range(copies - 1)]
    scales = [inp.keys.scale] + [None if inp.keys.scale is None else inp.keys.scale.clone()
                                 for _ in range(copies - 1)]
    return pages, scales


def sweep_point(inp: Inputs, sparsity_bp: int, steps: int, warmup: int, pages, scales,
                dense: bool):
    """One point of the sparsity sweep on len(pages) copies of the workload:
    per-layer step time of (a) spin_step on each copy round robin and (b) the
    copies as the layers of one spin_stack_step on one stream (each layer's
    plan inside the previous layer's launches), each from a reset, steps back
    to back.  With `dense` (0 % sparsity), also the dense indexer: score +
    top-K over every block (spin_step_finish without the EMA) round robin."""
    from sparse_attention_indexer_spin_amd import SpinLayer, SpinStack, api
    w = inp.w
    copies = len(pages)
    pt = inp.keys.page_table
    lays = []
    for c in range(copies):
        lay = SpinLayer(batch=w.batch, max_blocks=w.max_blocks,
                        d_cap=G.d_capacity(w, steps + warmup), topk=w.topk,
                        sparsity_bp=sparsity_bp, n_rows=1, explore_bp=w.explore_bp,
                        ema_alpha=w.alpha, combine=w.combine, layer=c,
                        key_dtype={"fp8": torch.uint8, "bf16": torch.bfloat16}[w.key_dtype],
                        q_dtype=torch.bfloat16 if w.q_dtype == "bf16" else torch.float32)
        lays.append(lay)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def reset():
        for lay in lays:
            lay.set_requests(inp.ctx.cuda(), inp.pos[0].cuda())
            lay.reset()

    def timed(step):
        reset()
        for s in range(warmup):
            step(s)
        torch.cuda.synchronize()
        e0.record(stream)
        for s in range(warmup, warmup + steps):
            step(s)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (steps * copies)

    def seq(s):
        for c, lay in enumerate(lays):
            lay.step(inp.q[s], inp.weights, pages[c], scales[c], pt)

    out = {"spin_step": timed(seq)}
    n_sel = int(sum(int(lay.n_sel.sum()) for lay in lays)) / copies
    stack = SpinStack(lays, one_stream=True)

    def stk(s):
        stack.step([inp.q[s]] * copies, [inp.weights] * copies, pages, scales, [pt] * copies)

    out["one_stream_stack"] = timed(stk)
    for lay in lays:
        assert int(lay.err.item()) == 0, f"device error word {int(lay.err.item())}"
    out["realized_sparsity"] = 1.0 - n_sel / float(sum(-(-int(c) // 64) for c in inp.ctx))
    if dense:
        bts = [lay.batch(pages[c].shape[0]) for c, lay in enumerate(lays)]
        ios = [lay.make_io(inp.q[warmup], inp.weights, pages[c], scales[c], pt)
               for c, lay in enumerate(lays)]
        for c, lay in enumerate(lays):
            api.spin_step_plan(lay.cfg, bts[c], ios[c])   # every block (0 % sparsity)

        def finish():
            for c, lay in enumerate(lays):
                api.spin_step_finish(lay.cfg, bts[c], ios[c], defer_ema=True)

        out["dense_indexer"] = _timed_us(finish, 10, stream) / copies
    del stack, lays
    return out


def fixed_cost(inp: Inputs, sparsities, steps: int, warmup: int, copies: int, runs: int):
    """The step time over the sparsity sweep, `runs` times: per run and mode,
    the least-squares fit T = a (1 - rho) + c and, with the slope pinned to the
    dense indexer time T_d (score + top-K over every block, same protocol),
    the overhead T(rho) - (1 - rho) T_d at each point and its mean.  Medians
    over the runs, with their spread."""
    pages, scales = _copies_of(inp, copies)
    per_run = []
    for _ in range(runs):
        pts = {sp: sweep_point(inp, sp, steps, warmup, pages, scales, dense=(sp == 0))
               for sp in sorted(set(sparsities) | {0})}
        td = pts[0]["dense_indexer"]
        rho = np.array([pts[sp]["realized_sparsity"] for sp in sorted(pts)])
        run = {"dense_indexer_us": td, "rho": rho.tolist()}
        for mode in ("spin_step", "one_stream_stack"):
            T = np.array([pts[sp][mode] for sp in sorted(pts)])
            A = np.stack([1.0 - rho, np.ones_like(rho)], 1)
            (a, c), *_ = np.linalg.lstsq(A, T, rcond=None)
            over = T - (1.0 - rho) * td
            run[mode] = {"T_us": T.tolist(), "a_us": float(a), "c_us": float(c),
                         "overhead_pinned_us": over.tolist(),
                         "c_pinned_us": float(over.mean())}
        per_run.append(run)
    med = lambda xs: float(np.median(xs))
    spread = lambda xs: [float(min(xs)), float(max(xs))]
    sp_list = sorted(set(sparsities) | {0})
    td = [r["dense_indexer_us"] for r in per_run]
    out = {"sparsity_bp": sp_list, "runs": runs,
           "realized_sparsity": per_run[0]["rho"],
           "dense_indexer_us": med(td), "dense_indexer_us_spread": spread(td)}
    for mode in ("spin_step", "one_stream_stack"):
        rs = [r[mode] for r in per_run]
        c, cp = [r["c_us"] for r in rs], [r["c_pinned_us"] for r in rs]
        out[mode] = {
            "us_per_step_layer": {str(sp): med([r["T_us"][i] for r in rs])
                                  for i, sp in enumerate(sp_list)},
            "fit_free": {"a_us": med([r["a_us"] for r in rs]), "c_us": med(c),
                         "c_us_spread": spread(c),
                         "c_over_dense_indexer": med(c) / med(td)},
            "fit_slope_pinned_to_dense": {
                "overhead_us": {str(sp): med([r["overhead_pinned_us"][i] for r in rs])
                                for i, sp in enumerate(sp_list)},
                "c_us": med(cp), "c_us_spread": spread(cp),
                "c_over_dense_indexer": med(cp) / med(td)}}
    return out


def miss_eval(inp: Inputs, sparsity_bp: int, steps: int, variants: dict):
    """Closed loop of one variant; after every sparse step, the dense top-K of
    the same queries (every block scored through the library) and the share
    of its slots that fall in blocks the step did not score.  Returns the
    per-(step, request, row) miss rates and the realized block sparsity."""
    from sparse_attention_indexer_spin_amd import SpinLayer, api
    w = inp.w
    kd = {"fp8": torch.uint8, "bf16": torch.bfloat16, "f32": torch.float32}[w.key_dtype]
    qd = torch.bfloat16 if w.q_dtype == "bf16" else torch.float32
    variants = dict(variants)
    explore_bp = variants.pop("explore_bp", w.explore_bp)
    lay = SpinLayer(batch=w.batch, max_blocks=w.max_blocks, d_cap=G.d_capacity(w, steps),
                    topk=w.topk, sparsity_bp=sparsity_bp, n_rows=w.rows,
                    explore_bp=explore_bp, ema_alpha=w.alpha, combine=w.combine,
                    key_dtype=kd, q_dtype=qd, **variants)
    lay.set_requests(inp.ctx.cuda(), inp.pos[0].cuda())
    lay.reset()
    pages, scale, pt = inp.keys.pages, inp.keys.scale, inp.keys.page_table
    bt = lay.batch(pages.shape[0])
    dev = pages.device
    B = (inp.ctx.to(dev).long() + 63) // 64
    ar = torch.arange(w.max_blocks, device=dev)
    sel_all = torch.where(ar[None, :] < B[:, None], ar[None, :], torch.full_like(ar, -1)[None, :])
    sel_all = sel_all.to(torch.int32).contiguous()
    n_all = B.to(torch.int32).contiguous()
    z_d = torch.zeros_like(lay.z)
    top_d = torch.full_like(lay.topk_idx, -1)
    ws_d = torch.zeros_like(lay.workspace)
    misses, sparsity = [], []
    for s in range(steps):
        nv = inp.accept_dev[s] if w.rows > 1 else None
        # the dense reference first: it reads the counters the step advances
        api.spin_sparse_index_score(lay.cfg, bt, inp.q[s], inp.weights, pages, scale, pt,
                                    sel_all, n_all, z_d)
        api.spin_topk(lay.cfg, bt, z_d, sel_all, n_all, top_d, ws_d)
        lay.step(inp.q[s], inp.weights, pages, scale, pt, n_valid=nv)
        if s == 0:
            continue                                   # the dense warm-up step
        mask = torch.zeros(w.batch, w.max_blocks + 1, dtype=torch.bool, device=dev)
        ns = lay.n_sel.long()
        for r in range(w.batch):
            mask[r, lay.sel[r, :int(ns[r])].long()] = True
        blk = torch.where(top_d >= 0, top_d // 64, torch.full_like(top_d, w.max_blocks)).long()
        valid = top_d >= 0
        hit = torch.gather(mask[:, None, :].expand(-1, w.rows, -1), 2, blk) & valid
        m = 1.0 - hit.sum(-1).float() / valid.sum(-1).clamp(min=1).float()
        misses.append(m.flatten().cpu())
        sparsity.append(float(1.0 - ns.sum().item() / B.sum().item()))
    torch.cuda.synchronize()
    assert int(lay.err.item()) == 0
    return torch.cat(misses).numpy(), float(np.mean(sparsity))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_keys_per_s(w: G.Workload, inp: Inputs, sparsity_bp: int, budget_s: float,
                       max_requests: int):
    """The CPU oracle on whole requests of the workload until about `budget_s`
    seconds of timed work: per request one dense warm-up step (untimed, t = 0
    is dense by definition), then two sparse steps (timed)."""
    from oracle import spin_oracle as O
    pt = inp.keys.page_table.cpu().numpy()
    pages_dev, scale_dev = inp.keys.pages, inp.keys.scale
    st_keys = 0
    elapsed = 0.0
    n_req = 0
    for r in range(min(w.batch, max_requests)):
        if elapsed >= budget_s:
            break
        phys = torch.from_numpy(pt[r]).long().cuda()
        if w.key_dtype == "bf16":
            pages = pages_dev[phys].cpu().view(torch.int16).numpy().astype(np.uint16)
        else:
            pages = pages_dev[phys].cpu().numpy()
        scale = scale_dev[phys].cpu().numpy() if scale_dev is not None else None
        local_pt = np.arange(w.max_blocks)
        state = O.RequestState(w.n_slots + 64, G.d_capacity(w, 8))
        N = int(inp.ctx[r])
        for s in range(3):
            q = inp.q[s, r].cpu()
            qn = q.view(torch.int16).numpy().astype(np.uint16) if q.dtype == torch.bfloat16 \
                else q.numpy()
            t = time.perf_counter()
            res = O.spin_step(state, q=qn, q_dtype=w.q_dtype, w=inp.weights[r].cpu().numpy(),
                              pages=pages, page_table_row=local_pt, key_dtype=w.key_dtype,
                              scale=scale, n_slots=N, q_pos=int(inp.pos[s, r]), K=w.topk,
                              sparsity_bp=sparsity_bp, explore_bp=w.explore_bp, alpha=w.alpha,
                              layer=0, req_id=r, seed=G.PHILOX_SEED, combine=w.combine)
            dt = time.perf_counter() - t
            if s > 0:
                elapsed += dt
                st_keys += len(res["slots"]) * w.rows
        n_req += 1
    return st_keys / elapsed, n_req, st_keys, elapsed


def cpu_baseline(w: G.Workload, inp: Inputs, sparsity_bp: int, budget_s: float,
                 max_requests: int):
    """The oracle as it stands, on the host's cores (its scores are fp64
    matrix products, threaded by the BLAS), and on one thread; budget_s seconds
    of timed work each."""
    from threadpoolctl import threadpool_info, threadpool_limits
    v, n_req, keys, el = _oracle_keys_per_s(w, inp, sparsity_bp, budget_s, max_requests)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    with threadpool_limits(limits=1):
        v1, n1, k1, e1 = _oracle_keys_per_s(w, inp, sparsity_bp, budget_s, max_requests)
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"value": v, "unit": "keys/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_req} of {w.batch} requests x 2 sparse steps after an untimed dense "
                      f"warm-up step ({keys} keys scored in {el:.1f} s; numpy fp64 oracle, "
                      f"BLAS on {threads} threads)",
            "single_thread": {"value": v1, "unit": "keys/s", "cores": 1,
                              "sample": f"{n1} requests x 2 sparse steps ({k1} keys in "
                                        f"{e1:.1f} s)"},
            "cpu_model": _cpu_model(), "nproc": os.cpu_count(), "usable_cpus": usable}


SCORE_SOURCES = ("sparse_attention_indexer_spin_amd/csrc/k_score.hip",
                 "sparse_attention_indexer_spin_amd/csrc/spin_dev.h",
                 "sparse_attention_indexer_spin_amd/csrc/plan_dev.h", "include/spin.h")


def score_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in SCORE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, sparsity_bp: int):
    """HBM bytes per score launch from the committed counter summary, or None when
    there is none for this workload or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"k_score_{workload}_rho{sparsity_bp}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != score_source_hash():
        return None
    return float(kv["traffic_bytes_per_launch"])


def copy_calibration():
    n = 256 * 1024 * 1024  # 1 GiB of fp32
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "copies": 3}))


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 "
                                   "(requests shard across GPUs with no exchange)"}))
        sys.exit(2)
    w = G.WORKLOADS[args.workload]
    sp = w.sparsity_bp[0] if args.sparsity_bp is None else args.sparsity_bp
    total_steps = args.steps + args.warmup
    if args.stack:
        main_stack(args, w, sp)
        return
    inp = Inputs(w, total_steps)
    if args.miss_eval:
        variants = [("A1-max (default)", {}), ("A1-top4", {"pooling": "top4"}),
                    ("A1-mean", {"pooling": "mean"}),
                    ("A0 (top-K predicted slots expanded)", {"reduction": "A0"}),
                    ("A2-max (block-level EMA)", {"reduction": "A2"}),
                    ("A2-top4", {"reduction": "A2", "pooling": "top4"}),
                    ("A2-mean", {"reduction": "A2", "pooling": "mean"}),
                    ("no exploration", {"explore_bp": 0}),
                    ("block-age exploration", {"explore": "age"}),
                    ("staleness-score exploration", {"explore": "staleness"})]
        if w.rows > 1:
            variants += [("row-0 mask", {"mtp_row0_mask": True}),
                         ("row-0 update", {"mtp_row0_update": True}),
                         ("row-0 mask + row-0 update", {"mtp_row0_mask": True,
                                                        "mtp_row0_update": True}),
                         ("per-row exploration", {"explore_per_row": True})]
        res = {}
        for spb in sorted(set(w.sparsity_bp) | {sp}):
            for name, v in variants:
                m, rs = miss_eval(inp, spb, total_steps, v)
                res.setdefault(str(spb), {})[name] = {
                    "mean_miss": float(m.mean()), "p99_miss": float(np.quantile(m, 0.99)),
                    "realized_sparsity": rs}
        print(json.dumps({"workload": w.name, "steps": total_steps, "miss_eval": res,
                          "data": "synthetic (seeded generator)"}))
        return
    evictor = Evictor()
    # the two other protocols first, for reference; then the reported one
    refs = {}
    if args.cache != "warm":
        refs["warm"] = run_gpu(inp, sp, args.steps, args.warmup)
    if args.cache != "cold":
        refs["cold"] = run_gpu(inp, sp, args.steps, args.warmup, evict=evictor)
    if args.cache == "rotate":
        res = run_rotate(inp, sp, args.steps, args.warmup, args.stage_reps, args.copies,
                         args.runs)
    else:
        res = run_gpu(inp, sp, args.steps, args.warmup, stage_reps=args.stage_reps,
                      evict=evictor if args.cache == "cold" else None)
    evict = evictor if args.cache == "cold" else None
    score_us = res["stage_us"]["score"]
    keys_row = res["keys_per_step"]
    score_bytes = algorithmic_score_bytes(w, keys_row // w.rows, res["n_sel"])
    achieved = score_bytes / (score_us * 1e-6) / 1e9
    value = keys_row / (res["ms_per_step"] * 1e-3)
    out = {
        "metric": "indexer keys scored/s + us/decode-step/layer at 512K ctx; % HBM peak",
        "value": value, "unit": "keys/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.key_dtype,
        "data": "synthetic (seeded generator: Gaussian keys + heavy slots + RoPE, AR(1) queries)",
        "config": {"workload": w.name, "requests": w.batch, "slots_per_request": w.n_slots,
                   "layers": 1, "verifier_rows": w.rows, "topk": w.topk,
                   "sparsity_bp": sp, "explore_bp": w.explore_bp, "key_dtype": w.key_dtype,
                   "q_dtype": w.q_dtype},
        "us_per_step_layer": res["ms_per_step"] * 1e3,
        "us_per_step_layer_runs": [t * 1e3 for t in res.get("ms_per_step_runs", [])] or None,
        "cache": {"mode": args.cache,
                  "how": {"rotate": f"{args.copies} independent copies of the workload (own "
                                    "pages and state) stepped round robin back to back",
                          "cold": "1 GiB read before each timed step and stage launch",
                          "warm": "one copy, steps back to back"}[args.cache],
                  **{f"{k}_us_per_step_layer": v["ms_per_step"] * 1e3 for k, v in refs.items()}},
        "stack_us_per_step_layer": (res["stack_ms_per_step"] * 1e3
                                    if "stack_ms_per_step" in res else None),
        "graph_us_per_step_layer": (res["graph_ms_per_step"] * 1e3
                                    if "graph_ms_per_step" in res else None),
        "stage_us": res["stage_us"],
        "stage_us_spread": res.get("stage_us_spread"),
        "stage_warm_rounds": res.get("stage_warm_rounds"),
        "page_read_probe": ({
            "how": "the score launch's pages read with its loads and nothing else "
                   "(spin_read_pages), timed like the stages",
            "us": res["page_read_us"], "us_spread": res["page_read_us_spread"],
            "key_bytes": res["page_read_bytes"],
            "gbs": res["page_read_bytes"] / (res["page_read_us"] * 1e-6) / 1e9,
            "frac_of_peak": res["page_read_bytes"] / (res["page_read_us"] * 1e-6) / 1e9
            / HBM_PEAK_GBS,
            "score_launch_over_read": res["stage_us"]["score"] / res["page_read_us"]}
            if "page_read_us" in res else None),
        "keys_scored_per_step": keys_row,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(w.name, sp),
                     "kernel": "spin::k_score_f32" if w.key_dtype == "f32" else "spin::k_score_wave",
                     "algorithmic_bytes_per_launch": score_bytes,
                     "launch_us": score_us},
    }
    if w.rows > 1 and w.key_dtype == "fp8":
        # several verifier rows: the contraction (2 n_h d flop per slot and row)
        # outgrows the bytes, so the score kernel is bound by the matrix cores;
        # it runs fp8 MFMA (dense peak 5.0 PFLOP/s), HBM figure alongside
        flops = keys_row * 2 * 64 * 128
        tflops = flops / (score_us * 1e-6) / 1e12
        hbm = out["roofline"]
        out["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": FP8_MFMA_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": tflops / FP8_MFMA_PEAK_TFLOPS,
                           "traffic": hbm["traffic"],
                           # 2-4 rows and at most 64 requests: the all-rows kernel
                           "kernel": ("spin::k_score_rows" if w.batch <= 64
                                      else hbm["kernel"]),
                           "algorithmic_flops_per_launch": flops,
                           "algorithmic_bytes_per_launch": score_bytes, "launch_us": score_us,
                           "hbm_achieved_gbs": achieved, "hbm_frac": achieved / HBM_PEAK_GBS}
    if not args.no_sweep and w.rows == 1 and len(w.sparsity_bp) > 1 and args.cache == "rotate":
        out["fixed_cost"] = fixed_cost(inp, w.sparsity_bp, min(args.steps, 20), args.warmup,
                                       args.copies, args.sweep_runs)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, inp, sp, args.cpu_seconds, args.cpu_max_requests)
    print(json.dumps(out))


def stack_sweep(inp: StackInputs, steps: int, warmup: int, evict=None):
    """Per-layer step time over the workload's sparsity sweep, one spin_step per
    layer on one stream and with the stack schedule, with the fit
    t = a (1 - rho) + c of each."""
    w = inp.w
    out = {"us_per_step_layer": {}, "realized_sparsity": {}}
    rho, t_seq, t_stk, t_one = [], [], [], []
    for sp in sorted(set(w.sparsity_bp)):
        res = run_stack(inp, sp, steps, warmup, evict, modes=("seq", "stack", "one_stream"))
        total_blocks = w.layers * int(sum(-(-int(c) // 64) for c in inp.ctx))
        r = 1.0 - res["n_sel"] / total_blocks
        rho.append(r)
        t_seq.append(res["ms_seq"] * 1e3 / w.layers)
        t_stk.append(res["ms_stack"] * 1e3 / w.layers)
        t_one.append(res["ms_one_stream"] * 1e3 / w.layers)
        out["us_per_step_layer"][str(sp)] = {"sequential": t_seq[-1], "stack": t_stk[-1],
                                             "one_stream": t_one[-1]}
        out["realized_sparsity"][str(sp)] = r
    A = np.stack([1.0 - np.array(rho), np.ones(len(rho))], 1)
    for name, T in (("sequential", t_seq), ("stack", t_stk), ("one_stream", t_one)):
        (a, c), *_ = np.linalg.lstsq(A, np.array(T), rcond=None)
        out[f"fit_{name}_us"] = {"a": float(a), "c": float(c)}
    return out


def main_stack(args, w: G.Workload, sp: int):
    """The multi-layer bench line: whole decode steps of every layer."""
    if w.layers < 2:
        w = dataclasses.replace(w, layers=args.stack_layers, name=f"{w.name}_x{args.stack_layers}")
    if w.key_dtype != "fp8" or w.rows != 1:
        print(json.dumps({"error": "--stack needs an fp8 workload with one row"}))
        sys.exit(2)
    inp = StackInputs(w, args.steps + args.warmup)
    evict = Evictor() if args.cache == "cold" else None
    if args.sweep and len(w.sparsity_bp) > 1:
        sw = stack_sweep(inp, min(args.steps, 20), args.warmup, evict)
        print(json.dumps({"workload": w.name, "cache": args.cache, "stack_sweep": sw}))
        return
    res = run_stack(inp, sp, args.steps, args.warmup, evict, args.budget_policy,
                    args.probe_period, drift_bp=args.budget_drift_bp)
    score_bytes = algorithmic_score_bytes(w, res["keys_layer0"], res["n_sel_layer0"])
    achieved = score_bytes / (res["score_us_layer0"] * 1e-6) / 1e9
    out = {
        "metric": "indexer keys scored/s + us/decode-step/layer at 512K ctx; % HBM peak",
        "value": res["keys_per_step"] / (res["ms_stack"] * 1e-3), "unit": "keys/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_stack"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.key_dtype,
        "data": "synthetic (seeded generator: Gaussian keys + heavy slots + RoPE, AR(1) queries;"
                " per-layer heavy fraction and direction norm)",
        "config": {"workload": w.name, "requests": w.batch, "slots_per_request":
                   [int(inp.ctx.min()), int(inp.ctx.max())], "layers": w.layers,
                   "verifier_rows": w.rows, "topk": w.topk, "sparsity_bp": sp,
                   "explore_bp": w.explore_bp, "key_dtype": w.key_dtype, "q_dtype": w.q_dtype},
        "us_per_step_layer": res["ms_stack"] * 1e3 / w.layers,
        "cache": {"mode": args.cache,
                  "how": "1 GiB read before each timed whole step" if evict is not None
                  else "steps back to back (the layers' own pages evict each other)"},
        "stack": {"sequential_us_per_step": res["ms_seq"] * 1e3,
                  "overlapped_us_per_step": res["ms_stack"] * 1e3,
                  "sequential_us_per_step_layer": res["ms_seq"] * 1e3 / w.layers,
                  "overlapped_us_per_step_layer": res["ms_stack"] * 1e3 / w.layers,
                  "overlapped_ema_stream_us_per_step_layer":
                      res["ms_stack_ema_stream"] * 1e3 / w.layers,
                  "one_stream_us_per_step_layer": res["ms_one_stream"] * 1e3 / w.layers,
                  "per_layer_budgets": res["budget"]},
        "keys_scored_per_step": res["keys_per_step"],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "spin::k_score_wave (mean launch, layers round robin)",
                     "algorithmic_bytes_per_launch": score_bytes,
                     "launch_us": res["score_us_layer0"]},
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
