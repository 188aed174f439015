"""SpinLayer: the per-layer SPIN state and step buffers in GPU memory.

Owns V, D (the vertical and diagonal EMA states), the per-request counters
and the step's output buffers, allocated once with torch; every step call is
one pass through libspin.so's C ABI.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import api


class SpinLayer:
    def __init__(self, *, batch: int, max_blocks: int, d_cap: int, topk: int, sparsity_bp: int,
                 n_rows: int = 1, explore_bp: int = 500, ema_alpha: float = 0.9,
                 combine: str = "max", key_dtype=torch.uint8, q_dtype=torch.bfloat16,
                 layer: int = 0, seed: int = 0x5350494E, device="cuda",
                 vmax_cache: Optional[bool] = None,
                 predict_ahead: bool = False, **variants):
        """`variants`: the design variants of api.config (pooling, mtp_row0_mask,
        mtp_row0_update, explore_per_row, explore, reduction); the paper's
        defaults without them.  predict_ahead: each step's EMA update also
        predicts the next step's block scores (SPIN_PREDICT_AHEAD; one
        verifier row, block reduction A1), the same scores the next step's own
        prediction would compute.  Off by default: the update then walks every
        block instead of the selected ones, and inside the top-K launch that
        costs about what the skipped prediction saves."""
        self.R, self.rows, self.max_blocks, self.K = batch, n_rows, max_blocks, topk
        self.cfg = api.config(topk=topk, sparsity_bp=sparsity_bp, explore_bp=explore_bp,
                              ema_alpha=ema_alpha, combine=combine, key_dtype=key_dtype,
                              q_dtype=q_dtype, layer=layer, seed=seed,
                              predict_ahead=predict_ahead, **variants)
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        n_cap = 64 * max_blocks
        self.V = torch.zeros(batch, n_cap, dtype=torch.float32, device=dev)
        self.D = torch.zeros(batch, d_cap, dtype=torch.float32, device=dev)
        # optional block maxima of V: predict then reads one float per block
        # instead of 64, kept by reset, the EMA update and every step.  By
        # default on where it applies (max combine, max pooling, block
        # reduction A1): with the state in HBM, halving the prediction's bytes
        # saves more than the upkeep costs the EMA update.
        if vmax_cache is None:
            vmax_cache = (combine == "max" and variants.get("pooling", "max") == "max"
                          and variants.get("reduction", "A1") == "A1")
        self.v_max = torch.zeros(batch, max_blocks, dtype=torch.float32, device=dev) \
            if vmax_cache else None
        self.S = torch.zeros(batch, n_rows, max_blocks, dtype=torch.float32, device=dev)
        # the step at which each block was last scored (exploration by block
        # age / staleness), kept by every step's selection
        self.last_obs = torch.zeros(batch, max_blocks, **i32)
        # per request: the (step, q position, context) S was predicted ahead
        # for by the last EMA update, -1 when none
        self.s_tag = torch.full((batch, 4), -1, **i32) if predict_ahead else None
        self.row_code = torch.zeros(batch, n_rows, max_blocks, dtype=torch.uint8, device=dev)
        self.sel = torch.full((batch, max_blocks), -1, **i32)
        self.n_sel = torch.zeros(batch, **i32)
        self.z = torch.zeros(batch, n_rows, n_cap, dtype=torch.float32, device=dev)
        self.topk_idx = torch.full((batch, n_rows, topk), -1, **i32)
        self.ctx_len = torch.ones(batch, **i32)
        self.q_pos = torch.ones(batch, **i32)
        self.step_ctr = torch.zeros(batch, **i32)
        self.req_id = torch.arange(batch, **i32)
        self.err = torch.zeros(1, **i32)
        nws = api.workspace_bytes(self.cfg, batch, n_rows, max_blocks)
        self.workspace = torch.zeros(max(nws, 1), dtype=torch.uint8, device=dev) if nws else None
        self.n_pages = 1
        self._bt = None

    # -- request bookkeeping -------------------------------------------------
    def set_requests(self, ctx_len: torch.Tensor, q_pos: torch.Tensor,
                     req_id: Optional[torch.Tensor] = None):
        self.ctx_len.copy_(ctx_len.to(torch.int32))
        self.q_pos.copy_(q_pos.to(torch.int32))
        if req_id is not None:
            self.req_id.copy_(req_id.to(torch.int32))
        if self.s_tag is not None:
            self.s_tag.fill_(-1)
        self._bt = None

    def reset(self, stream=None):
        api.spin_reset_state(self.V, self.D, self.step_ctr, stream=stream, v_max=self.v_max)
        st = torch.cuda.current_stream() if stream is None else stream
        with torch.cuda.stream(st):
            self.last_obs.zero_()
            if self.s_tag is not None:
                self.s_tag.fill_(-1)

    def batch(self, n_pages: int):
        if self._bt is None or self.n_pages != n_pages:
            self.n_pages = n_pages
            self._bt = api.batch(ctx_len=self.ctx_len, q_pos=self.q_pos, step=self.step_ctr,
                                 req_id=self.req_id, n_rows=self.rows,
                                 max_blocks=self.max_blocks, n_pages=n_pages, err=self.err)
        return self._bt

    # -- one decode step ---------------------------------------------------
    def make_io(self, q, w, k_pages, k_scale, page_table, n_valid=None, budget=None):
        return api.step_io(V=self.V, D=self.D, q=q, w=w, k_pages=k_pages, k_scale=k_scale,
                           page_table=page_table, S=self.S, row_code=self.row_code, sel=self.sel,
                           n_sel=self.n_sel, z=self.z, topk_idx=self.topk_idx, budget=budget,
                           n_valid=n_valid, q_pos_mut=self.q_pos, step_mut=self.step_ctr,
                           workspace=self.workspace, v_max=self.v_max, last_obs=self.last_obs,
                           s_tag=self.s_tag)

    def step(self, q, w, k_pages, k_scale, page_table, n_valid=None, budget=None,
             defer_ema: bool = False, stream=None):
        bt = self.batch(k_pages.shape[0])
        io = self.make_io(q, w, k_pages, k_scale, page_table, n_valid, budget)
        api.spin_step(self.cfg, bt, io, defer_ema=defer_ema, stream=stream)
        return self.topk_idx

    def commit(self, n_valid: Optional[torch.Tensor] = None, stream=None):
        """Deferred EMA replay of the first n_valid rows, then advance the counters."""
        bt = self.batch(self.n_pages)
        api.spin_ema_update(self.cfg, bt, self.z, self.sel, self.n_sel, self.V, self.D,
                            n_valid=n_valid, stream=stream, v_max=self.v_max)
        api.spin_advance(self.rows, self.q_pos, self.step_ctr, n_valid=n_valid, stream=stream)


class SpinStack:
    """The SPIN state of several layers and the multi-layer schedule: every
    layer's plan (predict + select) runs on a side stream, overlapped with the
    score / top-K / EMA of other layers on the main stream (spin_stack_step),
    or with one_stream inside the previous layer's launches.

    `layers` are SpinLayer objects (own EMA state, counters and buffers each).
    step() takes per-layer queries, weights and key caches.

    Per-layer block budgets (optional, `budget_policy` "minimax" or
    "proportional"): the stack runs them in the library
    (spin_stack_set_budget_policy): every `probe_period` steps after a reset a
    dense probe step measures the layers' miss curves, and a device kernel
    re-sizes the levels (their sum stays n_layers x the target level of the
    layers' sparsity) into the device-side level table and the layers'
    budgets, used from the next step on; with `budget_drift_bp` > 0 only
    when some layer's miss curve moved by more than that many basis points
    since the last re-sizing.  This object only owns the buffers.  Until the
    first probe every layer runs at the target level."""

    def __init__(self, layers, device="cuda", budget_policy=None, probe_period: int = 8,
                 levels: int = 100, ema_stream: bool = False, one_stream: bool = False,
                 budget_drift_bp: int = 0):
        self.layers = list(layers)
        # one_stream: every layer's plan inside the previous layer's score and
        # top-K + EMA launches on the main stream (no side stream, no events)
        assert not (one_stream and ema_stream)
        self.one_stream = one_stream
        self.stack = api.Stack(len(self.layers))
        # default priority (streams of another priority are not used)
        self.side = torch.cuda.Stream(device=device)
        # optionally the EMA updates on a third stream, off the main stream
        # (see join()).  Off by default: the update is bandwidth-bound like
        # the score kernel beside it, so running them together slows both;
        # fused with the latency-bound top-K on the main stream it is free.
        self.ema = torch.cuda.Stream(device=device) if ema_stream else None
        self._order_next = True
        self._deferred = None
        self.policy = budget_policy
        if budget_policy is not None:
            assert budget_policy in ("minimax", "proportional")
            L, R = len(self.layers), self.layers[0].R
            rows = self.layers[0].rows
            sp = {lay.cfg.sparsity_bp for lay in self.layers}
            assert len(sp) == 1 and 10000 % levels == 0 and (10000 - sp.pop()) % (10000 // levels) == 0
            self.levels, self.P = levels, probe_period
            self.target = (10000 - self.layers[0].cfg.sparsity_bp) // (10000 // levels)
            dev = torch.device(device)
            i32 = dict(dtype=torch.int32, device=dev)
            self.level_table = torch.full((L,), self.target, **i32)
            self.budget = torch.zeros(L, R, **i32)
            self.probe_budget = torch.zeros(R, **i32)
            self.covered = torch.zeros(L, R, rows, levels + 1, **i32)
            self.kprime = torch.zeros(L, R, rows, **i32)
            self.state = torch.zeros(api.spin_budget_state_bytes(L, levels), dtype=torch.uint8,
                                     device=dev)
            api.spin_stack_set_budget_policy(
                self.stack, budget_policy, probe_period=probe_period, levels=levels,
                target_level=self.target, level_table=self.level_table, budget=self.budget,
                probe_budget=self.probe_budget, covered=self.covered, kprime=self.kprime,
                state=self.state, drift_bp=budget_drift_bp)
            self.reset_budgets()

    # -- budgets -------------------------------------------------------------
    def reset_budgets(self, stream=None):
        """Uniform target levels, no probe history (on the current stream):
        call with a reset of the layers, and after set_requests (the budgets
        follow the contexts)."""
        bts = [lay.batch(lay.n_pages) for lay in self.layers]
        api.spin_stack_reset_budgets(self.stack, [lay.cfg for lay in self.layers], bts,
                                     main_stream=stream)

    def levels_now(self):
        """The layers' current budget levels (reads the device table: a host
        synchronisation, for inspection only)."""
        return self.level_table.cpu().tolist()

    def commit(self, n_valid=None, stream=None):
        """The deferred EMA updates of the last step: layer l replays its rows
        0 .. n_valid[l] - 1 (every row when None) and advances its counters."""
        cfgs, bts, ios = self._deferred
        for l, io in enumerate(ios):
            io.n_valid = None if n_valid is None else api._p(n_valid[l])
        api.spin_stack_commit(self.stack, cfgs, bts, ios, main_stream=stream)
        self._deferred = None

    def join(self, stream=None):
        """Order `stream` (default: the current one) after everything the stack
        issued; needed before reading or writing a layer's EMA state or
        counters there when the EMA runs on its own stream."""
        st = torch.cuda.current_stream() if stream is None else stream
        st.wait_stream(self.side)
        if self.ema is not None:
            st.wait_stream(self.ema)

    def reset(self):
        """Reset every layer (EMA state to zero, next step dense), on the
        current stream after the stack's pending work."""
        self.join()
        for lay in self.layers:
            lay.reset()
        if self.policy is not None:
            self.reset_budgets()
        self.inputs_changed()

    def inputs_changed(self):
        """Call after writing a layer's plan inputs on the main stream since
        the last step (set_requests, reset, budgets): the next step's plans
        then wait for the main stream first."""
        self._order_next = True

    def step(self, qs, ws, k_pages, k_scales, page_tables, n_valid=None, budgets=None,
             stream=None, n_layers=None, defer_ema: bool = False):
        """One decode step of the first n_layers layers (default: all).
        defer_ema: the EMA updates wait for commit() (speculative decoding).
        With a budget policy the stack chooses the budgets (`budgets` unused)."""
        n = len(self.layers) if n_layers is None else n_layers
        cfgs, bts, ios = [], [], []
        for l, lay in enumerate(self.layers[:n]):
            bts.append(lay.batch(k_pages[l].shape[0]))
            cfgs.append(lay.cfg)
            ios.append(lay.make_io(qs[l], ws[l], k_pages[l], k_scales[l], page_tables[l],
                                   None if n_valid is None else n_valid[l],
                                   None if budgets is None else budgets[l]))
        api.spin_stack_step(self.stack, cfgs, bts, ios, order_after_main=self._order_next,
                            main_stream=stream,
                            side_stream=None if self.one_stream else self.side,
                            ema_stream=self.ema, defer_ema=defer_ema)
        self._order_next = False
        if defer_ema:
            self._deferred = (cfgs, bts, ios)
        return [lay.topk_idx for lay in self.layers[:n]]
