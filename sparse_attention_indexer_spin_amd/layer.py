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
                 layer: int = 0, seed: int = 0x5350494E, device="cuda", vmax_cache: bool = False):
        self.R, self.rows, self.max_blocks, self.K = batch, n_rows, max_blocks, topk
        self.cfg = api.config(topk=topk, sparsity_bp=sparsity_bp, explore_bp=explore_bp,
                              ema_alpha=ema_alpha, combine=combine, key_dtype=key_dtype,
                              q_dtype=q_dtype, layer=layer, seed=seed)
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        n_cap = 64 * max_blocks
        self.V = torch.zeros(batch, n_cap, dtype=torch.float32, device=dev)
        self.D = torch.zeros(batch, d_cap, dtype=torch.float32, device=dev)
        # optional block maxima of V: predict then reads one float per block
        # instead of 64 (max combine), kept by reset, the EMA update and every
        # step.  Off by default: the predict kernel is latency-bound, so the
        # bytes it saves buy less than the upkeep costs the EMA update.
        self.v_max = torch.zeros(batch, max_blocks, dtype=torch.float32, device=dev) \
            if vmax_cache else None
        self.S = torch.zeros(batch, n_rows, max_blocks, dtype=torch.float32, device=dev)
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
        self._bt = None

    def reset(self, stream=None):
        api.spin_reset_state(self.V, self.D, self.step_ctr, stream=stream, v_max=self.v_max)

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
                           workspace=self.workspace, v_max=self.v_max)

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
    score / top-K / EMA of other layers on the main stream (spin_stack_step).

    `layers` are SpinLayer objects (own EMA state, counters and buffers each).
    step() takes per-layer queries, weights and key caches."""

    def __init__(self, layers, device="cuda"):
        self.layers = list(layers)
        self.stack = api.Stack(len(self.layers))
        # default priority (a side stream of another priority is not used)
        self.side = torch.cuda.Stream(device=device)
        self._order_next = True

    def inputs_changed(self):
        """Call after writing a layer's plan inputs on the main stream since
        the last step (set_requests, reset, budgets): the next step's plans
        then wait for the main stream first."""
        self._order_next = True

    def step(self, qs, ws, k_pages, k_scales, page_tables, n_valid=None, budgets=None,
             stream=None, n_layers=None):
        """One decode step of the first n_layers layers (default: all)."""
        n = len(self.layers) if n_layers is None else n_layers
        cfgs, bts, ios = [], [], []
        for l, lay in enumerate(self.layers[:n]):
            bts.append(lay.batch(k_pages[l].shape[0]))
            cfgs.append(lay.cfg)
            ios.append(lay.make_io(qs[l], ws[l], k_pages[l], k_scales[l], page_tables[l],
                                   None if n_valid is None else n_valid[l],
                                   None if budgets is None else budgets[l]))
        api.spin_stack_step(self.stack, cfgs, bts, ios, order_after_main=self._order_next,
                            main_stream=stream, side_stream=self.side)
        self._order_next = False
        return [lay.topk_idx for lay in self.layers]
