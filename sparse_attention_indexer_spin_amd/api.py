"""Python binding of the SPIN C ABI: same entry points, torch tensors in.

Argument marshalling only -- every stage runs in libspin.so's HIP kernels.
Tensors must be CUDA (HIP) tensors, contiguous, of the dtypes include/spin.h
states; torch supplies device memory and the current stream.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional

import torch

from . import _lib as L

_KEY = {torch.float32: L.SPIN_F32, torch.bfloat16: L.SPIN_BF16, torch.uint8: L.SPIN_FP8_E4M3,
        torch.float8_e4m3fn: L.SPIN_FP8_E4M3}
_Q = {torch.float32: L.SPIN_F32, torch.bfloat16: L.SPIN_BF16}


def _p(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("SPIN buffers must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("SPIN buffers must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


_POOL = {"max": L.SPIN_POOL_MAX, "top4": L.SPIN_POOL_TOP4, "mean": L.SPIN_POOL_MEAN}
_EXPLORE = {"random": 0, "age": L.SPIN_EXPLORE_AGE, "staleness": L.SPIN_EXPLORE_STALENESS}
_REDUCE = {"A1": 0, "A0": L.SPIN_REDUCE_A0, "A2": L.SPIN_REDUCE_A2}


def config(*, topk: int, sparsity_bp: int, explore_bp: int = 500, ema_alpha: float = 0.9,
           combine: str = "max", key_dtype: torch.dtype = torch.uint8,
           q_dtype: torch.dtype = torch.bfloat16, layer: int = 0, seed: int = 0x5350494E,
           n_heads: int = 64, head_dim: int = 128, block_size: int = 64, pooling: str = "max",
           mtp_row0_mask: bool = False, mtp_row0_update: bool = False,
           explore_per_row: bool = False, explore: str = "random",
           reduction: str = "A1", predict_ahead: bool = False) -> L.SpinConfig:
    """spin_config; the keyword variants map to spin_config.flags (defaults: the paper's).
    predict_ahead (SPIN_PREDICT_AHEAD) changes where the prediction runs, not its results."""
    flags = (_POOL[pooling] | (L.SPIN_MTP_ROW0_MASK if mtp_row0_mask else 0)
             | (L.SPIN_MTP_ROW0_UPDATE if mtp_row0_update else 0)
             | (L.SPIN_EXPLORE_PER_ROW if explore_per_row else 0)
             | _EXPLORE[explore] | _REDUCE[reduction]
             | (L.SPIN_PREDICT_AHEAD if predict_ahead else 0))
    return L.SpinConfig(n_heads=n_heads, head_dim=head_dim, block_size=block_size, topk=topk,
                        sparsity_bp=sparsity_bp, explore_bp=explore_bp, ema_alpha=ema_alpha,
                        combine=L.SPIN_COMBINE_SUM if combine == "sum" else L.SPIN_COMBINE_MAX,
                        key_dtype=_KEY[key_dtype], q_dtype=_Q[q_dtype], layer=layer, flags=flags,
                        seed=seed)


def batch(*, ctx_len, q_pos, step, req_id, n_rows: int, max_blocks: int, n_pages: int,
          err: Optional[torch.Tensor] = None) -> L.SpinBatch:
    for t in (ctx_len, q_pos, step, req_id):
        assert t.dtype == torch.int32
    return L.SpinBatch(batch=ctx_len.numel(), n_rows=n_rows, max_blocks=max_blocks,
                       n_pages=n_pages, ctx_len=_p(ctx_len), q_pos=_p(q_pos), step=_p(step),
                       req_id=_p(req_id), err=_p(err))


def _ld(t: torch.Tensor) -> int:
    return t.shape[-1]


def spin_predict_blocks(cfg, bt, V, D, S, stream=None, v_max=None):
    L.check(L.load().spin_predict_blocks(C.byref(cfg), C.byref(bt), _p(V), _ld(V), _p(D), _ld(D),
                                         _p(v_max),
                                         _p(S), _stream(stream)))


def spin_select_blocks(cfg, bt, S, row_code, sel, n_sel, budget=None, stream=None,
                       last_obs=None):
    L.check(L.load().spin_select_blocks(C.byref(cfg), C.byref(bt), _p(S), _p(budget),
                                        _p(last_obs), _p(row_code), _p(sel), _p(n_sel),
                                        _stream(stream)))


def spin_sparse_index_score(cfg, bt, q, w, k_pages, k_scale, page_table, sel, n_sel, z,
                            stream=None, workspace=None):
    """workspace (optional): the layer's workspace; the call then runs the kernel
    spin_step runs (with the top-K candidate filter)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    L.check(L.load().spin_sparse_index_score(
        C.byref(cfg), C.byref(bt), _p(q), _p(w), _p(k_pages), _p(k_scale), _p(page_table),
        _ld(page_table), _p(sel), _p(n_sel), _p(z), _ld(z), _p(workspace), ws_bytes,
        _stream(stream)))


def workspace_bytes(cfg, batch_size: int, n_rows: int, max_blocks: int) -> int:
    return int(L.load().spin_workspace_bytes(C.byref(cfg), batch_size, n_rows, max_blocks))


def spin_topk(cfg, bt, z, sel, n_sel, topk_idx, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    L.check(L.load().spin_topk(C.byref(cfg), C.byref(bt), _p(z), _ld(z), _p(sel), _p(n_sel),
                               _p(topk_idx), _p(workspace), ws_bytes, _stream(stream)))


def spin_ema_update(cfg, bt, z, sel, n_sel, V, D, n_valid=None, stream=None, v_max=None):
    L.check(L.load().spin_ema_update(C.byref(cfg), C.byref(bt), _p(z), _ld(z), _p(sel),
                                     _p(n_sel), _p(n_valid), _p(V), _ld(V), _p(D), _ld(D),
                                     _p(v_max), _stream(stream)))


def spin_advance(n_rows: int, q_pos, step, n_valid=None, stream=None):
    L.check(L.load().spin_advance(q_pos.numel(), n_rows, _p(n_valid), _p(q_pos), _p(step),
                                  _stream(stream)))


def spin_reset_state(V, D, step, stream=None, v_max=None):
    L.check(L.load().spin_reset_state(V.shape[0], _p(V), _ld(V), _p(D), _ld(D), _p(v_max),
                                      0 if v_max is None else _ld(v_max), _p(step),
                                      _stream(stream)))


def step_io(*, V, D, q, w, k_pages, k_scale, page_table, S, row_code, sel, n_sel, z, topk_idx,
            budget=None, n_valid=None, q_pos_mut=None, step_mut=None, workspace=None,
            v_max=None, last_obs=None, s_tag=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return L.SpinStepIO(V=_p(V), v_ld=_ld(V), D=_p(D), d_ld=_ld(D), v_max=_p(v_max), q=_p(q),
                        w=_p(w),
                        k_pages=_p(k_pages), k_scale=_p(k_scale), page_table=_p(page_table),
                        pt_ld=_ld(page_table), budget=_p(budget), n_valid=_p(n_valid), S=_p(S),
                        row_code=_p(row_code), sel=_p(sel), n_sel=_p(n_sel), z=_p(z),
                        z_ld=_ld(z), topk_idx=_p(topk_idx), q_pos_mut=_p(q_pos_mut),
                        step_mut=_p(step_mut), workspace=_p(workspace), workspace_bytes=ws_bytes,
                        last_obs=_p(last_obs), s_tag=_p(s_tag))


def spin_step(cfg, bt, io, defer_ema: bool = False, stream=None):
    L.check(L.load().spin_step(C.byref(cfg), C.byref(bt), C.byref(io), int(bool(defer_ema)),
                               _stream(stream)))


def spin_step_noalloc(cfg, bt, io, defer_ema: bool = False, stream=None):
    """spin_step on the library's static scratch (io's workspace is ignored)."""
    L.check(L.load().spin_step_noalloc(C.byref(cfg), C.byref(bt), C.byref(io),
                                       int(bool(defer_ema)), _stream(stream)))


def spin_step_plan(cfg, bt, io, stream=None):
    L.check(L.load().spin_step_plan(C.byref(cfg), C.byref(bt), C.byref(io), _stream(stream)))


def spin_step_finish(cfg, bt, io, defer_ema: bool = False, stream=None):
    L.check(L.load().spin_step_finish(C.byref(cfg), C.byref(bt), C.byref(io),
                                      int(bool(defer_ema)), _stream(stream)))


class Stack:
    """Handle of a spin_stack (host events of the multi-layer schedule)."""

    def __init__(self, n_layers: int):
        h = C.c_void_p()
        L.check(L.load().spin_stack_create(n_layers, C.byref(h)))
        self.handle, self.n_layers = h, n_layers

    def close(self):
        if self.handle:
            L.load().spin_stack_destroy(self.handle)
            self.handle = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _layer_arrays(cfgs, bts, ios):
    n = len(cfgs)
    assert len(bts) == n and len(ios) == n
    return n, (L.SpinConfig * n)(*cfgs), (L.SpinBatch * n)(*bts), (L.SpinStepIO * n)(*ios)


def spin_stack_step(stack: Stack, cfgs, bts, ios, order_after_main: bool = False,
                    main_stream=None, side_stream=None, ema_stream=None, defer_ema=False):
    """One decode step of len(cfgs) layers: plans on side_stream, finishes on
    main_stream (default: the current stream), EMA updates on ema_stream when
    given (else inside the finishes).  side_stream None: one stream, each
    layer's plan inside the previous layer's launches where possible.
    defer_ema: the EMA updates wait for spin_stack_commit."""
    n, ca, ba, ia = _layer_arrays(cfgs, bts, ios)
    L.check(L.load().spin_stack_step(stack.handle, n, ca, ba, ia, int(bool(order_after_main)),
                                     int(bool(defer_ema)), _stream(main_stream),
                                     None if side_stream is None else side_stream.cuda_stream,
                                     None if ema_stream is None else ema_stream.cuda_stream))


def spin_stack_commit(stack: Stack, cfgs, bts, ios, main_stream=None):
    """The deferred EMA updates (ios[l].n_valid rows) of the last stack step."""
    n, ca, ba, ia = _layer_arrays(cfgs, bts, ios)
    L.check(L.load().spin_stack_commit(stack.handle, n, ca, ba, ia, _stream(main_stream)))


def spin_miss_curve(cfg, bt, S, topk_idx, levels: int, covered, kprime, stream=None):
    L.check(L.load().spin_miss_curve(C.byref(cfg), C.byref(bt), _p(S), _p(topk_idx), levels,
                                     _p(covered), _p(kprime), _stream(stream)))


def spin_budget_fill(cfg, bt, level_table, levels: int, budget, stream=None):
    L.check(L.load().spin_budget_fill(C.byref(cfg), C.byref(bt), _p(level_table), levels,
                                      _p(budget), _stream(stream)))


def spin_budget_allocate(policy: str, levels: int, target_level: int, covered=None, total=None,
                         running_miss=None):
    """Host-only allocation of per-layer levels (numpy in, list of ints out)."""
    import numpy as np
    if policy == "minimax":
        cov = np.ascontiguousarray(covered, dtype=np.int64)
        tot = np.ascontiguousarray(total, dtype=np.int64)
        n = tot.shape[0]
        assert cov.shape == (n, levels + 1)
        args = (L.SPIN_BUDGET_MINIMAX, cov.ctypes.data, tot.ctypes.data, None)
    elif policy == "proportional":
        miss = np.ascontiguousarray(running_miss, dtype=np.float64)
        n = miss.shape[0]
        args = (L.SPIN_BUDGET_PROPORTIONAL, None, None, miss.ctypes.data)
    else:
        raise ValueError(f"unknown budget policy {policy!r}")
    out = np.zeros(n, dtype=np.int32)
    L.check(L.load().spin_budget_allocate(args[0], n, levels, target_level, args[1], args[2],
                                          args[3], out.ctypes.data))
    return out.tolist()


def spin_budget_state_bytes(n_layers: int, levels: int) -> int:
    return int(L.load().spin_budget_state_bytes(n_layers, levels))


def spin_stack_set_budget_policy(stack: Stack, policy: Optional[str], probe_period: int = 8,
                                 levels: int = 100, target_level: int = 0, level_table=None,
                                 budget=None, probe_budget=None, covered=None, kprime=None,
                                 state=None, drift_bp: int = 0):
    """The stack runs per-layer budgets itself (policy "minimax" or
    "proportional"; None clears it; drift_bp > 0 publishes new levels only
    past that drift of the miss curves).  Buffers: see include/spin.h."""
    if policy is None:
        L.check(L.load().spin_stack_set_budget_policy(stack.handle, None))
        return
    code = {"minimax": L.SPIN_BUDGET_MINIMAX, "proportional": L.SPIN_BUDGET_PROPORTIONAL}[policy]
    p = L.SpinBudgetPolicy(policy=code, probe_period=probe_period, levels=levels,
                           target_level=target_level, drift_bp=drift_bp,
                           level_table=_p(level_table),
                           budget=_p(budget), probe_budget=_p(probe_budget), covered=_p(covered),
                           kprime=_p(kprime), state=_p(state))
    L.check(L.load().spin_stack_set_budget_policy(stack.handle, C.byref(p)))


def spin_stack_reset_budgets(stack: Stack, cfgs, bts, main_stream=None):
    n = len(cfgs)
    ca, ba = (L.SpinConfig * n)(*cfgs), (L.SpinBatch * n)(*bts)
    L.check(L.load().spin_stack_reset_budgets(stack.handle, n, ca, ba, _stream(main_stream)))


def spin_budget_update(policy: str, levels: int, target_level: int, covered, kprime, state,
                       level_table, stream=None, drift_bp: int = 0):
    """One probe's allocation on the device.  covered: i32 [L, rows_total,
    levels + 1], kprime: i32 [L, rows_total] (device tensors); with
    drift_bp > 0 level_table changes only past that drift of the curves."""
    code = {"minimax": L.SPIN_BUDGET_MINIMAX, "proportional": L.SPIN_BUDGET_PROPORTIONAL}[policy]
    n_layers = level_table.numel()
    rows_total = kprime.numel() // n_layers
    L.check(L.load().spin_budget_update(code, n_layers, levels, target_level, drift_bp, rows_total,
                                        _p(covered), _p(kprime), _p(state), _p(level_table),
                                        _stream(stream)))


def spin_read_pages(k_pages, page_ids, sink, stream=None):
    """The HBM read probe of include/spin_probe.h (measurement only): reads
    the listed 8 KB pages of k_pages with the fp8 score kernel's loads.
    page_ids: i32 device tensor; sink: u32/i32 device tensor of
    SPIN_READ_PROBE_SINK_WORDS words."""
    assert sink.numel() >= L.SPIN_READ_PROBE_SINK_WORDS and k_pages.element_size() == 1
    n_pages = k_pages.numel() // 8192
    L.check(L.load().spin_read_pages(_p(k_pages), n_pages, _p(page_ids), page_ids.numel(),
                                     _p(sink), _stream(stream)))
