"""Test-side helpers: build a synthetic workload once (CPU tensors from
spin_synth) and drive the CPU oracle over it.  GPU tests hand the very same
input bytes to the HIP library."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import spin_synth as G
from oracle import spin_oracle as O


@dataclass
class LayerInputs:
    w: G.Workload
    layer: int
    ctx: torch.Tensor          # [R] int32
    keys: G.KeyCache
    weights: torch.Tensor      # [R, rows, 64] f32
    pos: torch.Tensor          # [S, R] int64
    accept: torch.Tensor       # [S, R] int32
    q: torch.Tensor            # [S, R, rows, 64, 128] (f32 or bf16)

    # numpy views for the oracle ------------------------------------------
    def np_pages(self):
        p = self.keys.pages
        if p.dtype == torch.bfloat16:
            return p.view(torch.int16).numpy().astype(np.uint16)
        return p.numpy()

    def np_q(self, s):
        q = self.q[s]
        if q.dtype == torch.bfloat16:
            return q.view(torch.int16).numpy().astype(np.uint16)
        return q.numpy()


def build_layer(w: G.Workload, layer: int = 0, integer: bool = False, n_steps=None):
    ctx = G.context_lengths(w)
    keys = G.make_keys(w, layer, "cpu", ctx, integer=integer)
    weights = G.make_weights(w, layer, "cpu", integer=integer)
    pos, acc = G.make_schedule(w, ctx, n_steps)
    q = G.cast_queries(w, G.make_queries(w, layer, keys, pos, "cpu", integer=integer))
    return LayerInputs(w, layer, ctx, keys, weights, pos, acc, q)


d_capacity = G.d_capacity


def run_oracle(li: LayerInputs, n_steps: int, sparsity_bp: int, reqs=None, seed=G.PHILOX_SEED,
               combine=None, states=None, keep_state_history=False, **variants):
    """Closed-loop oracle over n_steps; returns per-step lists of per-request results.
    keep_state_history: each result also holds "state_after", copies of the
    request's (V, D) after the step."""
    w = li.w
    reqs = range(w.batch) if reqs is None else reqs
    pages = li.np_pages()
    scale = None if li.keys.scale is None else li.keys.scale.numpy()
    pt = li.keys.page_table.numpy()
    d_cap = d_capacity(w, w.steps)
    if states is None:
        states = {r: O.RequestState(w.n_slots + 64, d_cap) for r in reqs}
    out = []
    for s in range(n_steps):
        step_res = {}
        q_all = li.np_q(s)
        for r in reqs:
            res = O.spin_step(states[r], q=q_all[r], q_dtype=w.q_dtype,
                              w=li.weights[r].numpy(), pages=pages, page_table_row=pt[r],
                              key_dtype=w.key_dtype, scale=scale, n_slots=int(li.ctx[r]),
                              q_pos=int(li.pos[s, r]), K=w.topk, sparsity_bp=sparsity_bp,
                              explore_bp=w.explore_bp, alpha=w.alpha, layer=li.layer,
                              req_id=r, seed=seed, combine=combine or w.combine,
                              n_valid=int(li.accept[s, r]), **variants)
            if keep_state_history:
                res["state_after"] = (states[r].V.copy(), states[r].D.copy())
            step_res[r] = res
        out.append(step_res)
    return out, states
