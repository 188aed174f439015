"""Helpers for GPU tests: move a synthetic workload to the device and run the
HIP library through its C ABI.  No oracle arithmetic here."""
from __future__ import annotations

import numpy as np
import torch

import spin_synth as G
from tests.harness import LayerInputs, d_capacity

DEV = "cuda"

KEY_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
Q_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


def banner(msg: str):
    print(f"[gpu-test] {msg}", flush=True)


def device_keys(li: LayerInputs):
    pages = li.keys.pages.to(DEV)
    scale = li.keys.scale.to(DEV) if li.keys.scale is not None else None
    return pages, scale, li.keys.page_table.to(DEV)


def make_layer(li: LayerInputs, sparsity_bp: int, seed=G.PHILOX_SEED, combine=None,
               vmax_cache: bool = False, **variants):
    from sparse_attention_indexer_spin_amd import SpinLayer
    w = li.w
    lay = SpinLayer(batch=w.batch, max_blocks=w.max_blocks, d_cap=d_capacity(w, w.steps),
                    topk=w.topk, sparsity_bp=sparsity_bp, n_rows=w.rows,
                    explore_bp=w.explore_bp, ema_alpha=w.alpha, combine=combine or w.combine,
                    key_dtype=KEY_TORCH[w.key_dtype], q_dtype=Q_TORCH[w.q_dtype],
                    layer=li.layer, seed=seed, device=DEV, vmax_cache=vmax_cache, **variants)
    lay.set_requests(li.ctx.to(DEV), li.pos[0].to(DEV))
    lay.reset()
    return lay


def np_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy; bf16 as raw uint16 codes."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().astype(np.uint16)
    return t.numpy()


def z_close(z_gpu: np.ndarray, z_ref: np.ndarray, rtol: float) -> tuple[bool, float]:
    """|dz| <= rtol * max(|z|, 1e-3 * rms(z)) elementwise; returns (ok, worst ratio)."""
    z_ref = np.asarray(z_ref, dtype=np.float64)
    floor = 1e-3 * np.sqrt(np.mean(z_ref ** 2)) if z_ref.size else 0.0
    den = np.maximum(np.abs(z_ref), floor)
    den = np.where(den == 0, 1.0, den)
    ratio = np.abs(np.asarray(z_gpu, dtype=np.float64) - z_ref) / den
    worst = float(ratio.max()) if ratio.size else 0.0
    return worst <= rtol, worst
