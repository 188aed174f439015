"""Seeded synthetic inputs for the SPIN decode step.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It produces *inputs only* -- key caches, queries, head weights, page
tables, positions, acceptance lengths and synthetic EMA/score states.  None of
SPIN's own arithmetic (block prediction, selection, indexer scoring, top-K, EMA
update) lives here.

Workload recipe (SPIN paper, Sec. 2 indexer definition; Sec. 3.2 slot
coordinates; Sec. 4.1 block size):
  * one indexer key per compressed KV slot, k_i ~ N(0, I_128); a seeded 2 % of
    the slots are "heavy" and carry an added persistent direction u (||u|| = 3);
  * RoPE (base 10000, interleaved pairs) rotates dims 0..63 of every key at its
    slot position and of every query head at its query position -- this is
    what produces diagonal bands;
  * queries follow a per-head AR(1) drift q_t = 0.95 q_{t-1} + 0.31 N(0, I)
    + 0.5 u, started from its stationary law, RoPE applied to the emitted q;
  * head weights w_h ~ U(0.5, 1.5);
  * keys live in 64-slot pages of one global pool, reached through a shuffled
    page table (the paged-attention layout the method targets);
  * fp8 keys are OCP E4M3 codes with a per-slot fp32 scale amax/448.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import torch

BLOCK = 64          # slots per KV block == slots per page
N_HEADS = 64
HEAD_DIM = 128
ROPE_DIMS = 64      # RoPE on half of each head's dims
E4M3_MAX = 448.0
SEED_BASE = 20261202
PHILOX_SEED = 0x5350494E

KEY_DTYPES = ("f32", "bf16", "fp8")
Q_DTYPES = ("f32", "bf16")


@dataclass(frozen=True)
class Workload:
    """Shape of one synthetic SPIN workload (sizes in compressed KV slots)."""
    name: str
    batch: int
    layers: int
    rows: int                 # verifier queries per step (1 = no MTP)
    n_slots: int              # context length per request (max when ragged)
    n_slots_min: int          # == n_slots unless ragged
    topk: int
    sparsity_bp: Sequence[int]  # target block sparsity sweep, basis points
    key_dtype: str
    q_dtype: str
    steps: int
    explore_bp: int = 500
    alpha: float = 0.9
    combine: str = "max"      # "max" (Eq. 1) or "sum"
    heavy_frac: Sequence[float] = (0.02, 0.02)   # per-layer range
    heavy_norm: Sequence[float] = (3.0, 3.0)     # per-layer range
    accept_probs: Optional[Sequence[float]] = None  # P[L = 1..rows]
    shuffled_pages: bool = True
    cfg_id: int = 0

    @property
    def max_blocks(self) -> int:
        return -(-self.n_slots // BLOCK)

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # tiny, checkable on the CPU in full
    "tiny_f32_4k": Workload(
        name="tiny_f32_4k", batch=1, layers=1, rows=1, n_slots=4096,
        n_slots_min=4096, topk=512, sparsity_bp=(4000,), key_dtype="f32",
        q_dtype="f32", steps=32, combine="sum", shuffled_pages=False, cfg_id=0),
    # one layer, 16 requests of 64K slots, bf16
    "bf16_64k_b16": Workload(
        name="bf16_64k_b16", batch=16, layers=1, rows=1, n_slots=65536,
        n_slots_min=65536, topk=2048, sparsity_bp=(4000,), key_dtype="bf16",
        q_dtype="bf16", steps=256, cfg_id=1),
    # 512K tokens at 4x compression, 32 requests, fp8 keys, sparsity sweep
    "fp8_128k_b32": Workload(
        name="fp8_128k_b32", batch=32, layers=1, rows=1, n_slots=131072,
        n_slots_min=131072, topk=2048, sparsity_bp=(4000, 0, 2000, 3000, 5000),
        key_dtype="fp8", q_dtype="bf16", steps=128, cfg_id=2),
    # speculative decoding: 4 verifier rows per step
    "fp8_128k_b32_mtp4": Workload(
        name="fp8_128k_b32_mtp4", batch=32, layers=1, rows=4, n_slots=131072,
        n_slots_min=131072, topk=2048, sparsity_bp=(4000,), key_dtype="fp8",
        q_dtype="bf16", steps=128, accept_probs=(0.25, 0.30, 0.25, 0.20),
        cfg_id=3),
    # 1M tokens, 8 layers, 24 ragged requests
    "fp8_256k_ragged_8l": Workload(
        name="fp8_256k_ragged_8l", batch=24, layers=8, rows=1, n_slots=262144,
        n_slots_min=65536, topk=2048, sparsity_bp=(4000,), key_dtype="fp8",
        q_dtype="bf16", steps=64, heavy_frac=(0.01, 0.04),
        heavy_norm=(2.0, 4.0), cfg_id=4),
}


# --------------------------------------------------------------------------
# small helpers
# --------------------------------------------------------------------------
def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def sub_seed(w: Workload, layer: int, req: int, salt: int = 0) -> int:
    return SEED_BASE + w.cfg_id + 1_000_003 * (layer + 1) + 7919 * (req + 1) + 104_729 * salt


def rope(x: torch.Tensor, pos: torch.Tensor) -> torch.Tensor:
    """Rotate dims 0..63 of the last axis (interleaved pairs) at positions pos.

    x: [..., P, 128] float32, pos: [P] int64 (broadcast over leading dims).
    """
    j = torch.arange(ROPE_DIMS // 2, device=x.device, dtype=torch.float64)
    theta = torch.pow(torch.tensor(10000.0, dtype=torch.float64, device=x.device),
                      -2.0 * j / ROPE_DIMS)
    ang = pos.to(torch.float64)[:, None] * theta[None, :]          # [P, 32]
    c, s = torch.cos(ang).to(torch.float32), torch.sin(ang).to(torch.float32)
    out = x.clone()
    xe, xo = x[..., 0:ROPE_DIMS:2], x[..., 1:ROPE_DIMS:2]
    out[..., 0:ROPE_DIMS:2] = xe * c - xo * s
    out[..., 1:ROPE_DIMS:2] = xe * s + xo * c
    return out


def encode_fp8(k: torch.Tensor):
    """Per-slot scaled OCP E4M3 codes: returns (uint8 codes [..., 128], f32 scale [...])."""
    amax = k.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).to(torch.float32)
    y = (k / scale[..., None]).clamp(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def encode_bf16(x: torch.Tensor) -> torch.Tensor:
    """bfloat16 (round to nearest even) as raw uint16 codes."""
    return x.to(torch.bfloat16).view(torch.int16).view(torch.uint16) if hasattr(torch, "uint16") \
        else x.to(torch.bfloat16).view(torch.int16)


def bf16_tensor(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


# --------------------------------------------------------------------------
# key caches
# --------------------------------------------------------------------------
@dataclass
class KeyCache:
    """Paged key cache of one layer for all requests of a workload."""
    pages: torch.Tensor        # [n_pages, 64, 128] float32 | bfloat16 | uint8
    scale: Optional[torch.Tensor]  # [n_pages, 64] float32 (fp8 only)
    page_table: torch.Tensor   # [R, max_blocks] int32
    u: torch.Tensor            # [R, 128] float32 heavy direction per request
    heavy: list = field(default_factory=list)  # per request: int64 heavy slot ids


def _layer_params(w: Workload, layer: int):
    if w.layers <= 1:
        return float(w.heavy_frac[0]), float(w.heavy_norm[0])
    g = _gen(SEED_BASE + w.cfg_id + 31 * (layer + 1), "cpu")
    a = torch.rand(2, generator=g, dtype=torch.float64)
    hf = w.heavy_frac[0] + (w.heavy_frac[1] - w.heavy_frac[0]) * float(a[0])
    hn = w.heavy_norm[0] + (w.heavy_norm[1] - w.heavy_norm[0]) * float(a[1])
    return hf, hn


def d_capacity(w: Workload, n_steps: int) -> int:
    """Length of the diagonal-state axis: offsets reach q_pos + rows - 1 < N + rows * (steps + 1)."""
    return w.n_slots + w.rows * (n_steps + 1) + 64


def context_lengths(w: Workload) -> torch.Tensor:
    """Per-request context length (slots); uniform in [n_slots_min, n_slots] when ragged."""
    if w.n_slots_min == w.n_slots:
        return torch.full((w.batch,), w.n_slots, dtype=torch.int32)
    g = _gen(SEED_BASE + w.cfg_id + 17, "cpu")
    return torch.randint(w.n_slots_min, w.n_slots + 1, (w.batch,), generator=g,
                         dtype=torch.int64).to(torch.int32)


def make_keys(w: Workload, layer: int, device="cpu", ctx: Optional[torch.Tensor] = None,
              integer: bool = False) -> KeyCache:
    """Build the paged key cache of one layer.

    integer=True draws small integer keys (and power-of-two fp8 scales) so that
    every indexer score is exactly representable in fp32 whatever the
    summation order; used for bit-exact closed-loop checks.
    """
    R, Bc = w.batch, w.max_blocks
    ctx = context_lengths(w) if ctx is None else ctx
    n_pages = R * Bc
    if w.key_dtype == "f32":
        pages = torch.zeros(n_pages, BLOCK, HEAD_DIM, dtype=torch.float32, device=device)
    elif w.key_dtype == "bf16":
        pages = torch.zeros(n_pages, BLOCK, HEAD_DIM, dtype=torch.bfloat16, device=device)
    else:
        pages = torch.zeros(n_pages, BLOCK, HEAD_DIM, dtype=torch.uint8, device=device)
    scale = torch.ones(n_pages, BLOCK, dtype=torch.float32, device=device) \
        if w.key_dtype == "fp8" else None
    gp = _gen(sub_seed(w, layer, 0, salt=9), "cpu")
    perm = torch.randperm(n_pages, generator=gp) if w.shuffled_pages else torch.arange(n_pages)
    page_table = perm.view(R, Bc).to(torch.int32).contiguous()
    hf, hn = _layer_params(w, layer)
    us, heavies = [], []
    for r in range(R):
        N = int(ctx[r])
        g = _gen(sub_seed(w, layer, r), device)
        if integer:
            k = torch.randint(-4, 5, (N, HEAD_DIM), generator=g, device=device).to(torch.float32)
            u = torch.zeros(HEAD_DIM, device=device)
            u[:8] = 2.0
        else:
            k = torch.randn(N, HEAD_DIM, generator=g, device=device, dtype=torch.float32)
            gu = torch.randn(HEAD_DIM, generator=g, device=device, dtype=torch.float32)
            u = hn * gu / gu.norm()
        n_heavy = int(round(hf * N))
        heavy = torch.randperm(N, generator=g, device=device)[:n_heavy]
        k[heavy] += u
        if not integer:
            k = rope(k, torch.arange(N, device=device))
        Bn = -(-N // BLOCK)
        kp = torch.zeros(Bn * BLOCK, HEAD_DIM, dtype=torch.float32, device=device)
        kp[:N] = k
        kp = kp.view(Bn, BLOCK, HEAD_DIM)
        phys = page_table[r, :Bn].to(device=device, dtype=torch.int64)
        if w.key_dtype == "f32":
            pages[phys] = kp
        elif w.key_dtype == "bf16":
            pages[phys] = kp.to(torch.bfloat16)
        else:
            if integer:
                gs = torch.randint(-1, 2, (Bn, BLOCK), generator=g, device=device)
                sc = torch.pow(2.0, gs.to(torch.float32))
                codes = kp.to(torch.float8_e4m3fn).view(torch.uint8)
            else:
                codes, sc = encode_fp8(kp)
            pages[phys] = codes
            scale[phys] = sc
        us.append(u)
        heavies.append(heavy.cpu())
    return KeyCache(pages=pages, scale=scale, page_table=page_table.to(device),
                    u=torch.stack(us), heavy=heavies)


# --------------------------------------------------------------------------
# queries, weights, positions
# --------------------------------------------------------------------------
def make_weights(w: Workload, layer: int, device="cpu", integer: bool = False) -> torch.Tensor:
    """Head weights [R, rows, 64] float32 (fixed per request and layer)."""
    out = torch.empty(w.batch, N_HEADS, dtype=torch.float32)
    for r in range(w.batch):
        g = _gen(sub_seed(w, layer, r, salt=3), "cpu")
        if integer:
            out[r] = 0.5 * torch.randint(1, 5, (N_HEADS,), generator=g).to(torch.float32)
        else:
            out[r] = 0.5 + torch.rand(N_HEADS, generator=g, dtype=torch.float32)
    return out[:, None, :].expand(w.batch, w.rows, N_HEADS).contiguous().to(device)


def make_schedule(w: Workload, ctx: Optional[torch.Tensor] = None, n_steps: Optional[int] = None):
    """Row-0 query positions and acceptance lengths per step.

    Returns (pos [S, R] int64, accept [S, R] int32).  The first decode query
    sits at position N (one past the last cached slot); a step advances the
    position by its acceptance length (1 without speculative decoding).
    """
    ctx = context_lengths(w) if ctx is None else ctx
    S = w.steps if n_steps is None else n_steps
    if w.accept_probs is None or w.rows == 1:
        acc = torch.ones(S, w.batch, dtype=torch.int32)
    else:
        g = _gen(SEED_BASE + w.cfg_id + 101, "cpu")
        p = torch.tensor(w.accept_probs, dtype=torch.float64)
        acc = (torch.multinomial(p, S * w.batch, replacement=True, generator=g) + 1)
        acc = acc.view(S, w.batch).to(torch.int32)
    pos = torch.empty(S, w.batch, dtype=torch.int64)
    cur = ctx.to(torch.int64).clone()
    for s in range(S):
        pos[s] = cur
        cur = cur + acc[s].to(torch.int64)
    return pos, acc


def make_queries(w: Workload, layer: int, keys: KeyCache, pos: torch.Tensor,
                 device="cpu", integer: bool = False) -> torch.Tensor:
    """Queries for every step: [S, R, rows, 64, 128] float32 (RoPE applied).

    Row r of step s is the query at position pos[s] + r.  The AR(1) chain runs
    over positions, so re-evaluated draft positions see the same query.
    """
    S, R = pos.shape
    p0 = pos[0]
    span = int((pos[-1] - p0).max()) + w.rows
    out = torch.empty(S, R, w.rows, N_HEADS, HEAD_DIM, dtype=torch.float32, device=device)
    for r in range(R):
        g = _gen(sub_seed(w, layer, r, salt=5), device)
        if integer:
            chain = torch.randint(-3, 4, (span, N_HEADS, HEAD_DIM), generator=g,
                                  device=device).to(torch.float32)
        else:
            u = keys.u[r].to(device)
            chain = torch.empty(span, N_HEADS, HEAD_DIM, dtype=torch.float32, device=device)
            sd = 0.31 / math.sqrt(1.0 - 0.95 ** 2)
            q = 10.0 * u + sd * torch.randn(N_HEADS, HEAD_DIM, generator=g, device=device)
            for t in range(span):
                if t > 0:
                    q = 0.95 * q + 0.31 * torch.randn(N_HEADS, HEAD_DIM, generator=g,
                                                      device=device) + 0.5 * u
                chain[t] = q
            posv = p0[r] + torch.arange(span, device=device)
            chain = rope(chain.transpose(0, 1), posv).transpose(0, 1)
        idx = (pos[:, r] - p0[r])[:, None] + torch.arange(w.rows)[None, :]   # [S, rows]
        out[:, r] = chain[idx.to(device)]
    return out


def cast_queries(w: Workload, q: torch.Tensor) -> torch.Tensor:
    return q.to(torch.bfloat16) if w.q_dtype == "bf16" else q.to(torch.float32)


# --------------------------------------------------------------------------
# synthetic stage inputs (for per-stage parity with identical input bytes)
# --------------------------------------------------------------------------
def make_ema_state(R: int, n_cap: int, d_cap: int, seed: int, ties: bool = False,
                   zero_frac: float = 0.0):
    """Random non-negative fp32 V [R, n_cap] and D [R, d_cap] EMA states."""
    g = _gen(seed, "cpu")
    V = torch.randn(R, n_cap, generator=g).abs() * 10.0
    D = torch.randn(R, d_cap, generator=g).abs() * 10.0
    if ties:
        V = torch.round(V)
        D = torch.round(D)
    if zero_frac > 0:
        V[torch.rand(R, n_cap, generator=g) < zero_frac] = 0.0
        D[torch.rand(R, d_cap, generator=g) < zero_frac] = 0.0
    return V.to(torch.float32), D.to(torch.float32)


def make_scores(shape, seed: int, ties: bool = False, signed: bool = False) -> torch.Tensor:
    """Random fp32 indexer-score-like values; ties=True rounds to a coarse grid."""
    g = _gen(seed, "cpu")
    z = torch.randn(*shape, generator=g) * 20.0
    if not signed:
        z = z.abs()
    if ties:
        z = torch.round(z * 0.25) * 4.0
    return z.to(torch.float32)


def make_selection(R: int, n_blocks: torch.Tensor, max_blocks: int, frac: float, seed: int):
    """Random ascending block lists: (sel [R, max_blocks] int32 padded -1, n_sel [R] int32)."""
    g = _gen(seed, "cpu")
    sel = torch.full((R, max_blocks), -1, dtype=torch.int32)
    n_sel = torch.zeros(R, dtype=torch.int32)
    for r in range(R):
        B = int(n_blocks[r])
        keep = torch.rand(B, generator=g) < frac
        keep[0] = True
        keep[B - 1] = True
        idx = torch.nonzero(keep).flatten().to(torch.int32)
        sel[r, :idx.numel()] = idx
        n_sel[r] = idx.numel()
    return sel, n_sel
