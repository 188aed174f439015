"""Plain, slow, obviously-correct CPU oracle for SPIN's decode step.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library.

Sources (cited by page title and section):
  * "SPIN: Shadow Predictive Indexer for Sparse Attention" (arXiv 2610.09025),
    Sec. 2 (indexer score z_t[i] = sum_h w_h ReLU(q_{t,h} . k_{i,h})),
    Sec. 3.2 Eq. 1 (predicted slot score), Eq. 2 (block max pooling),
    Algorithm 1 (block budget, block top-m, indexer, top-K, EMA update) and the
    prose after it (reset, dense first step, sink and newest block always kept),
    Sec. 3.2.1 (exploration share inside the budget), Sec. 3.2.2 (verifier
    rows, mask union, deferred in-order EMA replay of prefix-valid rows),
    Sec. 4.1 (64-slot logical blocks, max pooling).
  * The project blog "Sparse Attention Still Has a Dense Problem", sections
    "Score only where history points" and "SPIN works with speculative
    decoding" (same method, prose form).
  * Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
    Easy as 1, 2, 3", SC'11 (the counter-based generator used for exploration).

Readings where the pages are silent (each is listed in the design doc):
  * All positions are compressed-slot coordinates; row r of a step sits at
    q_pos + r; D is indexed by the offset q - i >= 1.
  * combine = max (Eq. 1) by default; combine = sum (one fp32 add) is the
    variant the tiny workload states.
  * Ties rank the lower index first (blocks and slots).  -0 ranks as +0.
  * Budget arithmetic in integer basis points: m = min(B, max(ceil(K/b),
    ceil((10000 - rho_bp) * B / 10000))).
  * Forced blocks {0, B-1} count toward m; n_e = min(floor(m*gamma_bp/1e4),
    m - n_f); ranked = top (m - n_f - n_e) of the rest; explored = the n_e
    smallest Philox priorities (ties: lower block) among blocks neither forced
    nor ranked.  Priority of block j = first output word of
    Philox4x32-10(counter=(j, t, layer, req_id), key=(seed_lo, seed_hi)); the
    counter has no row field, so verifier rows share priorities.
  * If m < n_f (only possible for B <= 2 blocks budgets), the forced blocks are
    still all kept.
  * Step t = 0 after a reset scores every block (dense warm-up).
  * With bf16 or fp8 keys the indexer score is evaluated in fp64 from the
    decoded inputs (fp8 keys dequantised as code * scale).  Everything
    downstream of the score (top-K, EMA) consumes it rounded to fp32, the
    storage precision of the state.
  * With fp32 keys and fp32 queries (the exact mode) the score is one
    canonical fp32 evaluation: per head a sequential fmaf chain over the 128
    dims, ReLU, then a sequential fmaf chain over the heads (score_f32.c).
  * EMA in fp32 with three roundings: V' = fl(fl(a*V) + fl(b*z)), b = fl(1 - a).
  * top-K returns min(K, |dom|) slot ids in ascending order, padded with -1.
  * MTP: each row predicts its own mask; the union is scored for every row;
    each row's top-K runs over the whole union; after acceptance the first L
    rows are replayed in row order.
"""
from __future__ import annotations

import numpy as np

BLOCK = 64
CODE_SKIP, CODE_FORCED, CODE_RANKED, CODE_EXPLORED, CODE_DENSE = 0, 1, 2, 3, 4
MASK32 = 0xFFFFFFFF

# --------------------------------------------------------------------------
# Philox4x32-10 (Salmon et al., SC'11): 10 rounds of the 4x32 S-box with
# multipliers 0xD2511F53 / 0xCD9E8D57 and Weyl key increments 0x9E3779B9 /
# 0xBB67AE85.
# --------------------------------------------------------------------------
PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85


def philox4x32_10(ctr, key):
    """Vectorised Philox4x32-10.

    ctr: 4 arrays (or ints) of uint32 words (c0, c1, c2, c3); key: (k0, k1).
    Returns four uint64 arrays holding the 32-bit output words.
    """
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & MASK32 for c in ctr)
    k0 = np.uint64(int(key[0]) & MASK32)
    k1 = np.uint64(int(key[1]) & MASK32)
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    w0, w1 = np.uint64(PHILOX_W0), np.uint64(PHILOX_W1)
    mask, sh = np.uint64(MASK32), np.uint64(32)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + w0) & mask
            k1 = (k1 + w1) & mask
        p0 = m0 * c0               # < 2^64, exact in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> sh, p0 & mask
        hi1, lo1 = p1 >> sh, p1 & mask
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0
    return c0, c1, c2, c3


def block_priority(n_blocks: int, step: int, layer: int, req_id: int, seed: int):
    """Exploration priority of blocks 0..n_blocks-1 (uint64 holding u32)."""
    j = np.arange(n_blocks, dtype=np.uint64)
    z = np.zeros_like(j)
    out = philox4x32_10((j, z + np.uint64(step & MASK32), z + np.uint64(layer & MASK32),
                         z + np.uint64(req_id & MASK32)),
                        (seed & MASK32, (seed >> 32) & MASK32))
    return out[0]


# --------------------------------------------------------------------------
# number formats (decoded exactly into float64)
# --------------------------------------------------------------------------
def decode_e4m3(codes) -> np.ndarray:
    """OCP FP8 E4M3 (bias 7, no infinities, S.1111.111 = NaN) -> float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = s * (m / 8.0) * 2.0 ** -6
    nrm = s * (1.0 + m / 8.0) * np.exp2(e - 7.0)
    out = np.where(e == 0, sub, nrm)
    return np.where((e == 15) & (m == 7), np.nan, out)


def decode_bf16(codes) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 (exact: bf16 is the top half of fp32)."""
    c = np.asarray(codes).astype(np.uint32) << np.uint32(16)
    return c.view(np.float32).astype(np.float64)


def f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32)


def canon32(x) -> np.ndarray:
    """Round to fp32 and map -0 to +0 (ranking treats them as equal anyway)."""
    y = np.asarray(x, dtype=np.float32)
    return (y + np.float32(0.0)).astype(np.float32)


# --------------------------------------------------------------------------
# Stage 1 -- predicted block scores (Eq. 1, Eq. 2; Algorithm 1 steps 1-3)
# --------------------------------------------------------------------------
def n_blocks(n_slots: int, b: int = BLOCK) -> int:
    return -(-int(n_slots) // b)


def pool_block(vals, pooling: str = "max"):
    """Pool one block's predicted slot scores (fp32, the valid slots in slot
    order) into its block score (paper Sec. 4.6, "Block reduction", A1):
      max  -- the largest (Eq. 2, the default);
      top4 -- the up to four largest, summed largest first in fp32, divided
              by their count;
      mean -- the 64 slot values (0 past the context) summed as a balanced
              pairwise tree in fp32, ((s0 + s1) + (s2 + s3)) + ..., divided by
              the number of valid slots."""
    vals = np.asarray(vals, dtype=np.float32)
    n = len(vals)
    if pooling == "max":
        return np.float32(vals.max())
    if pooling == "top4":
        top = np.sort(vals)[::-1][:min(4, n)]
        s = np.float32(top[0])
        for x in top[1:]:
            s = np.float32(s + x)
        return np.float32(s / np.float32(len(top)))
    if pooling == "mean":
        v = np.zeros(BLOCK, dtype=np.float32)
        v[:n] = vals
        while len(v) > 1:
            v = (v[0::2] + v[1::2]).astype(np.float32)
        return np.float32(v[0] / np.float32(n))
    raise ValueError(pooling)


def predict_block_scores(V, D, n_slots: int, q: int, combine: str = "max", b: int = BLOCK,
                         pooling: str = "max"):
    """S[j] = pool over jb <= i < min((j+1)b, N) of C(V[i], D[q - i]).

    V: fp32 [>= N]; D: fp32 [> q]; q: the query position of this row.
    C = max (Eq. 1) or an fp32 sum; pool = max (Eq. 2) or a variant of
    pool_block.  Returns fp32 [B].
    """
    N = int(n_slots)
    i = np.arange(N)
    v = f32(V)[:N]
    d = f32(D)[q - i]
    if combine == "max":
        zhat = np.maximum(v, d)
    elif combine == "sum":
        zhat = (v + d).astype(np.float32)
    else:
        raise ValueError(combine)
    B = n_blocks(N, b)
    S = np.empty(B, dtype=np.float32)
    for j in range(B):
        S[j] = pool_block(zhat[j * b:min((j + 1) * b, N)], pooling)
    return canon32(S)


# --------------------------------------------------------------------------
# Stage 2 -- budget and block selection (Algorithm 1 steps 4-5; Sec. 3.2.1)
# --------------------------------------------------------------------------
def block_budget(B: int, K: int, sparsity_bp: int, b: int = BLOCK) -> int:
    keep = -(-(10000 - int(sparsity_bp)) * int(B) // 10000)
    return min(int(B), max(-(-int(K) // b), keep))


def rank_desc(values, candidates):
    """candidates ordered by (value descending, index ascending)."""
    cand = np.asarray(candidates, dtype=np.int64)
    v = np.asarray(values)[cand].astype(np.float64)
    order = np.lexsort((cand, -v))
    return cand[order]


def exploration_order(pool, S, step: int, layer: int, req_id: int, seed: int,
                      explore: str = "random", last_obs=None):
    """The blocks of `pool` in the order exploration takes them (paper Sec. 3.2.1
    and Sec. 4.6, "Staleness mitigation"; ties: lower block):
      random    -- smallest Philox priority first (the method);
      age       -- least recently observed first: smallest last_obs[j], the
                   step at which block j was last scored;
      staleness -- predicted importance weighted by staleness first: largest
                   S[j] * (step - last_obs[j]), one fp32 product."""
    pool = np.asarray(pool, dtype=np.int64)
    if explore == "random":
        pri = block_priority(int(pool.max()) + 1 if pool.size else 0, step, layer, req_id, seed)
        return pool[np.lexsort((pool, pri[pool]))]
    obs = np.asarray(last_obs, dtype=np.int64)[pool]
    if explore == "age":
        return pool[np.lexsort((pool, obs))]
    if explore == "staleness":
        age = (np.int64(step) - obs).astype(np.float32)
        score = canon32((f32(S)[pool] * age).astype(np.float32)).astype(np.float64)
        return pool[np.lexsort((pool, -score))]
    raise ValueError(explore)


def select_blocks(S, n_slots: int, K: int, sparsity_bp: int, explore_bp: int, step: int,
                  layer: int, req_id: int, seed: int, budget=None, b: int = BLOCK,
                  explore: str = "random", last_obs=None):
    """Reason-coded block mask of one verifier row (uint8 [B]).

    Codes: 0 skip, 1 forced, 2 ranked, 3 explored, 4 dense warm-up.
    budget: optional override of m (used by per-layer budgets).
    explore / last_obs: the exploration policy (exploration_order).
    """
    B = n_blocks(n_slots, b)
    code = np.zeros(B, dtype=np.uint8)
    if step == 0:
        code[:] = CODE_DENSE
        return code
    m = block_budget(B, K, sparsity_bp, b) if budget is None or budget <= 0 \
        else min(B, int(budget))
    forced = sorted({0, B - 1})
    n_f = len(forced)
    m = max(m, n_f)
    n_e = min(m * int(explore_bp) // 10000, m - n_f)
    n_r = m - n_f - n_e
    code[forced] = CODE_FORCED
    rest = [j for j in range(B) if code[j] == CODE_SKIP]
    ranked = rank_desc(S, rest)[:n_r]
    code[ranked] = CODE_RANKED
    pool = np.array([j for j in range(B) if code[j] == CODE_SKIP], dtype=np.int64)
    if n_e > 0 and pool.size:
        order = exploration_order(pool, S, step, layer, req_id, seed, explore, last_obs)
        code[order[:n_e]] = CODE_EXPLORED
    return code


def a0_select(zhat, n_slots: int, K: int, explore_bp: int, step: int, layer: int, req_id: int,
              seed: int, S=None, explore: str = "random", last_obs=None, b: int = BLOCK):
    """Block mask of one verifier row under block reduction A0 (paper Sec. 4.6,
    "Block reduction"): the K slots with the largest predicted slot score
    zhat (fp32 [N]; ties: lower slot; K the post-indexer top-K size), then
    every block holding one of them (code 2), with the sink and newest blocks
    (code 1) and floor(|mask| gamma) exploration blocks (code 3) from the
    rest, |mask| the forced and expanded blocks.  The budget does not bound
    A0: its realized sparsity follows from how the K slots spread."""
    N = int(n_slots)
    B = n_blocks(N, b)
    code = np.zeros(B, dtype=np.uint8)
    if step == 0:
        code[:] = CODE_DENSE
        return code
    z = canon32(np.asarray(zhat, dtype=np.float32)[:N]).astype(np.float64)
    slots = np.arange(N)
    top = slots[np.lexsort((slots, -z))[:min(int(K), N)]]
    code[np.unique(top // b)] = CODE_RANKED
    code[sorted({0, B - 1})] = CODE_FORCED
    m = int((code != CODE_SKIP).sum())
    n_e = m * int(explore_bp) // 10000
    pool = np.array([j for j in range(B) if code[j] == CODE_SKIP], dtype=np.int64)
    if n_e > 0 and pool.size:
        order = exploration_order(pool, S, step, layer, req_id, seed, explore, last_obs)
        code[order[:n_e]] = CODE_EXPLORED
    return code


def predicted_slot_scores(V, D, n_slots: int, q: int, combine: str = "max"):
    """zhat[i] = C(V[i], D[q - i]) for i < N (Eq. 1), fp32."""
    N = int(n_slots)
    i = np.arange(N)
    v, d = f32(V)[:N], f32(D)[q - i]
    return (np.maximum(v, d) if combine == "max" else (v + d).astype(np.float32)).astype(np.float32)


# --------------------------------------------------------------------------
# Block reduction A2 (paper Sec. 4.6, "Block reduction"): block-level V / D
# EMA states updated from pooled indexer scores, predicting block scores
# directly.  Vb[j] per block, Db[floor(q / b) - j] per block offset.
# --------------------------------------------------------------------------
def predict_block_scores_a2(Vb, Db, n_slots: int, q: int, combine: str = "max", b: int = BLOCK):
    """S[j] = C(Vb[j], Db[floor(q / b) - j]) for j < B, fp32."""
    B = n_blocks(n_slots, b)
    j = np.arange(B)
    v, d = f32(Vb)[:B], f32(Db)[q // b - j]
    S = np.maximum(v, d) if combine == "max" else (v + d).astype(np.float32)
    return canon32(S)


def pool_scores(z32, sel_blocks, n_slots: int, pooling: str = "max", b: int = BLOCK):
    """The pooled indexer score of each selected block (pool_block over its
    valid slots' fp32 scores, in slot order)."""
    z32 = np.asarray(z32, dtype=np.float32)
    N = int(n_slots)
    out = np.empty(len(sel_blocks), dtype=np.float32)
    pos = 0
    for k, j in enumerate(sel_blocks):
        n = min(b, N - int(j) * b)
        out[k] = pool_block(canon32(z32[pos:pos + n]), pooling)
        pos += n
    return canon32(out)


def ema_update_a2(Vb, Db, z_rows, sel_blocks, n_slots: int, q_pos: int, n_valid: int,
                  alpha: float, pooling: str = "max", b: int = BLOCK):
    """In-place block-level EMA of rows 0..n_valid-1 in row order: for each
    selected block j, with zb its pooled score of that row,
      Vb[j] <- (a Vb[j]) + (be zb),  Db[floor((q + r) / b) - j] <- likewise,
    three fp32 roundings each, be = fl(1 - a)."""
    a = np.float32(alpha)
    bcoef = np.float32(np.float32(1.0) - a)
    blocks = np.asarray(sel_blocks, dtype=np.int64)
    for r in range(int(n_valid)):
        zb = pool_scores(z_rows[r], blocks, n_slots, pooling, b)
        Vb[blocks] = (a * Vb[blocks]).astype(np.float32) + (bcoef * zb).astype(np.float32)
        off = (q_pos + r) // b - blocks
        Db[off] = (a * Db[off]).astype(np.float32) + (bcoef * zb).astype(np.float32)


def union_blocks(codes_rows):
    """Ascending list of blocks selected by any verifier row (Sec. 3.2.2)."""
    any_sel = np.zeros(len(codes_rows[0]), dtype=bool)
    for c in codes_rows:
        any_sel |= np.asarray(c) != CODE_SKIP
    return np.nonzero(any_sel)[0].astype(np.int64)


def union_slots(sel_blocks, n_slots: int, b: int = BLOCK):
    """dom(z): the slots < N of the selected blocks, ascending."""
    if len(sel_blocks) == 0:
        return np.zeros(0, dtype=np.int64)
    s = (np.asarray(sel_blocks, dtype=np.int64)[:, None] * b + np.arange(b)[None, :]).ravel()
    return s[s < n_slots]


# --------------------------------------------------------------------------
# Stage 3a -- the indexer on the selected slots (Sec. 2)
# --------------------------------------------------------------------------
def gather_keys(pages, page_table_row, slots, key_dtype: str, scale=None):
    """Dequantised keys of the given logical slots of one request (float64 [n, d])."""
    slots = np.asarray(slots, dtype=np.int64)
    phys = np.asarray(page_table_row, dtype=np.int64)[slots // BLOCK]
    off = slots % BLOCK
    raw = np.asarray(pages)[phys, off]
    if key_dtype == "f32":
        k = raw.astype(np.float64)
    elif key_dtype == "bf16":
        k = decode_bf16(raw)
    elif key_dtype == "fp8":
        k = decode_e4m3(raw) * np.asarray(scale, dtype=np.float64)[phys, off][:, None]
    else:
        raise ValueError(key_dtype)
    return k


def decode_q(q, q_dtype: str):
    if q_dtype == "f32":
        return np.asarray(q, dtype=np.float64)
    if q_dtype == "bf16":
        return decode_bf16(q)
    raise ValueError(q_dtype)


def index_scores_exact_f32(q, w, keys):
    """z[i] = sum_h w_h * ReLU(q_h . k_i) in the canonical fp32 order (exact
    mode, fp32 keys and queries): see oracle/score_f32.c.  Returns fp32 [n]."""
    from .score_f32 import index_scores_f32
    return index_scores_f32(np.asarray(q, dtype=np.float32), np.asarray(w, dtype=np.float32),
                            np.asarray(keys, dtype=np.float32))


def index_scores(q, w, keys):
    """z[i] = sum_h w_h * ReLU(q_h . k_i) in float64.

    q: [n_h, d] float64, w: [n_h], keys: [n, d] float64 -> [n].
    """
    dots = np.asarray(keys, dtype=np.float64) @ np.asarray(q, dtype=np.float64).T  # [n, n_h]
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)


# --------------------------------------------------------------------------
# Stage 3b -- post-indexer top-K (Algorithm 1 step 7)
# --------------------------------------------------------------------------
def topk_slots(z32, slots, K: int):
    """min(K, n) slot ids with the largest fp32 z (ties: lower slot), ascending, -1 padded."""
    z = canon32(z32).astype(np.float64)
    slots = np.asarray(slots, dtype=np.int64)
    order = np.lexsort((slots, -z))
    chosen = np.sort(slots[order[:K]])
    out = np.full(K, -1, dtype=np.int64)
    out[:chosen.size] = chosen
    return out


# --------------------------------------------------------------------------
# Stage 4 -- EMA update (Algorithm 1 steps 8-10; Sec. 3.2.2 deferred replay)
# --------------------------------------------------------------------------
def ema_update(V, D, z_rows, slots, q_pos: int, n_valid: int, alpha: float):
    """In-place fp32 EMA update of V and D from rows 0..n_valid-1, in row order.

    z_rows: fp32 [rows, len(slots)]; row r's query sits at q_pos + r.
    """
    a = np.float32(alpha)
    bcoef = np.float32(np.float32(1.0) - a)
    slots = np.asarray(slots, dtype=np.int64)
    for r in range(int(n_valid)):
        z = canon32(z_rows[r])
        V[slots] = (a * V[slots]).astype(np.float32) + (bcoef * z).astype(np.float32)
        off = (q_pos + r) - slots
        D[off] = (a * D[off]).astype(np.float32) + (bcoef * z).astype(np.float32)


# --------------------------------------------------------------------------
# One decode step of one (request, layer)
# --------------------------------------------------------------------------
class RequestState:
    """V, D and the step counter of one request in one layer (reset: zeros, t = 0)."""

    def __init__(self, n_cap: int, d_cap: int):
        self.V = np.zeros(n_cap, dtype=np.float32)
        self.D = np.zeros(d_cap, dtype=np.float32)
        # the step at which each block was last scored (block age / staleness)
        self.last_obs = np.zeros(n_blocks(n_cap), dtype=np.int64)
        self.t = 0

    def reset(self):
        self.V[:] = 0
        self.D[:] = 0
        self.last_obs[:] = 0
        self.t = 0


def spin_step(state: RequestState, *, q, q_dtype, w, pages, page_table_row, key_dtype,
              scale, n_slots: int, q_pos: int, K: int, sparsity_bp: int, explore_bp: int,
              alpha: float, layer: int, req_id: int, seed: int, combine: str = "max",
              n_valid=None, budget=None, defer=False, pooling: str = "max",
              mtp_row0_mask: bool = False, mtp_row0_update: bool = False,
              explore_per_row: bool = False, exact_f32: bool = True,
              explore: str = "random", reduction: str = "A1"):
    """One SPIN decode step for one request: predict, select, union, score, top-K, EMA.

    q: [rows, n_h, d] (raw f32 or bf16 codes), w: [rows, n_h].
    Returns a dict with codes [rows, B], sel, slots, z64 [rows, n], z32, topk [rows, K].
    z32 is what top-K and the EMA consume: the fp64 score rounded to fp32, or,
    with fp32 keys and queries and exact_f32 (the default), the canonical fp32
    evaluation of index_scores_exact_f32.
    The EMA update uses rows 0..n_valid-1 (all rows when n_valid is None) unless
    defer=True, in which case the caller replays later with ema_update.
    Variants (the paper's ablations, Sec. 4.5 and 4.6; defaults = the method):
    `pooling` (pool_block); mtp_row0_mask: score row 0's mask alone (row-0
    sharing); mtp_row0_update: the EMA takes row 0 only (row-0 update);
    explore_per_row: row r's exploration priorities come from the counter
    (j, t, layer + 65536 r, req_id); explore: the exploration policy
    (exploration_order: random, age, staleness); reduction: where slot
    signals become blocks (Sec. 4.6): A1 pools predicted slot scores (the
    method), A0 expands the predicted top-K slots (a0_select), A2 keeps
    block-level V / D (state.V, state.D indexed by block and block offset).
    Every block of the scored union is recorded as observed at step t.
    """
    rows = q.shape[0]
    qd = decode_q(q, q_dtype)
    codes = []
    for r in range(rows):
        q = q_pos + r
        if reduction == "A2":
            S = predict_block_scores_a2(state.V, state.D, n_slots, q, combine)
        else:
            S = predict_block_scores(state.V, state.D, n_slots, q, combine, pooling=pooling)
        lay = layer + 65536 * r if explore_per_row else layer
        if reduction == "A0":
            zhat = predicted_slot_scores(state.V, state.D, n_slots, q, combine)
            codes.append(a0_select(zhat, n_slots, K, explore_bp, state.t, lay, req_id, seed,
                                   S=S, explore=explore, last_obs=state.last_obs))
        else:
            codes.append(select_blocks(S, n_slots, K, sparsity_bp, explore_bp, state.t, lay,
                                       req_id, seed, budget, explore=explore,
                                       last_obs=state.last_obs))
    codes = np.stack(codes)
    sel = union_blocks(codes[:1] if mtp_row0_mask else codes)
    state.last_obs[sel] = state.t
    slots = union_slots(sel, n_slots)
    keys = gather_keys(pages, page_table_row, slots, key_dtype, scale)
    z64 = np.stack([index_scores(qd[r], w[r], keys) for r in range(rows)])
    if key_dtype == "f32" and q_dtype == "f32" and exact_f32:
        z32 = np.stack([index_scores_exact_f32(qd[r], w[r], keys) for r in range(rows)])
    else:
        z32 = canon32(z64)
    top = np.stack([topk_slots(z32[r], slots, K) for r in range(rows)])
    if not defer:
        nv = 1 if mtp_row0_update else (rows if n_valid is None else n_valid)
        if reduction == "A2":
            ema_update_a2(state.V, state.D, z32, sel, n_slots, q_pos, nv, alpha, pooling)
        else:
            ema_update(state.V, state.D, z32, slots, q_pos, nv, alpha)
        state.t += 1
    return dict(codes=codes, sel=sel, slots=slots, z64=z64, z32=z32, topk=top)
