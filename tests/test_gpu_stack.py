"""Multi-layer decode steps through spin_stack_step (plans on a side stream,
score / top-K / EMA on the main stream): every layer's outputs and EMA state
must be bit-identical to the same layers stepped one after another with
spin_step on one stream, and to spin_step_plan + spin_step_finish; on
integer-valued inputs (every score exact in fp32) also to the CPU oracle,
closed loop."""
import numpy as np
import pytest
import torch

import spin_synth as G
from tests.gpu_util import DEV, banner, device_keys, make_layer
from tests.harness import build_layer, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_indexer_spin_amd import _lib
    return _lib.load()


def _workload(layers, steps=6):
    # ragged requests, per-layer heavy-slot fraction and direction norm
    return G.WORKLOADS["fp8_256k_ragged_8l"].scaled(batch=5, layers=layers, n_slots=64 * 150 + 9,
                                                    n_slots_min=3000, steps=steps, topk=256)


def _state(lay):
    return [t.clone() for t in (lay.topk_idx, lay.V, lay.D, lay.z, lay.row_code, lay.sel,
                                lay.n_sel, lay.q_pos, lay.step_ctr)]


@pytest.mark.parametrize("integer", [False, True])
@pytest.mark.parametrize("mode", ["side", "side+ema", "one_stream"])
def test_stack_matches_sequential_steps(integer, mode):
    banner(f"stack vs sequential integer={integer} mode={mode}")
    ema_stream, one_stream = mode == "side+ema", mode == "one_stream"
    from sparse_attention_indexer_spin_amd import SpinStack, api as A
    n_layers = 3
    w = _workload(n_layers)
    lis = [build_layer(w, layer=l, integer=integer) for l in range(n_layers)]
    keys = [device_keys(li) for li in lis]
    seq = [make_layer(li, 4000) for li in lis]
    stk_layers = [make_layer(li, 4000) for li in lis]
    split = [make_layer(li, 4000) for li in lis]
    stack = SpinStack(stk_layers, ema_stream=ema_stream, one_stream=one_stream)
    torch.cuda.synchronize()
    for s in range(w.steps):
        qs = [li.q[s].to(DEV).contiguous() for li in lis]
        ws = [li.weights.to(DEV) for li in lis]
        for l in range(n_layers):
            seq[l].step(qs[l], ws[l], *keys[l])
            lay = split[l]
            bt = lay.batch(keys[l][0].shape[0])
            io = lay.make_io(qs[l], ws[l], *keys[l])
            A.spin_step_plan(lay.cfg, bt, io)
            A.spin_step_finish(lay.cfg, bt, io)
        stack.step(qs, ws, [k[0] for k in keys], [k[1] for k in keys], [k[2] for k in keys])
        torch.cuda.synchronize()
        for l in range(n_layers):
            a, b, c = _state(seq[l]), _state(stk_layers[l]), _state(split[l])
            for x, y, z in zip(a, b, c):
                assert torch.equal(x, y), f"stack differs from spin_step: step {s} layer {l}"
                assert torch.equal(x, z), f"plan+finish differs from spin_step: step {s} layer {l}"
    for lay in stk_layers + seq + split:
        assert int(lay.err.item()) == 0
    if not integer:
        return
    # integer inputs: every layer against the closed-loop oracle
    for l in range(n_layers):
        ref, states = run_oracle(lis[l], w.steps, 4000)
        top = stk_layers[l].topk_idx.cpu().numpy()
        for r in range(w.batch):
            assert np.array_equal(top[r], ref[w.steps - 1][r]["topk"]), (l, r)
            N = int(lis[l].ctx[r])
            assert np.array_equal(stk_layers[l].V.cpu().numpy()[r, :N], states[r].V[:N]), (l, r)


@pytest.mark.parametrize("one_stream", [False, True])
def test_stack_reuse_after_reset_and_fewer_layers(one_stream):
    """A reset between steps (announced with inputs_changed) and a step over a
    prefix of the layers: still identical to sequential spin_step calls."""
    banner(f"stack reset / layer prefix one_stream={one_stream}")
    from sparse_attention_indexer_spin_amd import SpinStack
    n_layers = 4
    w = _workload(n_layers, steps=5)
    lis = [build_layer(w, layer=l) for l in range(n_layers)]
    keys = [device_keys(li) for li in lis]
    seq = [make_layer(li, 3000) for li in lis]
    stk_layers = [make_layer(li, 3000) for li in lis]
    stack = SpinStack(stk_layers, one_stream=one_stream)
    for s in range(w.steps):
        qs = [li.q[s].to(DEV).contiguous() for li in lis]
        ws = [li.weights.to(DEV) for li in lis]
        if s == 3:                                 # no host sync before the reset
            for lay in seq:
                lay.reset()
            stack.reset()
        use = n_layers if s != 2 else 2            # step 2 runs layers 0-1 only
        for l in range(use):
            seq[l].step(qs[l], ws[l], *keys[l])
        stack.step(qs, ws, [k[0] for k in keys], [k[1] for k in keys], [k[2] for k in keys],
                   n_layers=use)
        if s == 2:
            continue                               # step 3's reset follows without a host sync
        torch.cuda.synchronize()
        for l in range(n_layers):
            for x, y in zip(_state(seq[l]), _state(stk_layers[l])):
                assert torch.equal(x, y), f"step {s} layer {l}"


def test_stack_switches_between_one_and_two_streams():
    """Steps alternating the one-stream and the side-stream schedules on one
    stack: identical to sequential spin_step calls (a two-stream call after a
    one-stream call orders its plans after everything issued on main)."""
    banner("stack mode switch")
    from sparse_attention_indexer_spin_amd import SpinStack
    n_layers = 3
    w = _workload(n_layers, steps=6)
    lis = [build_layer(w, layer=l) for l in range(n_layers)]
    keys = [device_keys(li) for li in lis]
    seq = [make_layer(li, 4000) for li in lis]
    stk_layers = [make_layer(li, 4000) for li in lis]
    stack = SpinStack(stk_layers)
    for s in range(w.steps):
        stack.one_stream = s % 2 == 0
        qs = [li.q[s].to(DEV).contiguous() for li in lis]
        ws = [li.weights.to(DEV) for li in lis]
        for l in range(n_layers):
            seq[l].step(qs[l], ws[l], *keys[l])
        stack.step(qs, ws, [k[0] for k in keys], [k[1] for k in keys], [k[2] for k in keys])
    torch.cuda.synchronize()
    for l in range(n_layers):
        for x, y in zip(_state(seq[l]), _state(stk_layers[l])):
            assert torch.equal(x, y), f"layer {l}"


def test_stack_switches_from_ema_stream_to_one_stream():
    """A one-stream call right after a call whose EMA updates ran on the EMA
    stream: main waits for those updates before its first plan reads V / D."""
    banner("stack switch: side + EMA stream -> one stream")
    from sparse_attention_indexer_spin_amd import SpinStack
    n_layers = 3
    w = _workload(n_layers, steps=6)
    lis = [build_layer(w, layer=l) for l in range(n_layers)]
    keys = [device_keys(li) for li in lis]
    seq = [make_layer(li, 4000) for li in lis]
    stk_layers = [make_layer(li, 4000) for li in lis]
    stack = SpinStack(stk_layers, ema_stream=True)
    ema = stack.ema
    for s in range(w.steps):
        two = s % 2 == 0
        stack.one_stream, stack.ema = (False, ema) if two else (True, None)
        qs = [li.q[s].to(DEV).contiguous() for li in lis]
        ws = [li.weights.to(DEV) for li in lis]
        for l in range(n_layers):
            seq[l].step(qs[l], ws[l], *keys[l])
        stack.step(qs, ws, [k[0] for k in keys], [k[1] for k in keys], [k[2] for k in keys])
    stack.ema = ema
    stack.join()
    torch.cuda.synchronize()
    for l in range(n_layers):
        for x, y in zip(_state(seq[l]), _state(stk_layers[l])):
            assert torch.equal(x, y), f"layer {l}"


@pytest.mark.parametrize("rows", [1, 4])
@pytest.mark.parametrize("mode", ["side", "one_stream"])
def test_stack_deferred_ema_matches_step_and_commit(rows, mode):
    """Speculative decoding through the stack: spin_stack_step with the EMA
    deferred, then spin_stack_commit with each layer's accepted rows, equals
    per-layer spin_step(defer) + spin_ema_update / spin_advance (commit), bit
    for bit; on integer inputs also the closed-loop oracle with deferred
    replay (paper Sec. 3.2.2)."""
    banner(f"stack deferred EMA rows={rows} mode={mode}")
    from sparse_attention_indexer_spin_amd import SpinStack
    n_layers = 3
    base = "fp8_128k_b32_mtp4" if rows > 1 else "fp8_256k_ragged_8l"
    w = G.WORKLOADS[base].scaled(batch=4, layers=n_layers, n_slots=64 * 120 + 5, n_slots_min=3000,
                                 steps=6, topk=256, rows=rows)
    lis = [build_layer(w, layer=l, integer=True) for l in range(n_layers)]
    keys = [device_keys(li) for li in lis]
    seq = [make_layer(li, 4000) for li in lis]
    stk_layers = [make_layer(li, 4000) for li in lis]
    stack = SpinStack(stk_layers, one_stream=mode == "one_stream")
    for s in range(w.steps):
        qs = [li.q[s].to(DEV).contiguous() for li in lis]
        ws = [li.weights.to(DEV) for li in lis]
        nv = [li.accept[s].to(DEV) for li in lis]
        for l in range(n_layers):
            seq[l].step(qs[l], ws[l], *keys[l], n_valid=nv[l], defer_ema=True)
            seq[l].commit(nv[l])
        stack.step(qs, ws, [k[0] for k in keys], [k[1] for k in keys], [k[2] for k in keys],
                   defer_ema=True)
        if s == 1:   # a second step before the commit is refused
            from sparse_attention_indexer_spin_amd import _lib
            with pytest.raises(_lib.SpinError):
                stack.step(qs, ws, [k[0] for k in keys], [k[1] for k in keys],
                           [k[2] for k in keys], defer_ema=True)
        stack.commit(nv)
        stack.join()
        torch.cuda.synchronize()
        for l in range(n_layers):
            for x, y in zip(_state(seq[l]), _state(stk_layers[l])):
                assert torch.equal(x, y), f"step {s} layer {l}"
    for l in range(n_layers):
        ref, states = run_oracle(lis[l], w.steps, 4000)
        top = stk_layers[l].topk_idx.cpu().numpy()
        for r in range(w.batch):
            assert np.array_equal(top[r], ref[w.steps - 1][r]["topk"]), (l, r)
            N = int(lis[l].ctx[r])
            assert np.array_equal(stk_layers[l].V.cpu().numpy()[r, :N], states[r].V[:N]), (l, r)
    for lay in stk_layers + seq:
        assert int(lay.err.item()) == 0


@pytest.mark.parametrize("blocks", [1100, 2100, 5000])
def test_one_stream_stack_selection_widths(blocks):
    """The one-stream schedule selects layer l + 1's blocks inside layer l's
    top-K + EMA launch with 1, 2, 4 or 8 blocks per thread (up to 1,024, 2,048,
    4,096 and 8,192 blocks): at ~1,100, 2,100 and 5,000 blocks (2, 4 and 8 per
    thread) every layer equals sequential spin_step on V, D, S, codes, the
    block list and top-K."""
    banner(f"one-stream stack, {blocks} blocks per request")
    from sparse_attention_indexer_spin_amd import SpinLayer, SpinStack
    n_layers, steps, R = 3, 4, 2
    w = G.WORKLOADS["fp8_256k_ragged_8l"].scaled(batch=R, layers=n_layers, n_slots=64 * blocks - 17,
                                                 n_slots_min=64 * blocks // 2, steps=steps,
                                                 topk=1024)
    ctx = G.context_lengths(w)
    pos, _ = G.make_schedule(w, ctx, steps)
    keys, W, Q = [], [], []
    for l in range(n_layers):
        k = G.make_keys(w, l, DEV, ctx)
        keys.append(k)
        W.append(G.make_weights(w, l, DEV))
        Q.append(G.cast_queries(w, G.make_queries(w, l, k, pos, DEV)).contiguous())

    def layers():
        out = []
        for l in range(n_layers):
            lay = SpinLayer(batch=R, max_blocks=w.max_blocks, d_cap=G.d_capacity(w, steps),
                            topk=w.topk, sparsity_bp=4000, layer=l, device=DEV)
            lay.set_requests(ctx.to(DEV), pos[0].to(DEV))
            lay.reset()
            out.append(lay)
        return out

    seq, stk = layers(), layers()
    stack = SpinStack(stk, one_stream=True)
    for s in range(steps):
        for l in range(n_layers):
            seq[l].step(Q[l][s], W[l], keys[l].pages, keys[l].scale, keys[l].page_table)
        stack.step([Q[l][s] for l in range(n_layers)], W, [k.pages for k in keys],
                   [k.scale for k in keys], [k.page_table for k in keys])
        torch.cuda.synchronize()
        for l in range(n_layers):
            for x, y in zip(_state(seq[l]) + [seq[l].S], _state(stk[l]) + [stk[l].S]):
                assert torch.equal(x, y), f"step {s} layer {l}"
    for lay in seq + stk:
        assert int(lay.err.item()) == 0
