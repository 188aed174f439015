"""HIP graph capture of a whole decode step (blog "Per-layer block budgets"
and "Faster decoding in vLLM": the method runs under CUDA graphs).

A spin_step, and a one-stream spin_stack_step of three layers, are captured
once (their launches only: the library issues no memset, copy or event on
these paths) and replayed once per decode step, with each step's query
copied into the captured input buffer beforehand.  Every replay must equal
the same step run eagerly on a twin layer, bit for bit; on integer-valued
inputs also the closed-loop oracle.  Eager work and host synchronisations
sit between the replays."""
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


def _state(lay):
    return [t.clone() for t in (lay.topk_idx, lay.V, lay.D, lay.z, lay.row_code, lay.sel,
                                lay.n_sel, lay.q_pos, lay.step_ctr, lay.S)]


@pytest.mark.parametrize("name", ["fp8", "fp8_mtp", "bf16"])
def test_graph_replay_of_spin_step(name):
    banner(f"graph replay of spin_step {name}")
    w = {"fp8": G.WORKLOADS["fp8_128k_b32"].scaled(batch=3, n_slots=8192, n_slots_min=6000,
                                                   steps=8, topk=512),
         "fp8_mtp": G.WORKLOADS["fp8_128k_b32_mtp4"].scaled(batch=3, n_slots=6000,
                                                            n_slots_min=4500, steps=8, topk=256),
         "bf16": G.WORKLOADS["bf16_64k_b16"].scaled(batch=3, n_slots=8192 + 64,
                                                    n_slots_min=5000, steps=8, topk=512)}[name]
    li = build_layer(w, integer=True)
    sp = w.sparsity_bp[0]
    eager, graphed = make_layer(li, sp), make_layer(li, sp)
    pages, scale, pt = device_keys(li)
    W = li.weights.to(DEV)
    q_in = li.q[0].to(DEV).contiguous().clone()
    nv_in = li.accept[0].to(DEV).clone()
    nv = (lambda t: t) if w.rows > 1 else (lambda t: None)
    # warm-up outside the capture (launch-configuration caches), then a
    # reset so both layers start from the same state
    graphed.step(q_in, W, pages, scale, pt, n_valid=nv(nv_in))
    torch.cuda.synchronize()
    graphed.set_requests(li.ctx.to(DEV), li.pos[0].to(DEV))
    graphed.reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.step(q_in, W, pages, scale, pt, n_valid=nv(nv_in))
    torch.cuda.synchronize()
    # capturing launched nothing: the layer is still fresh
    assert int(graphed.step_ctr.sum()) == 0
    ref, states = run_oracle(li, w.steps, sp)
    for s in range(w.steps):
        q_in.copy_(li.q[s].to(DEV))
        nv_in.copy_(li.accept[s].to(DEV))
        eager.step(li.q[s].to(DEV).contiguous(), W, pages, scale, pt,
                   n_valid=nv(li.accept[s].to(DEV)))
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(_state(eager), _state(graphed)):
            assert torch.equal(x, y), f"replay {s}"
        top = graphed.topk_idx.cpu().numpy()
        for r in range(w.batch):
            assert np.array_equal(top[r], ref[s][r]["topk"]), (s, r)
    for r in range(w.batch):
        N = int(li.ctx[r])
        assert np.array_equal(graphed.V.cpu().numpy()[r, :N], states[r].V[:N])
    assert int(graphed.err.item()) == 0 and int(eager.err.item()) == 0


def test_graph_replay_of_one_stream_stack():
    banner("graph replay of a one-stream 3-layer stack step")
    from sparse_attention_indexer_spin_amd import SpinStack
    n_layers = 3
    w = G.WORKLOADS["fp8_256k_ragged_8l"].scaled(batch=4, layers=n_layers, n_slots=64 * 150 + 9,
                                                 n_slots_min=3000, steps=6, topk=256)
    lis = [build_layer(w, layer=l, integer=True) for l in range(n_layers)]
    keys = [device_keys(li) for li in lis]
    eager = [make_layer(li, 4000) for li in lis]
    graphed = [make_layer(li, 4000) for li in lis]
    es = SpinStack(eager, one_stream=True)
    gs = SpinStack(graphed, one_stream=True)
    ws = [li.weights.to(DEV) for li in lis]
    q_in = [li.q[0].to(DEV).contiguous().clone() for li in lis]
    args = ([k[0] for k in keys], [k[1] for k in keys], [k[2] for k in keys])
    gs.step(q_in, ws, *args)                       # warm-up, then reset
    torch.cuda.synchronize()
    for lay, li in zip(graphed, lis):
        lay.set_requests(li.ctx.to(DEV), li.pos[0].to(DEV))
        lay.reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gs.step(q_in, ws, *args)
    torch.cuda.synchronize()
    for s in range(w.steps):
        for l, li in enumerate(lis):
            q_in[l].copy_(li.q[s].to(DEV))
        es.step([li.q[s].to(DEV).contiguous() for li in lis], ws, *args)
        g.replay()
        torch.cuda.synchronize()
        for l in range(n_layers):
            for x, y in zip(_state(eager[l]), _state(graphed[l])):
                assert torch.equal(x, y), f"replay {s} layer {l}"
    for l in range(n_layers):
        ref, states = run_oracle(lis[l], w.steps, 4000)
        top = graphed[l].topk_idx.cpu().numpy()
        for r in range(w.batch):
            assert np.array_equal(top[r], ref[w.steps - 1][r]["topk"]), (l, r)
    for lay in eager + graphed:
        assert int(lay.err.item()) == 0
