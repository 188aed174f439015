"""spin_step_noalloc: the whole decode step on the library's static device
scratch, for callers that cannot allocate.  Through the C ABI it must give
what spin_step with a caller workspace gives, bit for bit, on two calls in a
row (the second on a smaller input, so the scratch holds the first call's
contents), and it must refuse shapes beyond its scratch."""
import numpy as np
import pytest
import torch

import spin_synth as G
from tests.gpu_util import DEV, banner, device_keys, make_layer
from tests.harness import build_layer

pytestmark = pytest.mark.gpu

OUTPUTS = ("S", "row_code", "sel", "n_sel", "z", "topk_idx", "V", "D", "q_pos", "step_ctr")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_indexer_spin_amd import _lib
    return _lib.load()


def _case(batch, n_slots, n_slots_min, rows, key):
    base = "fp8_128k_b32_mtp4" if rows > 1 else "fp8_128k_b32"
    w = G.WORKLOADS[base].scaled(batch=batch, n_slots=n_slots, n_slots_min=n_slots_min, steps=4,
                                 topk=512, key_dtype=key, q_dtype="bf16")
    return build_layer(w)


def _run_pair(li, n_steps):
    """The same steps through spin_step (caller workspace) and spin_step_noalloc."""
    from sparse_attention_indexer_spin_amd import api
    ref, lay = make_layer(li, 4000), make_layer(li, 4000)
    pages, scale, pt = device_keys(li)
    W = li.weights.to(DEV)
    for s in range(n_steps):
        q = li.q[s].to(DEV).contiguous()
        nv = li.accept[s].to(DEV) if li.w.rows > 1 else None
        ref.step(q, W, pages, scale, pt, n_valid=nv)
        bt = lay.batch(pages.shape[0])
        io = lay.make_io(q, W, pages, scale, pt, n_valid=nv)
        io.workspace, io.workspace_bytes = None, 0     # ignored by the no-alloc entry point
        api.spin_step_noalloc(lay.cfg, bt, io)
        torch.cuda.synchronize()
        for name in OUTPUTS:
            a, b = getattr(ref, name), getattr(lay, name)
            assert torch.equal(a, b), (s, name)
    assert int(lay.err.item()) == 0


def test_noalloc_step_equals_spin_step_twice_second_smaller():
    banner("no-alloc step: 6 x fp8 requests up to 20,000 slots, 4 rows, then 2 x bf16, 1 row")
    _run_pair(_case(6, 20000, 9000, 4, "fp8"), 3)
    _run_pair(_case(2, 5000, 3000, 1, "bf16"), 3)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    from sparse_attention_indexer_spin_amd import _lib, api
    banner("no-alloc step: a shape beyond the static scratch")
    cfg = api.config(topk=2048, sparsity_bp=4000)
    need = api.workspace_bytes(cfg, 4096, 4, 8192)
    assert need > _lib.SPIN_NOALLOC_WORKSPACE_BYTES
    i32 = dict(dtype=torch.int32, device=DEV)
    z = torch.zeros(4096, **i32)
    bt = api.batch(ctx_len=z, q_pos=z, step=z, req_id=z, n_rows=4, max_blocks=8192, n_pages=1)
    io = _lib.SpinStepIO()
    with pytest.raises(_lib.SpinError) as e:
        api.spin_step_noalloc(cfg, bt, io)
    assert e.value.status == 4                                   # SPIN_E_WORKSPACE
