"""SPIN decode-step hot path for AMD Instinct MI355X (gfx950).

The compute lives in libspin.so (hand-written HIP kernels behind the C ABI of
include/spin.h); this package only marshals torch tensors into that ABI.
"""
from . import _lib  # noqa: F401
from .api import (batch, config, spin_advance, spin_ema_update, spin_predict_blocks,  # noqa: F401
                  spin_reset_state, spin_select_blocks, spin_sparse_index_score, spin_stack_step,
                  spin_step, spin_step_finish, spin_step_plan, spin_topk, step_io,
                  workspace_bytes, Stack)
from .layer import SpinLayer, SpinStack  # noqa: F401
