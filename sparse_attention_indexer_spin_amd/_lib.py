"""ctypes declarations of libspin.so (the C ABI in include/spin.h).

Loading fails loudly when the library has not been built: there is no other
implementation of the SPIN path in this package.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspin.so")

SPIN_OK = 0
STATUS = {0: "SPIN_OK", 1: "SPIN_E_NULL", 2: "SPIN_E_SHAPE", 3: "SPIN_E_UNSUPPORTED",
          4: "SPIN_E_WORKSPACE", 5: "SPIN_E_HIP"}
SPIN_F32, SPIN_BF16, SPIN_FP8_E4M3 = 0, 1, 2
SPIN_COMBINE_MAX, SPIN_COMBINE_SUM = 0, 1
SPIN_CODE_SKIP, SPIN_CODE_FORCED, SPIN_CODE_RANKED, SPIN_CODE_EXPLORED, SPIN_CODE_DENSE = range(5)
SPIN_DERR_CTX, SPIN_DERR_QPOS, SPIN_DERR_PAGE = 1, 2, 4
SPIN_MAX_ROWS, SPIN_MAX_BLOCKS, SPIN_MAX_TOPK, SPIN_MAX_LAYERS = 4, 8192, 8192, 256

EXPORTS = ["spin_predict_blocks", "spin_select_blocks", "spin_sparse_index_score", "spin_topk",
           "spin_ema_update", "spin_advance", "spin_reset_state", "spin_step",
           "spin_workspace_bytes", "spin_last_error", "spin_step_plan", "spin_step_finish",
           "spin_stack_create", "spin_stack_destroy", "spin_stack_step", "spin_miss_curve",
           "spin_budget_fill", "spin_budget_allocate", "spin_step_noalloc", "spin_stack_commit",
           "spin_budget_state_bytes", "spin_stack_set_budget_policy", "spin_stack_reset_budgets",
           "spin_budget_update", "spin_read_pages"]
SPIN_READ_PROBE_WAVES = 2048
SPIN_READ_PROBE_SINK_WORDS = SPIN_READ_PROBE_WAVES * 64
SPIN_NOALLOC_WORKSPACE_BYTES = 160 * 1024 * 1024
SPIN_BUDGET_MINIMAX, SPIN_BUDGET_PROPORTIONAL = 0, 1
SPIN_POOL_MAX, SPIN_POOL_TOP4, SPIN_POOL_MEAN = 0, 1, 2
SPIN_MTP_ROW0_MASK, SPIN_MTP_ROW0_UPDATE, SPIN_EXPLORE_PER_ROW = 4, 8, 16
SPIN_EXPLORE_AGE, SPIN_EXPLORE_STALENESS = 32, 64
SPIN_REDUCE_A0, SPIN_REDUCE_A2 = 128, 256
SPIN_PREDICT_AHEAD = 512


class SpinConfig(C.Structure):
    _fields_ = [("n_heads", C.c_int32), ("head_dim", C.c_int32), ("block_size", C.c_int32),
                ("topk", C.c_int32), ("sparsity_bp", C.c_int32), ("explore_bp", C.c_int32),
                ("ema_alpha", C.c_float), ("combine", C.c_int32), ("key_dtype", C.c_int32),
                ("q_dtype", C.c_int32), ("layer", C.c_int32), ("flags", C.c_int32),
                ("seed", C.c_uint64)]


class SpinBatch(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_rows", C.c_int32), ("max_blocks", C.c_int32),
                ("n_pages", C.c_int32), ("ctx_len", C.c_void_p), ("q_pos", C.c_void_p),
                ("step", C.c_void_p), ("req_id", C.c_void_p), ("err", C.c_void_p)]


class SpinStepIO(C.Structure):
    _fields_ = [("V", C.c_void_p), ("v_ld", C.c_int64), ("D", C.c_void_p), ("d_ld", C.c_int64),
                ("v_max", C.c_void_p), ("q", C.c_void_p), ("w", C.c_void_p), ("k_pages", C.c_void_p),
                ("k_scale", C.c_void_p), ("page_table", C.c_void_p), ("pt_ld", C.c_int64),
                ("budget", C.c_void_p), ("n_valid", C.c_void_p), ("S", C.c_void_p),
                ("row_code", C.c_void_p), ("sel", C.c_void_p), ("n_sel", C.c_void_p),
                ("z", C.c_void_p), ("z_ld", C.c_int64), ("topk_idx", C.c_void_p),
                ("q_pos_mut", C.c_void_p), ("step_mut", C.c_void_p), ("workspace", C.c_void_p),
                ("workspace_bytes", C.c_size_t), ("last_obs", C.c_void_p),
                ("s_tag", C.c_void_p)]


class SpinBudgetPolicy(C.Structure):
    _fields_ = [("policy", C.c_int32), ("probe_period", C.c_int32), ("levels", C.c_int32),
                ("target_level", C.c_int32), ("drift_bp", C.c_int32),
                ("level_table", C.c_void_p), ("budget", C.c_void_p),
                ("probe_budget", C.c_void_p), ("covered", C.c_void_p), ("kprime", C.c_void_p),
                ("state", C.c_void_p)]


_lib = None


def load() -> C.CDLL:
    """Load libspin.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libspin.so not built at {LIB_PATH}: run "
                           "`python -m sparse_attention_indexer_spin_amd.build`")
    lib = C.CDLL(LIB_PATH)
    P, I32, I64, SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    cfg, bt = C.POINTER(SpinConfig), C.POINTER(SpinBatch)
    sig = {
        "spin_predict_blocks": [cfg, bt, P, I64, P, I64, P, P, P],
        "spin_select_blocks": [cfg, bt, P, P, P, P, P, P, P],
        "spin_sparse_index_score": [cfg, bt, P, P, P, P, P, I64, P, P, P, I64, P, SZ, P],
        "spin_topk": [cfg, bt, P, I64, P, P, P, P, SZ, P],
        "spin_ema_update": [cfg, bt, P, I64, P, P, P, P, I64, P, I64, P, P],
        "spin_advance": [I32, I32, P, P, P, P],
        "spin_reset_state": [I32, P, I64, P, I64, P, I64, P, P],
        "spin_step": [cfg, bt, C.POINTER(SpinStepIO), I32, P],
        "spin_step_noalloc": [cfg, bt, C.POINTER(SpinStepIO), I32, P],
        "spin_step_plan": [cfg, bt, C.POINTER(SpinStepIO), P],
        "spin_step_finish": [cfg, bt, C.POINTER(SpinStepIO), I32, P],
        "spin_stack_create": [I32, C.POINTER(P)],
        "spin_stack_step": [P, I32, cfg, bt, C.POINTER(SpinStepIO), I32, I32, P, P, P],
        "spin_stack_commit": [P, I32, cfg, bt, C.POINTER(SpinStepIO), P],
        "spin_miss_curve": [cfg, bt, P, P, I32, P, P, P],
        "spin_budget_fill": [cfg, bt, P, I32, P, P],
        "spin_budget_allocate": [I32, I32, I32, I32, P, P, P, P],
        "spin_stack_set_budget_policy": [P, C.POINTER(SpinBudgetPolicy)],
        "spin_stack_reset_budgets": [P, I32, cfg, bt, P],
        "spin_budget_update": [I32, I32, I32, I32, I32, I32, P, P, P, P, P],
        "spin_read_pages": [P, I64, P, I32, P, P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = C.c_int
    lib.spin_stack_destroy.argtypes = [P]
    lib.spin_stack_destroy.restype = None
    lib.spin_workspace_bytes.argtypes = [cfg, I32, I32, I32]
    lib.spin_workspace_bytes.restype = SZ
    lib.spin_budget_state_bytes.argtypes = [I32, I32]
    lib.spin_budget_state_bytes.restype = SZ
    lib.spin_last_error.argtypes = []
    lib.spin_last_error.restype = C.c_char_p
    _lib = lib
    return lib


class SpinError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def check(status: int):
    if status != SPIN_OK:
        raise SpinError(status, load().spin_last_error().decode())
