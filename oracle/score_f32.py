"""Loader of the oracle's exact-fp32 indexer score (oracle/score_f32.c).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  The C file is compiled
with the host's gcc into oracle/_build/ on first use (or by build()), with
-ffp-contract=off so that the only fused operations are the explicit fmaf
calls of the canonical order.
"""
from __future__ import annotations

import ctypes as C
import os
import shutil
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "score_f32.c")
LIB = os.path.join(_HERE, "_build", "libspin_oracle.so")
_lib = None


def build() -> str:
    """Compile score_f32.c (always)."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no host C compiler to build the oracle's fp32 scorer")
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    tmp = LIB + ".tmp"
    subprocess.run([cc, "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-o", tmp, SRC, "-lm"], check=True, capture_output=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        lib = C.CDLL(LIB)
        P = C.c_void_p
        lib.oracle_score_f32.argtypes = [P, P, P, C.c_int64, C.c_int, C.c_int, P]
        lib.oracle_score_f32.restype = None
        lib.oracle_fmaf.argtypes = [C.c_float, C.c_float, C.c_float]
        lib.oracle_fmaf.restype = C.c_float
        _lib = lib
    return _lib


def index_scores_f32(q, w, keys) -> np.ndarray:
    """z[i] = sum_h w_h ReLU(q_h . k_i) in the canonical fp32 order (score_f32.c).

    q: [n_h, d] fp32, w: [n_h] fp32, keys: [n, d] fp32 -> fp32 [n]."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    k = np.ascontiguousarray(keys, dtype=np.float32)
    n_h, d = q.shape
    assert w.shape == (n_h,) and (k.size == 0 or k.shape[1] == d)
    n = k.shape[0] if k.size else 0
    z = np.zeros(n, dtype=np.float32)
    if n:
        _load().oracle_score_f32(q.ctypes.data, w.ctypes.data, k.ctypes.data, n, n_h, d,
                                 z.ctypes.data)
    return z


def fmaf(a, b, c) -> np.float32:
    """The C library's fused multiply-add on fp32 operands (one rounding)."""
    return np.float32(_load().oracle_fmaf(float(a), float(b), float(c)))
