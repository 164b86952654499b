"""CPU oracle for Prof-K exact top-k: TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The product (sampling_threshold_filtering_amd) never
imports it, and it imports nothing from the product.

Contents:
  topk / topk_batched / count_at_or_before  plain C (topk_oracle.c) via ctypes
  method_ref                                 sample set, threshold, count, rank simulator
  solver_ref                                 scipy reference of the parameter choice
  philox                                     Philox4x32-10 from its published definition
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import method_ref, philox, solver_ref  # noqa: F401
from .build import LIB, build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=True)
        lib = ctypes.CDLL(LIB)
        i64 = ctypes.c_int64
        fp = ctypes.c_void_p
        lib.oracle_topk.argtypes = [fp, i64, i64, ctypes.c_int, fp, fp]
        lib.oracle_topk.restype = ctypes.c_int
        lib.oracle_topk_batched.argtypes = [fp, i64, i64, i64, i64, ctypes.c_int, fp, fp]
        lib.oracle_topk_batched.restype = ctypes.c_int
        lib.oracle_count_at_or_before.argtypes = [fp, i64, ctypes.c_float, i64]
        lib.oracle_count_at_or_before.restype = i64
        _lib = lib
    return _lib


def topk(x: np.ndarray, k: int, nthreads: int = 1):
    """Exact top-k of a 1-D float32 array: (values float32[k], indices int64[k]),
    ordered by value descending, ties by lower index, NaN above everything."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 1:
        raise ValueError("1-D input expected")
    vals = np.empty(k, dtype=np.float32)
    idx = np.empty(k, dtype=np.int64)
    rc = _load().oracle_topk(x.ctypes.data, x.size, k, nthreads, vals.ctypes.data, idx.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_topk failed (bad arguments?)")
    return vals, idx


def topk_batched(x: np.ndarray, k: int, nthreads: int = 1):
    """Row-wise exact top-k of a 2-D float32 array: (values [B,k], column indices [B,k])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("2-D input expected")
    B, N = x.shape
    vals = np.empty((B, k), dtype=np.float32)
    idx = np.empty((B, k), dtype=np.int64)
    rc = _load().oracle_topk_batched(x.ctypes.data, B, N, N, k, nthreads, vals.ctypes.data,
                                     idx.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_topk_batched failed")
    return vals, idx


def count_at_or_before(x: np.ndarray, tau_val, tau_idx: int) -> int:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return int(_load().oracle_count_at_or_before(x.ctypes.data, x.size, ctypes.c_float(float(tau_val)),
                                                 int(tau_idx)))
