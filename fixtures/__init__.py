"""Seeded synthetic inputs (bf16 N(0,1) from a counter-based generator).

This package is the one piece shared by the GPU path's tests/bench and the
oracle's tests.  It produces inputs only; it contains none of the RoPE or
attention arithmetic.  ``gen.c`` documents the generator.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libfixtures.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile gen.c into libfixtures.so with gcc (OpenMP)."""
    if force or not os.path.exists(_SO):
        src = os.path.join(_HERE, "gen.c")
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               src, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_SO):
                build(force=False)
            lib = ctypes.CDLL(_SO)
            u64, u32, i64 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64
            vp = ctypes.c_void_p
            lib.fx_fill_bf16.argtypes = [u64, u32, u64, u64, vp]
            lib.fx_fill_bf16.restype = None
            lib.fx_fill_rows_bf16.argtypes = [u64, u32, vp, i64, i64, vp]
            lib.fx_fill_rows_bf16.restype = None
            lib.fx_fill_f64.argtypes = [u64, u32, u64, u64, vp]
            lib.fx_fill_f64.restype = None
            _lib = lib
    return _lib


# tensor ids of the workload recipe (DO: the upstream gradient dL/dO of the backward pass)
Q_ID, K_ID, V_ID, DO_ID = 0, 1, 2, 3


def normal_bf16(seed: int, tensor_id: int, shape, offset: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0,1) samples, flat index order = C order of ``shape``."""
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16)
    if n:
        lib.fx_fill_bf16(seed, tensor_id, offset, n, out.ctypes.data)
    return out.reshape(shape)


def rows_bf16(seed: int, tensor_id: int, row_idx, row_len: int) -> np.ndarray:
    """Rows ``row_idx`` (flat row numbers of a [..., row_len] tensor) as uint16 [len, row_len]."""
    lib = _load()
    idx = np.ascontiguousarray(np.asarray(row_idx, dtype=np.int64))
    out = np.empty((idx.size, row_len), dtype=np.uint16)
    if idx.size:
        lib.fx_fill_rows_bf16(seed, tensor_id, idx.ctypes.data, idx.size, row_len, out.ctypes.data)
    return out


def normal_f64(seed: int, tensor_id: int, count: int, offset: int = 0) -> np.ndarray:
    """The fp64 samples before bf16 rounding (distribution checks only)."""
    lib = _load()
    out = np.empty(count, dtype=np.float64)
    if count:
        lib.fx_fill_f64(seed, tensor_id, offset, count, out.ctypes.data)
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
