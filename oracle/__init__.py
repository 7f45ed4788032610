"""ORACLE — test infrastructure only (fp64 CPU reference).

Thin ctypes wrapper around ``oracle.c``.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  It shares no code with the GPU library and the GPU library never
calls it.  ``oracle.c`` cites the page sections each function follows and the
pins that check it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

# the oracle's own scheme ids (independent of the GPU library's enum)
SCHEMES = {"none": 0, "plain": 1, "pi": 2, "ntk": 3, "ntk_parts": 4, "yarn": 5, "dynamic_ntk": 6,
           "pair_factors": 7}


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc: -O2, no fast-math, OpenMP over rows."""
    if force or not os.path.exists(_SO):
        src = os.path.join(_HERE, "oracle.c")
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                               "-fPIC", "-shared", "-std=c11", src, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_SO):
                build(force=False)
            lib = ctypes.CDLL(_SO)
            vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
            lib.oracle_set_num_threads.restype = None
            lib.oracle_rope_freqs.argtypes = [ctypes.c_int, f64, ctypes.c_int, i64, i64, i64, f64, f64,
                                              vp, vp, vp, vp]
            lib.oracle_rope_freqs.restype = ctypes.c_int
            lib.oracle_rope_table.argtypes = [vp, ctypes.c_int, f64, i64, i64, vp, vp]
            lib.oracle_rope_table.restype = None
            lib.oracle_rope_rotate.argtypes = [vp, i64, ctypes.c_int, vp, vp, f64, vp]
            lib.oracle_rope_rotate.restype = None
            lib.oracle_attn_rows.argtypes = [vp, vp, vp, vp, i64, vp, vp, i32, i32, i32, i64, i64, i32,
                                             vp, f64, i32, f64, i32, i64, i32, vp, vp, vp]
            lib.oracle_attn_rows.restype = ctypes.c_int
            lib.oracle_attn_bwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i64, i64, i32, i64, i64, vp,
                                            f64, i32, f64, i32, i64, i32, vp, vp, vp, vp, vp]
            lib.oracle_attn_bwd.restype = ctypes.c_int
            lib.oracle_merge.argtypes = [vp, vp, i64, i64, ctypes.c_int, vp, vp]
            lib.oracle_merge.restype = None
            _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the later oracle calls (timing only)."""
    _load().oracle_set_num_threads(int(n))


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def rope_freqs(scheme: str, base: float, d: int, L_train: int = 1, L_target: int = 1,
               cur_len: int = 0, alpha: float = 1.0, beta: float = 32.0, factors=None):
    """(theta'[d/2], position factor, logit multiplier) — step a1.  factors: the
    d/2 per-pair factors of the pair_factors scheme."""
    lib = _load()
    theta = np.zeros(d // 2, dtype=np.float64)
    pf = ctypes.c_double(0.0)
    lm = ctypes.c_double(0.0)
    fac = None if factors is None else _c(factors, np.float64)
    if fac is not None and fac.shape != (d // 2,):
        raise ValueError("factors must hold d/2 values")
    rc = lib.oracle_rope_freqs(SCHEMES[scheme], float(base), int(d), int(L_train), int(L_target),
                               int(cur_len), float(alpha), float(beta),
                               fac.ctypes.data if fac is not None else None, theta.ctypes.data,
                               ctypes.addressof(pf), ctypes.addressof(lm))
    if rc != 0:
        raise ValueError("oracle_rope_freqs: invalid arguments")
    return theta, pf.value, lm.value


def rope_table(theta, d: int, pos_factor: float, pos0: int, n_pos: int):
    """fp64 cos/sin tables [n_pos][d/2] — step a2."""
    lib = _load()
    th = _c(theta, np.float64)
    c = np.empty((n_pos, d // 2), dtype=np.float64)
    s = np.empty((n_pos, d // 2), dtype=np.float64)
    lib.oracle_rope_table(th.ctypes.data, d, float(pos_factor), int(pos0), int(n_pos),
                          c.ctypes.data, s.ctypes.data)
    return c, s


def rope_rotate(x, pos, theta, pos_factor: float):
    """Rotate fp64 rows x[n][d] at absolute positions pos[n] — step a3."""
    lib = _load()
    xx = _c(x, np.float64)
    n, d = xx.shape
    p = _c(pos, np.int64)
    th = _c(theta, np.float64)
    out = np.empty_like(xx)
    lib.oracle_rope_rotate(xx.ctypes.data, n, d, p.ctypes.data, th.ctypes.data, float(pos_factor),
                           out.ctypes.data)
    return out


def attn_rows(q_rows, q_pos, q_head, q_batch, k, v, Hq: int, theta=None, pos_factor: float = 1.0,
              sm_scale: float | None = None, causal: bool = True, window: int = -1, n_sink: int = 0,
              k_pos0: int = 0, want_p: bool = False):
    """Attention for selected query rows — steps a4-a8.

    q_rows [R][d] bf16 bits; k, v [B][Hkv][n_kv][d] bf16 bits.  theta None means
    no rotation.  Returns (O [R][d], LSE [R]) and P [R][n_kv] if want_p.
    """
    lib = _load()
    qr = _c(q_rows, np.uint16)
    R, d = qr.shape
    kk = _c(k, np.uint16)
    vv = _c(v, np.uint16)
    B, Hkv, n_kv, d2 = kk.shape
    assert d2 == d and vv.shape == kk.shape
    qp = _c(q_pos, np.int64)
    qh = _c(q_head, np.int32)
    qb = _c(q_batch, np.int32)
    rope = theta is not None
    th = _c(theta if rope else np.zeros(max(d // 2, 1)), np.float64)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    o = np.zeros((R, d), dtype=np.float64)
    lse = np.zeros(R, dtype=np.float64)
    p = np.zeros((R, n_kv), dtype=np.float64) if want_p else None
    rc = lib.oracle_attn_rows(qr.ctypes.data, qp.ctypes.data, qh.ctypes.data, qb.ctypes.data, R,
                              kk.ctypes.data, vv.ctypes.data, B, Hq, Hkv, n_kv, int(k_pos0), d,
                              th.ctypes.data, float(pos_factor), int(rope), float(sm_scale),
                              int(bool(causal)), int(window), int(n_sink), o.ctypes.data,
                              lse.ctypes.data, p.ctypes.data if want_p else None)
    if rc != 0:
        raise ValueError("oracle_attn_rows: invalid arguments")
    return (o, lse, p) if want_p else (o, lse)


def attn_bwd(q, k, v, dout, theta=None, pos_factor: float = 1.0, sm_scale: float | None = None,
             causal: bool = True, window: int = -1, n_sink: int = 0, q_pos0: int = 0,
             k_pos0: int = 0, row_sel=None, key_sel=None, want=("dq", "dk", "dv")):
    """Gradients (dq, dk, dv) of the attention rows for dL/dO = dout.

    q, dout [B][Hq][n_q][d] and k, v [B][Hkv][n_kv][d] are bf16 bits; theta None
    means no rotation (gradients with respect to the given q, k), else the
    gradients are with respect to the raw q, k.  row_sel [B][Hq][n_q] and
    key_sel [B][Hkv][n_kv] (bool) restrict which dq rows / dk, dv keys are
    computed; the rest are 0.  Outputs not in `want` are None.
    """
    lib = _load()
    qq = _c(q, np.uint16)
    kk = _c(k, np.uint16)
    vv = _c(v, np.uint16)
    go = _c(dout, np.uint16)
    B, Hq, n_q, d = qq.shape
    B2, Hkv, n_kv, d2 = kk.shape
    assert B2 == B and d2 == d and vv.shape == kk.shape and go.shape == qq.shape
    rope = theta is not None
    th = _c(theta if rope else np.zeros(max(d // 2, 1)), np.float64)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    rs = None if row_sel is None else _c(row_sel, np.uint8)
    ks = None if key_sel is None else _c(key_sel, np.uint8)
    if rs is not None:
        assert rs.shape == (B, Hq, n_q)
    if ks is not None:
        assert ks.shape == (B, Hkv, n_kv)
    dq = np.zeros(qq.shape, dtype=np.float64) if "dq" in want else None
    dk = np.zeros(kk.shape, dtype=np.float64) if "dk" in want else None
    dv = np.zeros(kk.shape, dtype=np.float64) if "dv" in want else None

    def ptr(a):
        return a.ctypes.data if a is not None else None

    rc = lib.oracle_attn_bwd(qq.ctypes.data, kk.ctypes.data, vv.ctypes.data, go.ctypes.data, B, Hq,
                             Hkv, n_q, n_kv, d, int(q_pos0), int(k_pos0), th.ctypes.data,
                             float(pos_factor), int(rope), float(sm_scale), int(bool(causal)),
                             int(window), int(n_sink), ptr(rs), ptr(ks), ptr(dq), ptr(dk), ptr(dv))
    if rc != 0:
        raise ValueError("oracle_attn_bwd: invalid arguments")
    return dq, dk, dv


def merge(lse_parts, o_parts):
    """Merge per-chunk (LSE [C][R], O [C][R][d]) — step a9."""
    lib = _load()
    L = _c(lse_parts, np.float64)
    O = _c(o_parts, np.float64)
    C, R = L.shape
    d = O.shape[2]
    lse = np.empty(R, dtype=np.float64)
    o = np.empty((R, d), dtype=np.float64)
    lib.oracle_merge(L.ctypes.data, O.ctypes.data, C, R, d, lse.ctypes.data, o.ctypes.data)
    return o, lse
