"""Python binding of liblcx (scaled-RoPE causal GQA attention for MI355X).

Argument marshalling only: torch tensors supply device memory, strides and the
current HIP stream; every step of the computation runs in the library's gfx950
kernels behind the C ABI of ``include/lcx.h``.  If ``liblcx.so`` has not been
built, importing this package fails; there is no other implementation to fall
back on.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblcx.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; "
                      f"g.build()' or python long_context_attention_rope_amd/_build.py)")
_lib = ctypes.CDLL(LIB_PATH)

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP = 0, 1, 2, 3
SCHEMES = {"none": 0, "plain": 1, "pi": 2, "ntk": 3, "ntk_parts": 4, "yarn": 5, "dynamic_ntk": 6,
           "pair_factors": 7}
BF16, F32, F16 = 0, 1, 2
_DT = {torch.bfloat16: BF16, torch.float32: F32, torch.float16: F16}

_i32, _i64, _f64, _f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_float, ctypes.c_void_p


class RopeCfg(ctypes.Structure):
    _fields_ = [("scheme", _i32), ("head_dim", _i32), ("base", _f64), ("L_train", _i64),
                ("L_target", _i64), ("cur_len", _i64), ("alpha", _f64), ("beta", _f64),
                ("factors", ctypes.POINTER(_f64))]


class AttnArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("k", _vp), ("v", _vp), ("q_dtype", _i32), ("k_dtype", _i32),
                ("B", _i32), ("Hq", _i32), ("Hkv", _i32), ("d", _i32),
                ("n_q", _i64), ("n_kv", _i64),
                ("q_strides", _i64 * 3), ("k_strides", _i64 * 3), ("v_strides", _i64 * 3),
                ("o_strides", _i64 * 3), ("lse_strides", _i64 * 2),
                ("q_pos0", _i64), ("k_pos0", _i64), ("rope_q", _i32), ("rope_k", _i32),
                ("cos_tab", _vp), ("sin_tab", _vp), ("tab_pos0", _i64), ("tab_len", _i64),
                ("rope", ctypes.POINTER(RopeCfg)), ("softmax_scale", _f32), ("causal", _i32),
                ("window", _i64), ("n_sink", _i32), ("o", _vp), ("o_dtype", _i32),
                ("lse", _vp), ("accumulate", _i32), ("v_tiled", _i32), ("precise_qk", _i32),
                ("sched", _vp)]


class BwdArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("k", _vp), ("v", _vp), ("o", _vp), ("lse", _vp), ("d_o", _vp),
                ("o_dtype", _i32), ("B", _i32), ("Hq", _i32), ("Hkv", _i32), ("d", _i32),
                ("n_q", _i64), ("n_kv", _i64),
                ("q_strides", _i64 * 3), ("k_strides", _i64 * 3), ("v_strides", _i64 * 3),
                ("o_strides", _i64 * 3), ("do_strides", _i64 * 3), ("lse_strides", _i64 * 2),
                ("q_pos0", _i64), ("k_pos0", _i64), ("rope", ctypes.POINTER(RopeCfg)),
                ("softmax_scale", _f32), ("causal", _i32), ("window", _i64), ("n_sink", _i32),
                ("unrotate", _i32), ("cos_tab", _vp), ("sin_tab", _vp), ("tab_pos0", _i64),
                ("tab_len", _i64), ("dq", _vp), ("dk", _vp), ("dv", _vp), ("grad_dtype", _i32),
                ("dq_strides", _i64 * 3), ("dk_strides", _i64 * 3), ("dv_strides", _i64 * 3),
                ("workspace", _vp), ("sched", _vp)]


_P3 = ctypes.POINTER(_i64)
_lib.lcx_status_string.argtypes = [ctypes.c_int]
_lib.lcx_status_string.restype = ctypes.c_char_p
_lib.lcx_last_error.argtypes = []
_lib.lcx_last_error.restype = ctypes.c_char_p
_lib.lcx_rope_freqs.argtypes = [ctypes.POINTER(RopeCfg), _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.lcx_rope_freqs.restype = ctypes.c_int
_lib.lcx_rope_apply_qk.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _i32,
                                   _P3, _P3, _P3, _P3, _i64, _vp, _vp, _i64, _i64, _vp]
_lib.lcx_rope_apply_qk.restype = ctypes.c_int
_lib.lcx_attn_fwd.argtypes = [ctypes.POINTER(AttnArgs), _vp]
_lib.lcx_attn_fwd.restype = ctypes.c_int
_lib.lcx_attn_merge.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i64, _i32, _P3, _P3, _P3, _P3,
                                _vp, _i32, _P3, _vp]
_lib.lcx_attn_merge.restype = ctypes.c_int
_lib.lcx_attn_fwd_chunked.argtypes = [ctypes.POINTER(AttnArgs), _i64, _vp, _vp, _vp, _vp, _vp]
_lib.lcx_attn_fwd_chunked.restype = ctypes.c_int
_lib.lcx_attn_pack_v.argtypes = [_vp, _vp, _i32, _i32, _i64, _i32, _P3, _vp]
_lib.lcx_attn_decode.argtypes = [ctypes.POINTER(AttnArgs), _i32, _vp, _vp, _vp]
_lib.lcx_attn_decode.restype = ctypes.c_int
_lib.lcx_attn_decode_noalloc.argtypes = [ctypes.POINTER(AttnArgs), _i32, _vp]
_lib.lcx_attn_decode_noalloc.restype = ctypes.c_int
DECODE_SCRATCH_BYTES = 16 << 20  # LCX_DECODE_SCRATCH_BYTES
_lib.lcx_attn_pack_v.restype = ctypes.c_int
_lib.lcx_attn_bwd.argtypes = [ctypes.POINTER(BwdArgs), _vp]
_lib.lcx_attn_bwd.restype = ctypes.c_int


class LcxError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        name = _lib.lcx_status_string(status).decode()
        super().__init__(f"{name}: {message}")


def _check(st: int):
    if st != OK:
        raise LcxError(st, _lib.lcx_last_error().decode())


def _stream(t: torch.Tensor | None):
    if t is None or not t.is_cuda:
        return None
    return _vp(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else _vp(t.data_ptr())


def _s3(t):
    return (_i64 * 3)(*t.stride()[:3]) if t is not None else None


def _s2(t):
    return (_i64 * 2)(*t.stride()[:2])


def rope_cfg(scheme: str, base: float, head_dim: int, L_train: int = 1, L_target: int = 1,
             cur_len: int = 0, alpha: float = 1.0, beta: float = 32.0, factors=None) -> RopeCfg:
    """factors: the d/2 per-pair factors of the pair_factors scheme (copied here and
    kept alive with the returned struct)."""
    cfg = RopeCfg(SCHEMES[scheme], head_dim, base, L_train, L_target, cur_len, alpha, beta, None)
    if factors is not None:
        arr = (_f64 * len(factors))(*[float(x) for x in factors])
        cfg._factors_keep = arr
        cfg.factors = ctypes.cast(arr, ctypes.POINTER(_f64))
    return cfg


def rope_freqs(cfg: RopeCfg, cos: torch.Tensor | None = None, sin: torch.Tensor | None = None,
               pos0: int = 0):
    """lcx_rope_freqs: returns (inv_freq list, pos_factor, logit_mult); fills cos/sin
    (fp32 [n_pos][d/2] device tensors) when given."""
    half = cfg.head_dim // 2
    inv = (_f64 * max(half, 1))()
    pf, lm = _f64(0), _f64(0)
    n_pos = cos.shape[0] if cos is not None else 0
    _check(_lib.lcx_rope_freqs(ctypes.byref(cfg), pos0, n_pos, ctypes.cast(inv, _vp),
                               _vp(ctypes.addressof(pf)), _vp(ctypes.addressof(lm)), _ptr(cos),
                               _ptr(sin), _stream(cos)))
    return list(inv)[:half], pf.value, lm.value


def rope_tables(cfg: RopeCfg, n_pos: int, pos0: int = 0, device="cuda"):
    """Allocate and fill the fp32 cos/sin tables [n_pos][d/2] for positions pos0.."""
    half = cfg.head_dim // 2
    cos = torch.empty((n_pos, half), dtype=torch.float32, device=device)
    sin = torch.empty((n_pos, half), dtype=torch.float32, device=device)
    rope_freqs(cfg, cos, sin, pos0)
    return cos, sin


def rope_apply_qk(q, k, cos, sin, *, pos0: int = 0, tab_pos0: int = 0, q_out=None, k_out=None,
                  out_dtype=torch.float16):
    """lcx_rope_apply_qk on [B, H, n, d] bf16 tensors (either may be None).
    Outputs are allocated with torch when not given; returns (q_out, k_out)."""
    if q is not None and q_out is None:
        q_out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if k is not None and k_out is None:
        k_out = torch.empty(k.shape, dtype=out_dtype, device=k.device)
    for x, y, name in ((q, q_out, "q"), (k, k_out, "k")):
        if x is not None:
            _rows4(x, name, dtypes=(torch.bfloat16,))
            _rows4(y, name + "_out", shape=x.shape, dtypes=(torch.bfloat16, torch.float16))
    ref = q if q is not None else k
    B, _, n, d = ref.shape
    Hq = q.shape[1] if q is not None else 0
    Hkv = k.shape[1] if k is not None else 0
    od = _DT[(q_out if q_out is not None else k_out).dtype]
    _check(_lib.lcx_rope_apply_qk(_ptr(q), _ptr(q_out), _ptr(k), _ptr(k_out), od, B, Hq, Hkv, n, d,
                                  _s3(q), _s3(q_out), _s3(k), _s3(k_out), pos0, _ptr(cos), _ptr(sin),
                                  tab_pos0, cos.shape[0], _stream(ref)))
    return q_out, k_out


def _rows4(t, name, shape=None, dtypes=None):
    """A [B, H, n, d] tensor whose rows are contiguous (the library takes element
    strides of the first three dimensions and assumes unit stride in the last)."""
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, H, n, d], got {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} dtype {t.dtype} not in {dtypes}")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError(f"{name} rows must be contiguous (stride(-1) == 1)")


def _workspace(t, name, shape):
    """Caller-owned fp32 scratch the C side addresses as a contiguous block."""
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} (contiguous: {t.is_contiguous()})")


SCHED_BYTES = 64  # LCX_SCHED_BYTES


def _sched(sched, device):
    """The sched buffer of lcx_attn_args: True -> a new LCX_SCHED_BYTES device buffer
    (dynamic work order), a tensor -> that buffer, False/None -> NULL (static order)."""
    if sched is None or sched is False:
        return None
    if sched is True:
        return torch.empty(SCHED_BYTES // 8, dtype=torch.int64, device=device)
    if not isinstance(sched, torch.Tensor) or sched.device != device or \
            sched.numel() * sched.element_size() < SCHED_BYTES or sched.data_ptr() % 8 or \
            not sched.is_contiguous():
        raise ValueError(f"sched must be a contiguous tensor of >= {SCHED_BYTES} bytes on {device}")
    return sched


def _attn_args(q, k, v, o, lse, *, rope_q, rope_k, cos, sin, tab_pos0, cfg, softmax_scale,
               window, n_sink, q_pos0, k_pos0, accumulate, causal=True, precise_qk=False,
               sched=None):
    _rows4(q, "q", dtypes=(torch.bfloat16, torch.float16))
    B, Hq, n_q, d = q.shape
    _rows4(k, "k", dtypes=(torch.bfloat16, torch.float16))
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"k {tuple(k.shape)} does not match q {tuple(q.shape)}")
    Hkv, n_kv = k.shape[1], k.shape[2]
    if v.dim() == 5:
        if (v.shape[0], v.shape[1], v.shape[3], v.shape[4]) != (B, Hkv, d, 64) or v.shape[2] * 64 < n_kv \
                or v.stride(4) != 1 or v.stride(3) != 64 or v.stride(2) != 64 * d:
            raise ValueError(f"V tiles must be [B, Hkv, >= ceil(n_kv/64), d, 64] with contiguous tiles, "
                             f"got {tuple(v.shape)}")
    else:
        _rows4(v, "v", shape=(B, Hkv, n_kv, d), dtypes=(torch.bfloat16,))
    _rows4(o, "o", shape=(B, Hq, n_q, d), dtypes=(torch.bfloat16, torch.float32))
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, n_q):
        raise ValueError(f"lse must be float32 [B, Hq, n_q], got {lse.dtype} {tuple(lse.shape)}")
    a = AttnArgs()
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.q_dtype, a.k_dtype = _DT[q.dtype], _DT[k.dtype]
    a.B, a.Hq, a.Hkv, a.d = B, Hq, Hkv, d
    a.n_q, a.n_kv = n_q, n_kv
    a.q_strides, a.k_strides = _s3(q), _s3(k)
    if v.dim() == 5:  # tile layout from pack_v: [B, Hkv, T, d, 64] f16
        if v.dtype != torch.float16:
            raise ValueError("V tiles (pack_v output) are float16")
        a.v_strides = (_i64 * 3)(v.stride(0), v.stride(1), 0)
        a.v_tiled = 1
    else:
        a.v_strides = _s3(v)
    a.o_strides = _s3(o)
    if lse.stride(2) != 1:
        raise ValueError("lse rows must be contiguous")
    a.lse_strides = _s2(lse)
    a.q_pos0, a.k_pos0 = q_pos0, k_pos0
    a.rope_q, a.rope_k = int(rope_q), int(rope_k)
    a.cos_tab = cos.data_ptr() if cos is not None else None
    a.sin_tab = sin.data_ptr() if sin is not None else None
    a.tab_pos0 = tab_pos0
    a.tab_len = cos.shape[0] if cos is not None else 0
    a.rope = ctypes.pointer(cfg) if cfg is not None else None
    a.softmax_scale = softmax_scale
    a.causal = int(causal)
    a.window, a.n_sink = window, n_sink
    a.o, a.o_dtype = o.data_ptr(), _DT[o.dtype]
    a.lse = lse.data_ptr()
    a.accumulate = int(accumulate)
    a.precise_qk = int(precise_qk)
    a.sched = sched.data_ptr() if sched is not None else None
    return a


def pack_v(v, out=None):
    """lcx_attn_pack_v: v [B,Hkv,n,d] bf16 -> tile layout [B,Hkv,ceil(n/64),d,64] float16
    (V converted to f16), accepted by attn_fwd / attn_fwd_chunked / attn_decode in place of v."""
    _rows4(v, "v", dtypes=(torch.bfloat16,))
    B, Hkv, n, d = v.shape
    T = (n + 63) // 64
    if out is None:
        out = torch.empty((B, Hkv, T, d, 64), dtype=torch.float16, device=v.device)
    if tuple(out.shape) != (B, Hkv, T, d, 64) or not out.is_contiguous() or out.dtype != torch.float16:
        raise ValueError("out must be a contiguous float16 [B, Hkv, T, d, 64] tensor")
    _check(_lib.lcx_attn_pack_v(_ptr(v), _ptr(out), B, Hkv, n, d, _s3(v), _stream(v)))
    return out


def attn_fwd(q, k, v, o=None, lse=None, *, rope_q=False, rope_k=False, cos=None, sin=None,
             tab_pos0=0, rope=None, softmax_scale=0.0, window=-1, n_sink=0, q_pos0=0, k_pos0=0,
             accumulate=False, out_dtype=torch.bfloat16, causal=True, precise_qk=False, sched=True):
    """lcx_attn_fwd.  q [B,Hq,n_q,d], k [B,Hkv,n_kv,d], v [B,Hkv,n_kv,d] or its pack_v
    tile layout.  precise_qk (with rope_k): QK^T from f16 high/low parts of the rotated
    operands.  sched: True (a new queue buffer per call), a buffer of SCHED_BYTES, or
    False for the static work order.  Returns (o, lse)."""
    B, Hq, n_q, d = q.shape
    if o is None:
        o = torch.empty((B, Hq, n_q, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, n_q), dtype=torch.float32, device=q.device)
    a = _attn_args(q, k, v, o, lse, rope_q=rope_q, rope_k=rope_k, cos=cos, sin=sin,
                   tab_pos0=tab_pos0, cfg=rope, softmax_scale=softmax_scale, window=window,
                   n_sink=n_sink, q_pos0=q_pos0, k_pos0=k_pos0, accumulate=accumulate,
                   causal=causal, precise_qk=precise_qk, sched=_sched(sched, q.device))
    _check(_lib.lcx_attn_fwd(ctypes.byref(a), _stream(q)))
    return o, lse


def decode_splits(B: int, Hkv: int, n_kv: int, d: int) -> int:
    """Default split-KV factor of attn_decode: 256 workgroups (512 for d = 64) over
    the B·Hkv heads, with at least 8 KV tiles of 64 keys per split."""
    wgs = 256 if d == 128 else 512
    return max(1, min(-(-wgs // (B * Hkv)), n_kv // 512))


def attn_decode(q, k, v, o=None, lse=None, *, n_splits=None, o_part=None, lse_part=None,
                rope_q=False, cos=None, sin=None, tab_pos0=0, rope=None, softmax_scale=0.0, window=-1,
                n_sink=0, q_pos0=0, k_pos0=0, out_dtype=torch.bfloat16):
    """lcx_attn_decode.  q [B,Hq,n_q<=8,d], k pre-rotated f16 [B,Hkv,n_kv,d], v rows or
    pack_v tiles.  n_splits defaults to one workgroup per CU (two for d = 64: each holds
    NST stages of K/V tiles in LDS) over B·Hkv, at least 8 KV tiles per split.  Returns
    (o, lse)."""
    B, Hq, n_q, d = q.shape
    Hkv, n_kv = k.shape[1], k.shape[2]
    if n_splits is None:
        n_splits = decode_splits(B, Hkv, n_kv, d)
    if o is None:
        o = torch.empty((B, Hq, n_q, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, n_q), dtype=torch.float32, device=q.device)
    if o_part is None:
        o_part = torch.empty((n_splits, B, Hq, n_q, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((n_splits, B, Hq, n_q), dtype=torch.float32, device=q.device)
    _workspace(o_part, "o_part", (n_splits, B, Hq, n_q, d))
    _workspace(lse_part, "lse_part", (n_splits, B, Hq, n_q))
    a = _attn_args(q, k, v, o, lse, rope_q=rope_q, rope_k=False, cos=cos, sin=sin,
                   tab_pos0=tab_pos0, cfg=rope, softmax_scale=softmax_scale, window=window,
                   n_sink=n_sink, q_pos0=q_pos0, k_pos0=k_pos0, accumulate=False)
    _check(_lib.lcx_attn_decode(ctypes.byref(a), n_splits, _ptr(o_part), _ptr(lse_part), _stream(q)))
    return o, lse


def attn_decode_noalloc(q, k, v, o, lse, *, n_splits=None, rope_q=False, cos=None, sin=None, tab_pos0=0,
                        rope=None, softmax_scale=0.0, window=-1, n_sink=0, q_pos0=0, k_pos0=0):
    """lcx_attn_decode_noalloc: attn_decode with the split partials in the library's
    static device scratch (no workspace).  o [B,Hq,n_q,d] and lse [B,Hq,n_q] are the
    caller's outputs; nothing is allocated.  Calls that overlap on one device race."""
    B, Hq, n_q, d = q.shape
    Hkv, n_kv = k.shape[1], k.shape[2]
    if n_splits is None:
        n_splits = decode_splits(B, Hkv, n_kv, d)
    a = _attn_args(q, k, v, o, lse, rope_q=rope_q, rope_k=False, cos=cos, sin=sin,
                   tab_pos0=tab_pos0, cfg=rope, softmax_scale=softmax_scale, window=window,
                   n_sink=n_sink, q_pos0=q_pos0, k_pos0=k_pos0, accumulate=False)
    _check(_lib.lcx_attn_decode_noalloc(ctypes.byref(a), n_splits, _stream(q)))
    return o, lse


def attn_fwd_chunked(q, k, v, chunk: int, o_acc, lse_acc, o=None, lse=None, *, o_part=None,
                     lse_part=None, rope_q=False, rope_k=False, cos=None, sin=None, tab_pos0=0,
                     rope=None, softmax_scale=0.0, window=-1, n_sink=0, q_pos0=0, k_pos0=0,
                     out_dtype=torch.bfloat16, sched=True):
    """lcx_attn_fwd_chunked.  o_acc fp32 [B,Hq,n_q,d] / lse_acc fp32 [B,Hq,n_q] workspace;
    o_part/lse_part (same shapes) select the separate merge pass; sched as in attn_fwd.
    Returns (o, lse)."""
    B, Hq, n_q, d = q.shape
    _workspace(o_acc, "o_acc", (B, Hq, n_q, d))
    _workspace(lse_acc, "lse_acc", (B, Hq, n_q))
    if (o_part is None) != (lse_part is None):
        raise ValueError("o_part and lse_part go together")
    if o_part is not None:
        _workspace(o_part, "o_part", (B, Hq, n_q, d))
        _workspace(lse_part, "lse_part", (B, Hq, n_q))
    if o is None:
        o = torch.empty((B, Hq, n_q, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, n_q), dtype=torch.float32, device=q.device)
    a = _attn_args(q, k, v, o, lse, rope_q=rope_q, rope_k=rope_k, cos=cos, sin=sin,
                   tab_pos0=tab_pos0, cfg=rope, softmax_scale=softmax_scale, window=window,
                   n_sink=n_sink, q_pos0=q_pos0, k_pos0=k_pos0, accumulate=False,
                   sched=_sched(sched, q.device))
    _check(_lib.lcx_attn_fwd_chunked(ctypes.byref(a), chunk, _ptr(o_acc), _ptr(lse_acc),
                                     _ptr(o_part), _ptr(lse_part), _stream(q)))
    return o, lse


def attn_merge(o_acc, lse_acc, o_part, lse_part, o_final=None):
    """lcx_attn_merge over [B,H,rows,d] fp32 tensors (in place into o_acc/lse_acc)."""
    _rows4(o_acc, "o_acc", dtypes=(torch.float32,))
    B, H, rows, d = o_acc.shape
    _rows4(o_part, "o_part", shape=(B, H, rows, d), dtypes=(torch.float32,))
    if o_final is not None:
        _rows4(o_final, "o_final", shape=(B, H, rows, d), dtypes=(torch.bfloat16, torch.float32))
    for t, name in ((lse_acc, "lse_acc"), (lse_part, "lse_part")):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, H, rows):
            raise ValueError(f"{name} must be float32 [B, H, rows], got {t.dtype} {tuple(t.shape)}")
    if lse_acc.stride(2) != 1 or lse_part.stride(2) != 1:
        raise ValueError("lse rows must be contiguous")
    fdt = _DT[o_final.dtype] if o_final is not None else BF16
    _check(_lib.lcx_attn_merge(_ptr(o_acc), _ptr(lse_acc), _ptr(o_part), _ptr(lse_part), B, H, rows, d,
                               _s3(o_acc), _s3(o_part), _s2(lse_acc), _s2(lse_part), _ptr(o_final),
                               fdt, _s3(o_final) if o_final is not None else None, _stream(o_acc)))
    return o_acc, lse_acc


def attn_bwd(q, k, v, o, lse, dout, *, dq=None, dk=None, dv=None, workspace=None, unrotate=False,
             cos=None, sin=None, tab_pos0=0, rope=None, softmax_scale=0.0, window=-1, n_sink=0,
             q_pos0=0, k_pos0=0, grad_dtype=torch.float32, causal=True, sched=True):
    """lcx_attn_bwd.  q, k: the rotated bf16 q~ [B,Hq,n_q,d] and k~ [B,Hkv,n_kv,d] the
    forward used; v bf16 rows; o, lse: the forward's outputs; dout = dL/dO bf16.  With
    unrotate the gradients are those of the raw q, k (tables cos/sin required).
    Returns (dq, dk, dv) in grad_dtype; workspace (fp32 [B,Hq,n_q,2]) is allocated when
    not given; sched as in attn_fwd."""
    B, Hq, n_q, d = q.shape
    Hkv, n_kv = k.shape[1], k.shape[2]
    dev = q.device
    if dq is None:
        dq = torch.empty((B, Hq, n_q, d), dtype=grad_dtype, device=dev)
    if dk is None:
        dk = torch.empty((B, Hkv, n_kv, d), dtype=grad_dtype, device=dev)
    if dv is None:
        dv = torch.empty((B, Hkv, n_kv, d), dtype=grad_dtype, device=dev)
    if workspace is None:
        workspace = torch.empty((B, Hq, n_q, 2), dtype=torch.float32, device=dev)
    _workspace(workspace, "workspace", (B, Hq, n_q, 2))
    if not (dq.dtype == dk.dtype == dv.dtype):
        raise ValueError("dq, dk, dv must share one dtype")
    _rows4(q, "q", dtypes=(torch.bfloat16,))
    _rows4(k, "k", shape=(B, Hkv, n_kv, d), dtypes=(torch.bfloat16,))
    _rows4(v, "v", shape=(B, Hkv, n_kv, d), dtypes=(torch.bfloat16,))
    _rows4(o, "o", shape=(B, Hq, n_q, d), dtypes=(torch.bfloat16, torch.float32))
    _rows4(dout, "dout", shape=(B, Hq, n_q, d), dtypes=(torch.bfloat16,))
    _rows4(dq, "dq", shape=(B, Hq, n_q, d), dtypes=(torch.bfloat16, torch.float32))
    _rows4(dk, "dk", shape=(B, Hkv, n_kv, d))
    _rows4(dv, "dv", shape=(B, Hkv, n_kv, d))
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, n_q):
        raise ValueError(f"lse must be float32 [B, Hq, n_q], got {lse.dtype} {tuple(lse.shape)}")
    if lse.stride(2) != 1:
        raise ValueError("lse rows must be contiguous")
    a = BwdArgs()
    a.q, a.k, a.v, a.o, a.lse, a.d_o = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                        lse.data_ptr(), dout.data_ptr())
    a.o_dtype = _DT[o.dtype]
    a.B, a.Hq, a.Hkv, a.d = B, Hq, Hkv, d
    a.n_q, a.n_kv = n_q, n_kv
    a.q_strides, a.k_strides, a.v_strides = _s3(q), _s3(k), _s3(v)
    a.o_strides, a.do_strides, a.lse_strides = _s3(o), _s3(dout), _s2(lse)
    a.q_pos0, a.k_pos0 = q_pos0, k_pos0
    a.rope = ctypes.pointer(rope) if rope is not None else None
    a.softmax_scale = softmax_scale
    a.causal = int(causal)
    a.window, a.n_sink = window, n_sink
    a.unrotate = int(unrotate)
    a.cos_tab = cos.data_ptr() if cos is not None else None
    a.sin_tab = sin.data_ptr() if sin is not None else None
    a.tab_pos0 = tab_pos0
    a.tab_len = cos.shape[0] if cos is not None else 0
    a.dq, a.dk, a.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    a.grad_dtype = _DT[dq.dtype]
    a.dq_strides, a.dk_strides, a.dv_strides = _s3(dq), _s3(dk), _s3(dv)
    a.workspace = workspace.data_ptr()
    sched = _sched(sched, dev)
    a.sched = sched.data_ptr() if sched is not None else None
    _check(_lib.lcx_attn_bwd(ctypes.byref(a), _stream(q)))
    return dq, dk, dv
