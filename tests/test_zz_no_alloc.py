"""GPU test of lcx_attn_decode_noalloc (decode with its split partials in the
library's static device scratch): two calls in a row, the second smaller,
each equal bit for bit to lcx_attn_decode with a caller workspace and the same
split count, and within the stated tolerances of the fp64 oracle."""
import numpy as np
import pytest
import torch

from fixtures import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lcx():
    import long_context_attention_rope_amd as m
    return m


def _case(lcx, w, n_q, n_splits, v_tiled):
    qp0 = w.n - n_q
    q, _, _ = U.inputs(w, n_q=n_q)
    _, k, v = U.inputs(w)
    cfg = lcx.rope_cfg(w.scheme, w.base, w.d, w.L_train, w.L_target, w.cur_len, w.alpha, w.beta)
    cos, sin = lcx.rope_tables(cfg, w.n, device=U.dev())
    _, kr = lcx.rope_apply_qk(None, U.to_dev(k), cos, sin)
    vv = lcx.pack_v(U.to_dev(v)) if v_tiled else U.to_dev(v)
    qd = U.to_dev(q)
    kw = dict(rope_q=True, cos=cos, sin=sin, rope=cfg, window=w.window, n_sink=w.n_sink, q_pos0=qp0)
    o_ref_gpu, l_ref_gpu = lcx.attn_decode(qd, kr, vv, n_splits=n_splits, out_dtype=torch.float32, **kw)
    o = torch.full_like(o_ref_gpu, float("nan"))
    lse = torch.full_like(l_ref_gpu, float("nan"))
    lcx.attn_decode_noalloc(qd, kr, vv, o, lse, n_splits=n_splits, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref_gpu) and torch.equal(lse, l_ref_gpu), "differs from lcx_attn_decode"
    bb = np.zeros(w.Hq * n_q, np.int32)
    hh = np.repeat(np.arange(w.Hq), n_q).astype(np.int32)
    rr = np.tile(np.arange(n_q), w.Hq)
    o_or, l_or = U.oracle_rows(w, q, k, v, bb, hh, rr, q_pos0=qp0)
    U.check(o.cpu().numpy().reshape(-1, w.d), lse.cpu().numpy().reshape(-1), o_or, l_or,
            f"decode_noalloc/{w.name}/n_q={n_q}/splits={n_splits}")


def test_decode_noalloc_matches_decode_on_two_calls(lcx):
    # first call: 40 splits x 16 heads x 8 rows x (128 + 1) x 4 B = 2.6 MB of partials
    w1 = W.Workload("noalloc_big", 1, 16, 2, 128, 5000, "dynamic_ntk", 500000.0, 256, 5000,
                    cur_len=5000, seed=71)
    U.log("decode_noalloc: call 1 (Hq 16, Hkv 2, d 128, 5000 keys, 8 rows, 40 splits)")
    _case(lcx, w1, 8, 40, True)
    # second call, smaller: fewer splits, heads, rows and keys, d = 64, window + sinks
    w2 = W.Workload("noalloc_small", 1, 8, 1, 64, 1500, "yarn", 500000.0, 256, 1024, window=400, n_sink=4,
                    seed=72)
    U.log("decode_noalloc: call 2 (Hq 8, Hkv 1, d 64, 1500 keys, 3 rows, 7 splits)")
    _case(lcx, w2, 3, 7, False)
