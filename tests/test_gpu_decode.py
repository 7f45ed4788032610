"""GPU parity of split-KV decode (lcx_attn_decode) against the fp64 oracle:
a few new query rows of every query head against a long pre-rotated K/V
cache, every row compared, for several split counts (including more splits
than tiles), masks, GQA ratios, both head dims, rows and tiled V."""
import numpy as np
import pytest
import torch

import fixtures
from fixtures import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lcx():
    import long_context_attention_rope_amd as m
    return m


CASES = [
    # name, Hq, Hkv, d, n_kv, n_q, q_pos0 (None: last rows), scheme, window, n_sink, v_tiled, splits
    ("d128_g8_q1", 8, 1, 128, 3000, 1, None, "ntk", -1, 0, False, (1, 5, 64)),
    ("d128_g8_q4_tiles", 16, 2, 128, 5000, 4, None, "dynamic_ntk", -1, 0, True, (3, 40)),
    ("d128_g8_q8_win_sink", 8, 1, 128, 2000, 8, None, "yarn", 500, 4, False, (7,)),
    ("d128_g8_q8_win_tiles", 8, 1, 128, 2000, 8, None, "yarn", 500, 4, True, (7,)),
    ("d64_g4_q3", 4, 1, 64, 1000, 3, None, "pi", -1, 0, False, (2, 16)),
    ("d128_rows_mid", 8, 2, 128, 2000, 8, 100, "plain", -1, 0, True, (4,)),
    ("d64_g2_q8_pairs", 4, 2, 64, 700, 8, None, "pair_factors", 64, 2, True, (5,)),
    ("d64_g8_q8_two_pairs", 8, 1, 64, 1300, 8, None, "ntk", -1, 0, True, (1, 9, 30)),
]


@pytest.mark.parametrize("name,Hq,Hkv,d,n_kv,n_q,q_pos0,scheme,window,n_sink,v_tiled,splits", CASES)
def test_decode_matches_oracle(lcx, name, Hq, Hkv, d, n_kv, n_q, q_pos0, scheme, window, n_sink,
                               v_tiled, splits):
    factors = (tuple(np.exp(np.random.default_rng(d).uniform(0.0, np.log(64.0), d // 2)))
               if scheme == "pair_factors" else None)
    w = W.Workload(name, 1, Hq, Hkv, d, n_kv, scheme, 500000.0, 256, 1024, cur_len=n_kv,
                   window=window, n_sink=n_sink, seed=300 + n_kv, factors=factors)
    qp0 = n_kv - n_q if q_pos0 is None else q_pos0
    q, _, _ = U.inputs(w, n_q=n_q)
    _, k, v = U.inputs(w)
    cfg = lcx.rope_cfg(w.scheme, w.base, w.d, w.L_train, w.L_target, w.cur_len, w.alpha, w.beta,
                       factors=w.factors)
    cos, sin = lcx.rope_tables(cfg, n_kv, device=U.dev())
    qd, kd, vd = U.to_dev(q), U.to_dev(k), U.to_dev(v)
    _, kr = lcx.rope_apply_qk(None, kd, cos, sin)
    vv = lcx.pack_v(vd) if v_tiled else vd
    bb = np.zeros(Hq * n_q, np.int32)
    hh = np.repeat(np.arange(Hq), n_q).astype(np.int32)
    rr = np.tile(np.arange(n_q), Hq)
    o_ref, l_ref = U.oracle_rows(w, q, k, v, bb, hh, rr, q_pos0=qp0)
    for ns in splits:
        o, lse = lcx.attn_decode(qd, kr, vv, n_splits=ns, rope_q=True, cos=cos, sin=sin, rope=cfg,
                                 window=window, n_sink=n_sink, q_pos0=qp0, out_dtype=torch.float32)
        torch.cuda.synchronize()
        U.check(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, l_ref,
                f"decode/{name}/splits={ns}")


def test_decode_rows_before_the_cache_are_empty(lcx):
    w = W.TINY.with_(seed=9)
    q, k, v = U.inputs(w, n_q=4)
    cfg = lcx.rope_cfg(w.scheme, w.base, w.d, w.L_train, w.L_target)
    cos, sin = lcx.rope_tables(cfg, 600 + w.n, device=U.dev())
    _, kr = lcx.rope_apply_qk(None, U.to_dev(k), cos, sin, pos0=600)
    o, lse = lcx.attn_decode(U.to_dev(q), kr, U.to_dev(v), n_splits=3, rope_q=True, cos=cos, sin=sin,
                             rope=cfg, q_pos0=10, k_pos0=600)
    torch.cuda.synchronize()
    assert torch.isneginf(lse).all().item() and (o.float() == 0).all().item()


def test_decode_two_batches(lcx):
    # batch index on the grid's third axis: two caches of different content,
    # 3 new rows each, every row compared
    w = W.Workload("decode_b2", 2, 8, 2, 128, 1500, "yarn", 500000.0, 256, 1024, cur_len=1500, seed=41)
    n_q = 3
    q, _, _ = U.inputs(w, n_q=n_q)
    _, k, v = U.inputs(w)
    cfg = lcx.rope_cfg(w.scheme, w.base, w.d, w.L_train, w.L_target, w.cur_len, w.alpha, w.beta)
    cos, sin = lcx.rope_tables(cfg, w.n, device=U.dev())
    qd, kd, vd = U.to_dev(q), U.to_dev(k), U.to_dev(v)
    _, kr = lcx.rope_apply_qk(None, kd, cos, sin)
    qp0 = w.n - n_q
    bb, hh, rr = np.meshgrid(np.arange(w.B), np.arange(w.Hq), np.arange(n_q), indexing="ij")
    bb, hh, rr = bb.reshape(-1).astype(np.int32), hh.reshape(-1).astype(np.int32), rr.reshape(-1)
    o_ref, l_ref = U.oracle_rows(w, q, k, v, bb, hh, rr, q_pos0=qp0)
    for vv, ns in ((lcx.pack_v(vd), 6), (vd, 11)):
        o, lse = lcx.attn_decode(qd, kr, vv, n_splits=ns, rope_q=True, cos=cos, sin=sin, rope=cfg,
                                 q_pos0=qp0, out_dtype=torch.float32)
        torch.cuda.synchronize()
        U.check(o.cpu().numpy().reshape(-1, w.d), lse.cpu().numpy().reshape(-1), o_ref, l_ref,
                f"decode/B=2/splits={ns}")


@pytest.mark.parametrize("n_q", [1, 8])
def test_decode_at_the_benchmarked_shape(lcx, n_q):
    # the configuration the decode benchmark times: the 70B-shaped GQA cache at
    # its full length ("上下文擴充套件" KV Cache 的視訊記憶體架構; 128K, "上下文窗口扩展技术"
    # §3), 131072 pre-rotated f16 keys per KV head, V tiles, the default 32
    # splits per KV head (64 tiles each), the new rows' tables built for their
    # positions only; every (head, new row) against the oracle
    w = W.LLAMA70B_128K
    U.log(f"decode at the benchmarked shape, n_q={n_q}")
    q = fixtures.normal_bf16(w.seed, fixtures.Q_ID, (w.B, w.Hq, n_q, w.d))
    _, k, v = U.inputs(w, n_q=1)
    cfg = lcx.rope_cfg(w.scheme, w.base, w.d, w.L_train, w.L_target, w.cur_len, w.alpha, w.beta)
    cos_all, sin_all = lcx.rope_tables(cfg, w.n, device=U.dev())
    _, kr = lcx.rope_apply_qk(None, U.to_dev(k), cos_all, sin_all)
    vt = lcx.pack_v(U.to_dev(v))
    del cos_all, sin_all
    qp0 = w.n - n_q
    cos, sin = lcx.rope_tables(cfg, n_q, pos0=qp0, device=U.dev())
    ns = lcx.decode_splits(w.B, w.Hkv, w.n, w.d)
    assert ns == 32
    o, lse = lcx.attn_decode(U.to_dev(q), kr, vt, n_splits=ns, rope_q=True, cos=cos, sin=sin,
                             tab_pos0=qp0, rope=cfg, q_pos0=qp0)
    torch.cuda.synchronize()
    bb = np.zeros(w.Hq * n_q, np.int32)
    hh = np.repeat(np.arange(w.Hq), n_q).astype(np.int32)
    rr = np.tile(np.arange(n_q), w.Hq)
    o_ref, l_ref = U.oracle_rows(w, q, k, v, bb, hh, rr, q_pos0=qp0)
    U.check(o.float().cpu().numpy().reshape(-1, w.d), lse.cpu().numpy().reshape(-1), o_ref, l_ref,
            f"decode/70b_128k/n_q={n_q}/splits={ns}")
