"""GPU parity of the backward pass at full size, in the launch configuration
the benchmark times (forward: K rotated to f16, V tiles, RoPE fused into the
Q load; backward: q~ and k~ rotated to bf16, V rows, gradients of the raw
q, k in fp32).

The oracle computes, one by one: dq for 1024 seeded rows (edge rows on every
head plus uniform ones), and dk, dv for the keys whose rows it can afford
(the last 128 keys of every KV head under the causal mask; a 64-key block in
the middle of the sequence under the window).  Identities of the exact
gradient that hold at any size are checked on the whole output:
  sum_j dv_j = sum_i dO_i               (probability rows sum to 1)
  sum_j R(p_j) dk_j = 0                 (rows of dS sum to 0)
  sum_i <q_i, dq_i> = sum_j <k_j, dk_j> (both equal sum dS o S)
each per KV head, relative to the sum of the magnitudes of its terms.
"""
import time

import numpy as np
import pytest
import torch

import fixtures
import oracle
from fixtures import workloads as W
from tests import gpu_util as U
from tests.test_gpu_bwd import check_grads

pytestmark = pytest.mark.gpu

# of the sum of the terms' magnitudes: each term carries about three bf16
# roundings (relative standard deviation 2^-9/sqrt(3) each, ~2e-3 together),
# and a sum's error relative to its magnitude sum is at most that
IDENTITY_REL = 2e-3


@pytest.fixture(scope="module")
def lcx():
    import long_context_attention_rope_amd as m
    return m


def _run(lcx, w, q, k, v, dout):
    qd, kd, vd, gd = U.to_dev(q), U.to_dev(k), U.to_dev(v), U.to_dev(dout)
    cfg = lcx.rope_cfg(w.scheme, w.base, w.d, w.L_train, w.L_target, w.cur_len, w.alpha, w.beta)
    cos, sin = lcx.rope_tables(cfg, w.n, device=U.dev())
    _, kf = lcx.rope_apply_qk(None, kd, cos, sin)
    vt = lcx.pack_v(vd)
    o, lse = lcx.attn_fwd(qd, kf, vt, rope_q=True, cos=cos, sin=sin, rope=cfg, window=w.window,
                          n_sink=w.n_sink)
    del kf, vt
    qr, kr = lcx.rope_apply_qk(qd, kd, cos, sin, out_dtype=torch.bfloat16)
    del qd, kd
    dq, dk, dv = lcx.attn_bwd(qr, kr, vd, o, lse, gd, unrotate=True, cos=cos, sin=sin, rope=cfg,
                              window=w.window, n_sink=w.n_sink)
    torch.cuda.synchronize()
    return dq, dk, dv


def _key_sel(w):
    sel = np.zeros((w.B, w.Hkv, w.n), dtype=bool)
    if w.window < 0:
        sel[:, :, w.n - 128:] = True
    else:
        mid = (w.n // 2) // 64 * 64 + 5   # a ragged block, not tile aligned
        sel[:, :, mid:mid + 64] = True
    return sel


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w", [W.LLAMA70B_128K, W.SWA_SINK_64K], ids=lambda w: w.name)
def test_backward_full_size(lcx, w):
    t0 = time.time()
    q, k, v = U.inputs(w)
    dout = fixtures.normal_bf16(w.seed, fixtures.DO_ID, (w.B, w.Hq, w.n, w.d))
    U.log(f"{w.name}: inputs in {time.time() - t0:.1f}s")
    dq, dk, dv = _run(lcx, w, q, k, v, dout)
    U.log(f"{w.name}: GPU backward done")
    assert torch.isfinite(dq).all().item() and torch.isfinite(dk).all().item()
    assert torch.isfinite(dv).all().item()

    # sampled exact comparison
    bb, hh, rr = U.sample_rows(w, 1024, seed=w.seed + 7)
    row_sel = np.zeros((w.B, w.Hq, w.n), dtype=bool)
    row_sel[bb, hh, rr] = True
    key_sel = _key_sel(w)
    th, pf, lm = U.oracle_freqs(w)
    t1 = time.time()
    rq, rk, rv = oracle.attn_bwd(q, k, v, dout, th, pf, lm / np.sqrt(w.d), True, w.window, w.n_sink,
                                 row_sel=row_sel, key_sel=key_sel)
    U.log(f"{w.name}: oracle rows/keys in {time.time() - t1:.1f}s")
    kb, kh, kj = np.nonzero(key_sel)
    g_dq = dq[torch.from_numpy(bb.astype(np.int64)), torch.from_numpy(hh.astype(np.int64)),
              torch.from_numpy(rr)].cpu().numpy()
    ki = [torch.from_numpy(a.astype(np.int64)) for a in (kb, kh, kj)]
    g_dk = dk[ki[0], ki[1], ki[2]].cpu().numpy()
    g_dv = dv[ki[0], ki[1], ki[2]].cpu().numpy()
    check_grads((g_dq, g_dk, g_dv), (rq[bb, hh, rr], rk[kb, kh, kj], rv[kb, kh, kj]), w.name)

    # identities on the whole output, per KV head
    G = w.Hq // w.Hkv
    pos = np.arange(w.n)
    for b in range(w.B):
        for g in range(w.Hkv):
            heads = slice(g * G, (g + 1) * G)
            dvg = dv[b, g].double().cpu().numpy()
            dkg = dk[b, g].double().cpu().numpy()
            dqg = dq[b, heads].double().cpu().numpy()
            lhs = dvg.sum(axis=0)
            rhs = fixtures.bf16_to_f64(dout[b, heads]).sum(axis=(0, 1))
            e1 = np.abs(lhs - rhs).max() / np.abs(dvg).sum(axis=0).max()
            rot = oracle.rope_rotate(dkg, pos, th, pf)
            e2 = np.abs(rot.sum(axis=0)).max() / np.abs(rot).sum(axis=0).max()
            qdq = fixtures.bf16_to_f64(q[b, heads]) * dqg
            kdk = fixtures.bf16_to_f64(k[b, g]) * dkg
            e3 = abs(qdq.sum() - kdk.sum()) / (np.abs(qdq).sum() + np.abs(kdk).sum())
            del qdq, kdk, dqg
            U.log(f"{w.name} kv head {g}: sum dv {e1:.2e}, sum R dk {e2:.2e}, <q,dq> vs <k,dk> {e3:.2e}")
            assert e1 <= IDENTITY_REL and e2 <= IDENTITY_REL and e3 <= IDENTITY_REL, (g, e1, e2, e3)
