"""Pins for the oracle's backward pass (the gradient of the attention rows).

The pages never write the backward pass out; the oracle takes the exact
gradient of the forward definition.  It is pinned here against things other
than itself:
  * central differences of the (already pinned) forward oracle, Richardson-
    extrapolated, on inputs whose perturbed values are exact bf16 numbers:
    every element of dq, dk, dv, with RoPE (so the inverse rotation is
    checked), GQA, position offsets, window + sinks and empty rows;
  * exact identities of the softmax gradient at sizes where differences are
    too slow: sum_j dv_j = sum of dO over non-empty rows, sum_j R(p_j) dk_j = 0,
    sum_i <q_i, dq_i> = sum_j <k_j, dk_j>;
  * special cases: V = 0 gives dq = dk = 0; a row with one kept key passes its
    dO to that key's dv and nothing to dq; GQA equals MHA with repeated K/V
    whose per-head dk, dv are summed;
  * row/key selection returns the same entries as the full computation.
"""
import numpy as np
import pytest

import fixtures
import oracle

GRID = 64.0  # inputs are k/64 with |k| <= 96: x, x +- h, x +- 2h are all exact bf16


def _grid_bf16(rng, shape):
    x = rng.integers(-96, 97, size=shape).astype(np.float32) / np.float32(GRID)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _to_bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _rows(B, Hq, n_q, q_pos0):
    bb, hh, ii = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(n_q), indexing="ij")
    return (ii.reshape(-1) + q_pos0, hh.reshape(-1).astype(np.int32), bb.reshape(-1).astype(np.int32))


def _loss(q, k, v, dout, kw):
    """L = sum dO . O with O from the forward oracle (fp64)."""
    B, Hq, n_q, d = q.shape
    qp, qh, qb = _rows(B, Hq, n_q, kw["q_pos0"])
    o, _ = oracle.attn_rows(q.reshape(-1, d), qp, qh, qb, k, v, Hq, kw["theta"], kw["pf"],
                            sm_scale=kw["sm"], causal=kw["causal"], window=kw["window"],
                            n_sink=kw["n_sink"], k_pos0=kw["k_pos0"])
    return float(np.sum(fixtures.bf16_to_f64(dout).reshape(-1, d) * o))


def _fd_grad(x, which, q, k, v, dout, kw):
    """Richardson-extrapolated central difference of L for every element of x."""
    h = 1.0 / GRID
    g = np.zeros(x.shape)
    xf = fixtures.bf16_to_f64(x)
    args = {"q": q, "k": k, "v": v}
    for idx in np.ndindex(x.shape):
        vals = []
        for step in (h, -h, 2 * h, -2 * h):
            xp = x.copy()
            xp[idx] = _to_bits(xf[idx] + step)
            assert fixtures.bf16_to_f64(xp)[idx] == xf[idx] + step  # exact perturbation
            a = dict(args)
            a[which] = xp
            vals.append(_loss(a["q"], a["k"], a["v"], dout, kw))
        d1 = (vals[0] - vals[1]) / (2 * h)
        d2 = (vals[2] - vals[3]) / (4 * h)
        g[idx] = (4 * d1 - d2) / 3
    return g


FD_CASES = [
    # B, Hq, Hkv, n_q, n_kv, d, scheme, q_pos0, k_pos0, window, n_sink
    (1, 4, 2, 6, 11, 8, "yarn", 5, 0, -1, 0),     # GQA, rows at 5..10 over keys 0..10, temperature
    (1, 2, 1, 10, 10, 8, "pi", 0, 0, 3, 2),       # window + sinks
    (1, 2, 2, 5, 7, 8, "ntk", 0, 3, -1, 0),       # rows 0..2 see no key (empty rows)
    (2, 2, 1, 4, 6, 4, None, 2, 0, -1, 0),        # no rotation, two batches
]


@pytest.mark.parametrize("B,Hq,Hkv,n_q,n_kv,d,scheme,q_pos0,k_pos0,window,n_sink", FD_CASES)
def test_backward_equals_finite_differences_of_forward(B, Hq, Hkv, n_q, n_kv, d, scheme, q_pos0,
                                                       k_pos0, window, n_sink):
    rng = np.random.default_rng(1000 + n_q * 31 + n_kv)
    q = _grid_bf16(rng, (B, Hq, n_q, d))
    k = _grid_bf16(rng, (B, Hkv, n_kv, d))
    v = _grid_bf16(rng, (B, Hkv, n_kv, d))
    dout = _grid_bf16(rng, (B, Hq, n_q, d))
    if scheme is None:
        th, pf, lm = None, 1.0, 1.0
    else:
        th, pf, lm = oracle.rope_freqs(scheme, 100.0, d, 4, 16)
    kw = dict(theta=th, pf=pf, sm=lm / np.sqrt(d), causal=True, window=window, n_sink=n_sink,
              q_pos0=q_pos0, k_pos0=k_pos0)
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, th, pf, kw["sm"], True, window, n_sink, q_pos0,
                                 k_pos0)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = _fd_grad(x, name, q, k, v, dout, kw)
        err = np.max(np.abs(fd - g))
        assert err <= 1e-7 * (1.0 + np.max(np.abs(g))), (name, err)
        assert np.max(np.abs(g)) > 1e-3  # a non-trivial gradient


def _normal_case(B, Hq, Hkv, n_q, n_kv, d, seed):
    q = fixtures.normal_bf16(seed, fixtures.Q_ID, (B, Hq, n_q, d))
    k = fixtures.normal_bf16(seed, fixtures.K_ID, (B, Hkv, n_kv, d))
    v = fixtures.normal_bf16(seed, fixtures.V_ID, (B, Hkv, n_kv, d))
    dout = fixtures.normal_bf16(seed, fixtures.DO_ID, (B, Hq, n_q, d))
    return q, k, v, dout


def _kept(qpos, kpos, window, n_sink):
    m = kpos[None, :] <= qpos[:, None]
    if window >= 0:
        m &= (kpos[None, :] >= qpos[:, None] - window) | (kpos[None, :] < n_sink)
    return m


@pytest.mark.parametrize("window,n_sink,q_pos0,k_pos0", [(-1, 0, 0, 0), (9, 3, 0, 0), (-1, 0, 40, 0),
                                                         (5, 0, 0, 17)])
def test_backward_identities(window, n_sink, q_pos0, k_pos0):
    B, Hq, Hkv, n_q, n_kv, d = 2, 6, 2, 70, 90, 16
    q, k, v, dout = _normal_case(B, Hq, Hkv, n_q, n_kv, d, seed=21)
    th, pf, lm = oracle.rope_freqs("yarn", 10000.0, d, 32, 128)
    sm = lm / np.sqrt(d)
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, th, pf, sm, True, window, n_sink, q_pos0, k_pos0)
    G = Hq // Hkv
    qpos = np.arange(n_q) + q_pos0
    kpos = np.arange(n_kv) + k_pos0
    nonempty = _kept(qpos, kpos, window, n_sink).any(axis=1)
    assert nonempty.any() and (not nonempty.all() or k_pos0 == 0)
    go = fixtures.bf16_to_f64(dout)
    qf, kf = fixtures.bf16_to_f64(q), fixtures.bf16_to_f64(k)
    for b in range(B):
        for g in range(Hkv):
            heads = slice(g * G, (g + 1) * G)
            # probabilities of a non-empty row sum to 1: sum_j dv_j = sum_i dO_i
            lhs = dv[b, g].sum(axis=0)
            rhs = go[b, heads][:, nonempty].sum(axis=(0, 1))
            np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-11 * (1 + np.abs(rhs).max()))
            # rows of dS sum to 0: the rotated-frame dk sum vanishes
            dkr = oracle.rope_rotate(dk[b, g], kpos, th, pf)
            assert np.max(np.abs(dkr.sum(axis=0))) < 1e-11 * (1 + np.abs(dk[b, g]).sum())
            assert np.abs(dk[b, g]).max() > 1e-3
            # sum_i <q_i, dq_i> = sum_ij dS_ij S_ij = sum_j <k_j, dk_j>
            a = np.sum(qf[b, heads] * dq[b, heads])
            c = np.sum(kf[b, g] * dk[b, g])
            assert abs(a - c) < 1e-11 * (1 + np.abs(qf[b, heads] * dq[b, heads]).sum())


def test_zero_values_give_zero_dq_dk():
    B, Hq, Hkv, n, d = 1, 4, 2, 40, 8
    q, k, v, dout = _normal_case(B, Hq, Hkv, n, n, d, seed=22)
    th, pf, _ = oracle.rope_freqs("ntk", 10000.0, d, 16, 64)
    dq, dk, dv = oracle.attn_bwd(q, k, np.zeros_like(v), dout, th, pf, None, True, 7, 2)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    assert np.abs(dv).max() > 0.1


def test_single_kept_key_rows():
    # window 0 and no sinks: each row keeps only itself, P = 1, dS = 0
    B, Hq, Hkv, n, d = 1, 2, 1, 12, 8
    q, k, v, dout = _normal_case(B, Hq, Hkv, n, n, d, seed=23)
    th, pf, _ = oracle.rope_freqs("plain", 10000.0, d)
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, th, pf, None, True, 0, 0)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    np.testing.assert_array_equal(dv[0, 0], fixtures.bf16_to_f64(dout)[0].sum(axis=0))


def test_gqa_gradients_equal_summed_mha_gradients():
    B, Hq, Hkv, n, d = 1, 6, 2, 30, 8
    G = Hq // Hkv
    q, k, v, dout = _normal_case(B, Hq, Hkv, n, n, d, seed=24)
    th, pf, _ = oracle.rope_freqs("pi", 10000.0, d, 16, 64)
    dq1, dk1, dv1 = oracle.attn_bwd(q, k, v, dout, th, pf, None, True, 11, 2)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    dq2, dk2, dv2 = oracle.attn_bwd(q, kr, vr, dout, th, pf, None, True, 11, 2)
    np.testing.assert_allclose(dq1, dq2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk1, dk2.reshape(B, Hkv, G, n, d).sum(axis=2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv1, dv2.reshape(B, Hkv, G, n, d).sum(axis=2), rtol=0, atol=1e-12)


def test_selected_rows_and_keys_match_full():
    B, Hq, Hkv, n_q, n_kv, d = 1, 4, 2, 50, 60, 8
    q, k, v, dout = _normal_case(B, Hq, Hkv, n_q, n_kv, d, seed=25)
    th, pf, _ = oracle.rope_freqs("ntk", 10000.0, d, 16, 64)
    full = oracle.attn_bwd(q, k, v, dout, th, pf, None, True, 13, 1, 10, 0)
    rng = np.random.default_rng(7)
    rs = rng.random((B, Hq, n_q)) < 0.2
    ks = rng.random((B, Hkv, n_kv)) < 0.2
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, th, pf, None, True, 13, 1, 10, 0, row_sel=rs, key_sel=ks)
    np.testing.assert_allclose(dq[rs], full[0][rs], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk[ks], full[1][ks], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv[ks], full[2][ks], rtol=0, atol=1e-13)
    assert np.all(dq[~rs] == 0) and np.all(dk[~ks] == 0) and np.all(dv[~ks] == 0)
