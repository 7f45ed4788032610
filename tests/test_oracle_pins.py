"""Pins for the fp64 oracle: closed forms, invariants, special cases, values
printed on the pages, and a full-matrix brute force computed by another route
(matrix exponential of the rotation generator, scipy softmax/logsumexp).

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, index or exponent, a transposed operand) fails at least one test.
"""
import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.special

import fixtures
import oracle
from fixtures import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALED = ["pi", "ntk", "ntk_parts", "yarn", "dynamic_ntk"]


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            out.setdefault("rows", []).append(parts)
            if len(parts) == 2:
                out[parts[0]] = float(parts[1])
    return out


def plain(d, base):
    return oracle.rope_freqs("plain", base, d)[0]


# ---------------------------------------------------------------- a1: frequencies

@pytest.mark.parametrize("d", [8, 64, 128])
@pytest.mark.parametrize("base", [10000.0, 500000.0])
def test_plain_ladder_is_geometric_from_1_towards_1_over_base(d, base):
    th = plain(d, base)
    assert th.shape == (d // 2,)
    assert th[0] == 1.0
    np.testing.assert_allclose(th[1:] / th[:-1], base ** (-2.0 / d), rtol=1e-13)
    # one more rung of the ladder lands exactly on 1/base
    np.testing.assert_allclose(th[-1] * base ** (-2.0 / d), 1.0 / base, rtol=1e-13)


@pytest.mark.parametrize("scheme", SCALED)
@pytest.mark.parametrize("d", [64, 128])
def test_s_equal_1_reduces_every_scheme_to_plain(scheme, d):
    base = 500000.0
    th, pf, lm = oracle.rope_freqs(scheme, base, d, 8192, 8192, cur_len=8192)
    assert np.array_equal(th, plain(d, base))
    assert pf == 1.0 and lm == 1.0


@pytest.mark.parametrize("d,base,L,s", [(64, 1e4, 128, 4), (128, 5e5, 8192, 128), (128, 5e5, 8192, 3)])
def test_ntk_aware_keeps_top_frequency_and_interpolates_bottom_by_s(d, base, L, s):
    th, pf, lm = oracle.rope_freqs("ntk", base, d, L, L * s)
    p = plain(d, base)
    assert pf == 1.0 and lm == 1.0
    assert th[0] == 1.0
    np.testing.assert_allclose(th[-1], p[-1] / s, rtol=1e-13)
    ratio = th / p
    assert np.all(np.diff(ratio) < 0) and np.all(ratio <= 1.0) and np.all(ratio >= 1.0 / s * (1 - 1e-13))


def test_ntk_tiny_config_base():
    # base' = 10000 * 4^(64/62): the lowest pair is plain/4 and the whole ladder
    # is the plain ladder of base'
    th, _, _ = oracle.rope_freqs("ntk", 10000.0, 64, 128, 512)
    b2 = th[1] ** (-64 / 2.0)
    np.testing.assert_allclose(b2, 10000.0 * 4.0 ** (64 / 62), rtol=1e-11)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,s", [(8192, 4), (4096, 16), (128, 4), (8192, 128)])
def test_ntk_by_parts_endpoints_and_monotone(d, L, s):
    base = 500000.0
    th, pf, lm = oracle.rope_freqs("ntk_parts", base, d, L, L * s, alpha=1.0, beta=32.0)
    p = plain(d, base)
    r = th / p
    lam = 2 * math.pi / p
    lo, hi = L / 32.0, L / 1.0
    assert np.all(r[lam < lo] == 1.0)            # short wavelengths untouched
    np.testing.assert_allclose(r[lam > hi], 1.0 / s, rtol=1e-14)  # long ones fully interpolated
    order = np.argsort(lam)
    assert np.all(np.diff(r[order]) <= 1e-15)    # never increases with wavelength
    assert np.all((r >= 1.0 / s * (1 - 1e-14)) & (r <= 1.0))
    assert pf == 1.0 and lm == 1.0


def test_ntk_by_parts_is_continuous():
    # a very fine ladder (d = 4096) samples the ramp densely: no jump at either threshold
    d, base, L, s = 4096, 500000.0, 8192, 8
    th, _, _ = oracle.rope_freqs("ntk_parts", base, d, L, L * s)
    r = th / plain(d, base)
    assert (r == 1.0).any() and (np.abs(r - 1 / s) < 1e-14).any()
    assert np.max(np.abs(np.diff(r))) < 0.03


def test_pair_factors_reduce_to_plain_pi_and_by_parts():
    # [CW §2.5]: one factor per rotation plane dividing that plane's frequency.
    d, base, L, s = 128, 500000.0, 8192, 16
    th_plain = plain(d, base)
    th, pf, lm = oracle.rope_freqs("pair_factors", base, d, factors=np.ones(d // 2))
    assert np.array_equal(th, th_plain) and pf == 1.0 and lm == 1.0
    # all factors s: the angles of PI (positions scaled by 1/s), up to rounding
    th_s, _, _ = oracle.rope_freqs("pair_factors", base, d, factors=np.full(d // 2, float(s)))
    _, pf_pi, _ = oracle.rope_freqs("pi", base, d, L, L * s)
    c1, s1 = oracle.rope_table(th_s, d, 1.0, 0, 4096)
    c2, s2 = oracle.rope_table(th_plain, d, pf_pi, 0, 4096)
    assert np.max(np.abs(c1 - c2)) < 1e-12 and np.max(np.abs(s1 - s2)) < 1e-12
    # the by-parts ramp written as per-plane factors gives NTK-by-parts back
    th_bp, _, _ = oracle.rope_freqs("ntk_parts", base, d, L, L * s)
    th_f, _, _ = oracle.rope_freqs("pair_factors", base, d, factors=th_plain / th_bp)
    np.testing.assert_allclose(th_f, th_bp, rtol=1e-15, atol=0)
    # a factor that is not finite and > 0, or the wrong count, is rejected
    for bad in (np.zeros(d // 2), np.full(d // 2, -2.0), np.full(d // 2, np.nan), np.ones(d // 2 - 1), None):
        with pytest.raises(ValueError):
            oracle.rope_freqs("pair_factors", base, d, factors=bad)


def test_yarn_is_by_parts_plus_temperature():
    th_y, pf, lm = oracle.rope_freqs("yarn", 500000.0, 128, 8192, 32768)
    th_p, _, _ = oracle.rope_freqs("ntk_parts", 500000.0, 128, 8192, 32768)
    assert np.array_equal(th_y, th_p) and pf == 1.0
    assert 0 < lm < 1
    # t(s) - 1 is logarithmic in s: t(s^2) - 1 = 2 (t(s) - 1)
    _, _, lm2 = oracle.rope_freqs("yarn", 500000.0, 128, 8192, 8192 * 16)
    np.testing.assert_allclose(1 / lm2 - 1, 2 * (1 / lm - 1), rtol=1e-13)


def test_yarn_temperature_golden():
    # the oracle's logit multiplier is 1/t at the page's t for every listed s
    # (pins the coefficient 0.1 and the natural log, which the log-linearity
    # check above leaves open), and the 8B workload's softmax scale
    g = _golden("yarn_temperature.txt")
    rows = [r for r in g["rows"] if len(r) == 3]
    assert len(rows) == 5
    for lt, lg, t in rows:
        th, pf, lm = oracle.rope_freqs("yarn", 500000.0, 128, int(lt), int(lg))
        assert 1.0 / lm == pytest.approx(float(t), rel=5e-16, abs=0), (lt, lg)
        assert pf == 1.0
    _, _, lm4 = oracle.rope_freqs("yarn", 500000.0, 128, 8192, 32768)
    assert abs(lm4 / np.sqrt(128.0) - g["sigma_d128_s4"]) < 5e-8


@pytest.mark.parametrize("d", [64, 128])
def test_dynamic_ntk(d):
    base, L = 500000.0, 8192
    for l in (1, 100, 4096, 8192):
        th, _, _ = oracle.rope_freqs("dynamic_ntk", base, d, L, 131072, cur_len=l)
        assert np.array_equal(th, plain(d, base))
    for l in (8193, 16384, 131072, 1048576):
        th, _, _ = oracle.rope_freqs("dynamic_ntk", base, d, L, 131072, cur_len=l)
        ref, _, _ = oracle.rope_freqs("ntk", base, d, L, l)
        np.testing.assert_allclose(th, ref, rtol=1e-14)
    # cur_len 0 means the target length
    th0, _, _ = oracle.rope_freqs("dynamic_ntk", base, d, L, 131072, cur_len=0)
    th1, _, _ = oracle.rope_freqs("dynamic_ntk", base, d, L, 131072, cur_len=131072)
    assert np.array_equal(th0, th1)


@pytest.mark.parametrize("fname", ["pi_4k_to_8k.txt", "pi_4k_to_128k.txt"])
def test_pi_golden(fname):
    g = _golden(fname)
    th, pf, lm = oracle.rope_freqs("pi", 10000.0, 128, int(g["L_train"]), int(g["L_target"]))
    assert pf == g["position_factor"]
    if "s" in g:
        assert 1.0 / pf == g["s"]
    assert np.array_equal(th, plain(128, 10000.0)) and lm == 1.0


def test_invalid_arguments_rejected():
    with pytest.raises(ValueError):
        oracle.rope_freqs("plain", 10000.0, 63)
    with pytest.raises(ValueError):
        oracle.rope_freqs("plain", 1.0, 64)
    with pytest.raises(ValueError):
        oracle.rope_freqs("ntk", 10000.0, 64, 8192, 4096)
    with pytest.raises(ValueError):
        oracle.rope_freqs("yarn", 10000.0, 64, 8192, 32768, alpha=32.0, beta=1.0)


def test_quadratic_cost_golden():
    # the FLOP counter used for the throughput metric scales as n^2 (page figures)
    for row in _golden("quadratic_cost.txt")["rows"]:
        a, b, ratio = int(row[0]), int(row[1]), float(row[2])
        wa = W.LLAMA8B_32K.with_(n=a)
        wb = W.LLAMA8B_32K.with_(n=b)
        assert (b * b) / (a * a) == ratio
        # causal pairs n(n+1)/2 track n^2 to within 1/n
        np.testing.assert_allclose(wb.flop() / wa.flop(), ratio, rtol=2.0 / a)


# ---------------------------------------------------------------- a2: tables

@pytest.mark.parametrize("scheme", ["plain", "ntk", "yarn", "dynamic_ntk", "pi"])
def test_table_properties(scheme):
    d = 64
    th, pf, _ = oracle.rope_freqs(scheme, 10000.0, d, 128, 512, cur_len=512)
    c, s = oracle.rope_table(th, d, pf, 0, 300)
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)          # position 0: identity
    np.testing.assert_allclose(c * c + s * s, 1.0, atol=1e-15)
    # angles are linear in position: row a+b = row a composed with row b
    a, b = 37, 211
    np.testing.assert_allclose(c[a + b], c[a] * c[b] - s[a] * s[b], atol=1e-13)
    np.testing.assert_allclose(s[a + b], s[a] * c[b] + c[a] * s[b], atol=1e-13)
    # pos0 offsets the same rows
    c2, s2 = oracle.rope_table(th, d, pf, 100, 50)
    np.testing.assert_array_equal(c2, c[100:150])
    np.testing.assert_array_equal(s2, s[100:150])


def test_pi_table_row_sk_equals_plain_row_k():
    d, s = 128, 8
    thp, pfp, _ = oracle.rope_freqs("pi", 500000.0, d, 8192, 8192 * s)
    th0, _, _ = oracle.rope_freqs("plain", 500000.0, d)
    cp, sp = oracle.rope_table(thp, d, pfp, 0, 8 * 100)
    c0, s0 = oracle.rope_table(th0, d, 1.0, 0, 100)
    np.testing.assert_array_equal(cp[::s], c0)
    np.testing.assert_array_equal(sp[::s], s0)


# ---------------------------------------------------------------- a3: rotation

def _rot_expm(x, pos, theta, pf):
    """Brute-force R(p) x with R(p) = expm(p * G), G = blockdiag(theta_i [[0,-1],[1,0]])."""
    d = x.shape[1]
    G = np.zeros((d, d))
    for i, t in enumerate(theta):
        G[2 * i + 1, 2 * i] = t
        G[2 * i, 2 * i + 1] = -t
    out = np.empty_like(x)
    for r in range(x.shape[0]):
        out[r] = scipy.linalg.expm(float(pos[r]) * pf * G) @ x[r]
    return out


@pytest.mark.parametrize("scheme", ["plain", "ntk", "pi", "yarn"])
def test_rotation_matches_matrix_exponential(scheme):
    d = 16
    th, pf, _ = oracle.rope_freqs(scheme, 10000.0, d, 128, 512)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((12, d))
    pos = np.array([0, 1, 2, 3, 7, 31, 64, 127, 128, 300, 511, 1000])
    np.testing.assert_allclose(oracle.rope_rotate(x, pos, th, pf), _rot_expm(x, pos, th, pf),
                               atol=1e-11)


def test_rotation_preserves_norm():
    d = 128
    th, pf, _ = oracle.rope_freqs("dynamic_ntk", 500000.0, d, 8192, 131072, cur_len=131072)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, d))
    pos = rng.integers(0, 1 << 20, size=64)
    y = oracle.rope_rotate(x, pos, th, pf)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    assert not np.allclose(y[1:], x[1:])   # it does rotate


@pytest.mark.parametrize("scheme", ["plain", "ntk", "pi", "ntk_parts"])
def test_unscaled_dot_depends_only_on_relative_position(scheme):
    d = 64
    th, pf, _ = oracle.rope_freqs(scheme, 10000.0, d, 128, 512)
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, d))
    k = rng.standard_normal((1, d))
    for m, n in [(5, 3), (100, 0), (77, 77), (3, 90)]:
        ref = (oracle.rope_rotate(q, [m], th, pf) @ oracle.rope_rotate(k, [n], th, pf).T)[0, 0]
        for delta in (1, 17, 1000, 123457):
            got = (oracle.rope_rotate(q, [m + delta], th, pf)
                   @ oracle.rope_rotate(k, [n + delta], th, pf).T)[0, 0]
            np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-9)
    # and it does depend on m - n
    a = (oracle.rope_rotate(q, [10], th, pf) @ oracle.rope_rotate(k, [0], th, pf).T)[0, 0]
    b = (oracle.rope_rotate(q, [0], th, pf) @ oracle.rope_rotate(k, [10], th, pf).T)[0, 0]
    assert abs(a - b) > 1e-6


# ---------------------------------------------------------------- a4-a8: attention

def _inputs(B, Hq, Hkv, n, d, seed):
    q = fixtures.normal_bf16(seed, fixtures.Q_ID, (B, Hq, n, d))
    k = fixtures.normal_bf16(seed, fixtures.K_ID, (B, Hkv, n, d))
    v = fixtures.normal_bf16(seed, fixtures.V_ID, (B, Hkv, n, d))
    return q, k, v


def _all_rows(q, n_kv_pos0=0):
    B, Hq, n, d = q.shape
    bb, hh, ii = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(n), indexing="ij")
    return (q.reshape(-1, d), ii.reshape(-1) + n_kv_pos0, hh.reshape(-1).astype(np.int32),
            bb.reshape(-1).astype(np.int32))


def _brute(q, k, v, theta, pf, sm, causal, window, n_sink, q_pos0=0, k_pos0=0):
    """Full-matrix attention by another route: expm rotations, masked -inf, scipy softmax."""
    B, Hq, n, d = q.shape
    Hkv, n_kv = k.shape[1], k.shape[2]
    qf, kf, vf = (fixtures.bf16_to_f64(t) for t in (q, k, v))
    G = Hq // Hkv
    kf = np.repeat(kf, G, axis=1)
    vf = np.repeat(vf, G, axis=1)
    qpos = np.arange(n) + q_pos0
    kpos = np.arange(n_kv) + k_pos0
    mask = np.ones((n, n_kv), dtype=bool)
    if causal:
        mask &= kpos[None, :] <= qpos[:, None]
    if window >= 0:
        mask &= (kpos[None, :] >= qpos[:, None] - window) | (kpos[None, :] < n_sink)
    O = np.zeros((B, Hq, n, d))
    L = np.full((B, Hq, n), -np.inf)
    for b in range(B):
        for h in range(Hq):
            qr = _rot_expm(qf[b, h], qpos, theta, pf) if theta is not None else qf[b, h]
            kr = _rot_expm(kf[b, h], kpos, theta, pf) if theta is not None else kf[b, h]
            S = sm * (qr @ kr.T)
            S = np.where(mask, S, -np.inf)
            ok = mask.any(axis=1)
            L[b, h, ok] = scipy.special.logsumexp(S[ok], axis=1)
            P = np.zeros_like(S)
            P[ok] = scipy.special.softmax(S[ok], axis=1)
            O[b, h] = P @ vf[b, h]
    return O, L


CASES = [
    # B, Hq, Hkv, n, d, scheme, causal, window, n_sink
    (1, 4, 1, 48, 8, "ntk", True, -1, 0),
    (1, 2, 2, 40, 8, "plain", True, -1, 0),
    (2, 8, 2, 33, 8, "yarn", True, -1, 0),
    (1, 4, 1, 64, 64, "ntk", True, -1, 0),
    (1, 4, 2, 50, 8, "pi", True, 7, 4),
    (1, 2, 1, 45, 8, "dynamic_ntk", True, 0, 3),
    (1, 2, 1, 30, 8, "ntk_parts", True, 12, 0),
    (1, 2, 2, 20, 8, "plain", False, -1, 0),
]


@pytest.mark.parametrize("B,Hq,Hkv,n,d,scheme,causal,window,n_sink", CASES)
def test_attention_matches_full_matrix_brute_force(B, Hq, Hkv, n, d, scheme, causal, window, n_sink):
    q, k, v = _inputs(B, Hq, Hkv, n, d, seed=11)
    th, pf, lm = oracle.rope_freqs(scheme, 10000.0, d, 16, 64, cur_len=64)
    sm = lm / math.sqrt(d)
    qr, qp, qh, qb = _all_rows(q)
    o, lse = oracle.attn_rows(qr, qp, qh, qb, k, v, Hq, th, pf, sm, causal, window, n_sink)
    O, L = _brute(q, k, v, th, pf, sm, causal, window, n_sink)
    np.testing.assert_allclose(o, O.reshape(-1, d), atol=1e-12, rtol=1e-11)
    np.testing.assert_allclose(lse, L.reshape(-1), atol=1e-12, rtol=1e-12)


def test_attention_brute_force_with_key_offset():
    # a chunk of keys at positions k_pos0.. and queries further on (ring share)
    B, Hq, Hkv, n, d = 1, 4, 2, 24, 8
    q, k, v = _inputs(B, Hq, Hkv, n, d, seed=12)
    th, pf, lm = oracle.rope_freqs("ntk", 10000.0, d, 16, 64)
    sm = 1 / math.sqrt(d)
    qr, qp, qh, qb = _all_rows(q, n_kv_pos0=40)
    o, lse = oracle.attn_rows(qr, qp, qh, qb, k, v, Hq, th, pf, sm, True, -1, 0, k_pos0=30)
    O, L = _brute(q, k, v, th, pf, sm, True, -1, 0, q_pos0=40, k_pos0=30)
    np.testing.assert_allclose(o, O.reshape(-1, d), atol=1e-12)
    np.testing.assert_allclose(lse, L.reshape(-1), atol=1e-12)


def _count(i, causal, w, ns, n_kv):
    js = np.arange(n_kv)
    m = np.ones(n_kv, bool)
    if causal:
        m &= js <= i
    if w >= 0:
        m &= (js >= i - w) | (js < ns)
    return m


@pytest.mark.parametrize("w,ns", [(-1, 0), (10, 0), (10, 4), (0, 4), (100, 4)])
def test_zero_keys_give_log_count_and_mean_of_kept_values(w, ns):
    B, Hq, Hkv, n, d = 1, 2, 1, 200, 16
    q, _, v = _inputs(B, Hq, Hkv, n, d, seed=13)
    k = np.zeros((B, Hkv, n, d), dtype=np.uint16)
    th, pf, _ = oracle.rope_freqs("ntk", 10000.0, d, 64, 256)
    qr, qp, qh, qb = _all_rows(q)
    o, lse = oracle.attn_rows(qr, qp, qh, qb, k, v, Hq, th, pf, 0.3, True, w, ns)
    vf = fixtures.bf16_to_f64(v)[0, 0]
    for r in range(len(qp)):
        keep = _count(qp[r], True, w, ns, n)
        cnt = int(keep.sum())
        # closed forms of the definition: count = min(i+1, w+1) + min(ns, max(0, i-w))
        i = qp[r]
        exp_cnt = i + 1 if w < 0 else min(i + 1, w + 1) + min(ns, max(0, i - w))
        assert cnt == exp_cnt
        assert lse[r] == pytest.approx(math.log(cnt), abs=1e-13)
        np.testing.assert_allclose(o[r], vf[keep].mean(axis=0), atol=1e-13)


def test_probability_rows_sum_to_one_and_respect_mask():
    B, Hq, Hkv, n, d = 1, 4, 2, 96, 32
    q, k, v = _inputs(B, Hq, Hkv, n, d, seed=14)
    th, pf, lm = oracle.rope_freqs("yarn", 500000.0, d, 32, 128)
    qr, qp, qh, qb = _all_rows(q)
    o, lse, p = oracle.attn_rows(qr, qp, qh, qb, k, v, Hq, th, pf, lm / math.sqrt(d), True, 20, 4,
                                 want_p=True)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    for r in range(len(qp)):
        keep = _count(qp[r], True, 20, 4, n)
        assert np.all(p[r, ~keep] == 0.0) and np.all(p[r, keep] > 0.0)
    # O is the probability-weighted value rows
    vf = fixtures.bf16_to_f64(v)
    for r in range(0, len(qp), 17):
        g = qh[r] * 2 // 4
        np.testing.assert_allclose(o[r], p[r] @ vf[0, g], atol=1e-12)


def test_two_key_rows_are_logistic_of_score_gap_with_temperature():
    # row 1 sees keys 0 and 1: P(key 1) = 1 / (1 + exp(-(S_1 - S_0))), S including 1/t
    d = 64
    th, pf, lm = oracle.rope_freqs("yarn", 500000.0, d, 8192, 32768)
    rng = np.random.default_rng(3)
    qf = rng.standard_normal(d)
    kf = rng.standard_normal((2, d))
    to_bits = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q = to_bits(qf)[None, :]
    k = to_bits(kf)[None, None]
    v = to_bits(np.eye(2, d))[None, None]
    qd, kd = fixtures.bf16_to_f64(q), fixtures.bf16_to_f64(k)[0, 0]
    qrot = oracle.rope_rotate(qd, [1], th, pf)[0]
    krot = oracle.rope_rotate(kd, [0, 1], th, pf)
    S = lm / math.sqrt(d) * (krot @ qrot)
    p1 = 1.0 / (1.0 + math.exp(-(S[1] - S[0])))
    o, lse, p = oracle.attn_rows(q, [1], [0], [0], k, v, 1, th, pf, lm / math.sqrt(d), want_p=True)
    assert p[0, 1] == pytest.approx(p1, abs=1e-14)
    assert o[0, 1] == pytest.approx(p1, abs=1e-14) and o[0, 0] == pytest.approx(1 - p1, abs=1e-14)
    assert lse[0] == pytest.approx(S[0] + math.log1p(math.exp(S[1] - S[0])), abs=1e-13)
    # the temperature matters: without it the probability differs
    assert abs(p1 - 1.0 / (1.0 + math.exp(-(S[1] - S[0]) / lm))) > 1e-6


def test_gqa_equals_mha_with_repeated_kv():
    B, Hq, Hkv, n, d = 1, 8, 2, 64, 16
    q, k, v = _inputs(B, Hq, Hkv, n, d, seed=15)
    th, pf, _ = oracle.rope_freqs("ntk", 10000.0, d, 16, 64)
    qr, qp, qh, qb = _all_rows(q)
    o1, l1 = oracle.attn_rows(qr, qp, qh, qb, k, v, Hq, th, pf)
    kr, vr = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    o2, l2 = oracle.attn_rows(qr, qp, qh, qb, kr, vr, Hq, th, pf)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_empty_rows():
    # keys all in the future of the queries: LSE -inf, O = 0
    B, Hq, Hkv, n, d = 1, 2, 1, 8, 8
    q, k, v = _inputs(B, Hq, Hkv, n, d, seed=16)
    qr, qp, qh, qb = _all_rows(q)
    o, lse = oracle.attn_rows(qr, qp, qh, qb, k, v, Hq, None, k_pos0=100)
    assert np.all(lse == -np.inf) and np.all(o == 0.0)


@pytest.mark.parametrize("chunk", [1, 7, 16, 50])
def test_chunked_merge_equals_one_shot_in_any_order(chunk):
    B, Hq, Hkv, n, d = 1, 4, 2, 100, 16
    q, k, v = _inputs(B, Hq, Hkv, n, d, seed=17)
    th, pf, _ = oracle.rope_freqs("ntk", 10000.0, d, 16, 128)
    qr, qp, qh, qb = _all_rows(q)
    o_ref, l_ref = oracle.attn_rows(qr, qp, qh, qb, k, v, Hq, th, pf, 0.25, True, 30, 4)
    parts_o, parts_l = [], []
    starts = list(range(0, n, chunk))
    rng = np.random.default_rng(chunk)
    rng.shuffle(starts)
    for s0 in starts:
        kc, vc = k[:, :, s0:s0 + chunk], v[:, :, s0:s0 + chunk]
        o, l = oracle.attn_rows(qr, qp, qh, qb, kc, vc, Hq, th, pf, 0.25, True, 30, 4, k_pos0=s0)
        parts_o.append(o)
        parts_l.append(l)
    o, l = oracle.merge(np.stack(parts_l), np.stack(parts_o))
    np.testing.assert_allclose(o, o_ref, atol=1e-13)
    np.testing.assert_allclose(l, l_ref, atol=1e-13)
    # merging is associative: pairwise tree equals flat
    o2, l2 = oracle.merge(np.stack(parts_l[:1]), np.stack(parts_o[:1]))
    for i in range(1, len(parts_l)):
        o2, l2 = oracle.merge(np.stack([l2, parts_l[i]]), np.stack([o2, parts_o[i]]))
    np.testing.assert_allclose(o2, o_ref, atol=1e-13)
    np.testing.assert_allclose(l2, l_ref, atol=1e-13)


def test_merge_with_empty_partial_is_identity():
    rng = np.random.default_rng(4)
    o = rng.standard_normal((5, 8))
    l = rng.standard_normal(5)
    om, lm = oracle.merge(np.stack([l, np.full(5, -np.inf)]), np.stack([o, np.zeros((5, 8))]))
    np.testing.assert_array_equal(lm, l)
    np.testing.assert_allclose(om, o, atol=0, rtol=1e-15)
    oe, le = oracle.merge(np.full((2, 5), -np.inf), np.zeros((2, 5, 8)))
    assert np.all(le == -np.inf) and np.all(oe == 0)
