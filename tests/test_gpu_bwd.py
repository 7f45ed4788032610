"""GPU parity of the backward pass (lcx_attn_bwd) against the fp64 oracle's
gradient, every element of dq, dk, dv, at sizes the oracle finishes in
seconds: several tiles and ragged tails, all RoPE schemes, GQA ratios,
window/sink masks, position offsets with empty rows, bf16 outputs, the
gradients of q~/k~ (no unrotation), strided inputs and empty inputs.

The forward O and LSE come from the HIP forward (as in training); the oracle
recomputes everything from the raw inputs.  Tolerance: every gradient term is
a product of factors rounded to bf16 once each (q~ or k~, P or dS, O inside
D: about three roundings of relative standard deviation 2^-9/sqrt(3) each),
so a tensor's error is about sqrt(3)·1.1e-3 ≈ 2e-3 of its Frobenius norm
with fp32 accumulation; the bar is five times that: per tensor,
||g - r||_F <= 1e-2 ||r||_F and max |g - r| <= 2e-2 max |r|.
"""
import numpy as np
import pytest
import torch

import fixtures
import oracle
from fixtures import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

REL_FRO = 1e-2
REL_MAX = 2e-2


@pytest.fixture(scope="module")
def lcx():
    import long_context_attention_rope_amd as m
    return m


def _cfg(lcx, w):
    return lcx.rope_cfg(w.scheme, w.base, w.d, w.L_train, w.L_target, w.cur_len, w.alpha, w.beta,
                        factors=w.factors)


def _dout(w, n_q):
    return fixtures.normal_bf16(w.seed, fixtures.DO_ID, (w.B, w.Hq, n_q, w.d))


def gpu_grads(lcx, w, q, k, v, dout, *, q_pos0=0, k_pos0=0, unrotate=True, grad_dtype=torch.float32,
              strided=False):
    """HIP forward (O bf16, LSE), then the rotated bf16 q~, k~ and the backward."""
    qd, kd, vd, gd = U.to_dev(q), U.to_dev(k), U.to_dev(v), U.to_dev(dout)
    cfg = _cfg(lcx, w)
    n_tab = max(q_pos0 + q.shape[2], k_pos0 + k.shape[2], 1)
    cos, sin = lcx.rope_tables(cfg, n_tab, device=U.dev())
    _, kf = lcx.rope_apply_qk(None, kd, cos, sin, pos0=k_pos0, out_dtype=torch.float16)
    o, lse = lcx.attn_fwd(qd, kf, vd, rope_q=True, cos=cos, sin=sin, rope=cfg, window=w.window,
                          n_sink=w.n_sink, q_pos0=q_pos0, k_pos0=k_pos0)
    qr, _ = lcx.rope_apply_qk(qd, None, cos, sin, pos0=q_pos0, out_dtype=torch.bfloat16)
    _, kr = lcx.rope_apply_qk(None, kd, cos, sin, pos0=k_pos0, out_dtype=torch.bfloat16)
    if strided:
        # every input a view into a wider buffer (row strides of 3d elements)
        def widen(t):
            big = torch.zeros(t.shape[:-1] + (3 * t.shape[-1],), dtype=t.dtype, device=t.device)
            big[..., w.d:2 * w.d] = t
            return big[..., w.d:2 * w.d]
        qr, kr, vd, o, gd = (widen(t) for t in (qr, kr, vd, o, gd))
    dq, dk, dv = lcx.attn_bwd(qr, kr, vd, o, lse, gd, unrotate=unrotate, cos=cos, sin=sin, rope=cfg,
                              window=w.window, n_sink=w.n_sink, q_pos0=q_pos0, k_pos0=k_pos0,
                              grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return (dq.float().cpu().numpy(), dk.float().cpu().numpy(), dv.float().cpu().numpy())


def oracle_grads(w, q, k, v, dout, q_pos0=0, k_pos0=0, **kw):
    th, pf, lm = U.oracle_freqs(w)
    return oracle.attn_bwd(q, k, v, dout, th, pf, lm / np.sqrt(w.d), True, w.window, w.n_sink,
                           q_pos0, k_pos0, **kw)


def check_grads(got, ref, what, rel_fro=REL_FRO, rel_max=REL_MAX):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        if r is None:
            continue
        assert np.all(np.isfinite(g)), f"{what}/{name}: non-finite"
        e = g.astype(np.float64) - r
        nr = np.linalg.norm(r)
        fro = np.linalg.norm(e) / nr if nr > 0 else np.linalg.norm(e)
        mx = np.abs(e).max() / np.abs(r).max() if np.abs(r).max() > 0 else np.abs(e).max()
        U.log(f"{what}/{name}: rel-fro {fro:.3e} rel-max {mx:.3e} (|r|max {np.abs(r).max():.3e})")
        assert fro <= rel_fro, f"{what}/{name}: rel-fro {fro}"
        assert mx <= rel_max, f"{what}/{name}: rel-max {mx}"


SMALL = [
    # name, Hq, Hkv, d, n, scheme, window, n_sink, B
    ("n1", 4, 1, 64, 1, "ntk", -1, 0, 1),
    ("n63", 4, 2, 128, 63, "plain", -1, 0, 1),
    ("n65_d64", 8, 2, 64, 65, "yarn", -1, 0, 1),
    ("n129", 2, 1, 128, 129, "pi", -1, 0, 1),
    ("n333_b2", 4, 4, 128, 333, "ntk_parts", -1, 0, 2),
    ("n700_gqa8", 8, 1, 128, 700, "dynamic_ntk", -1, 0, 1),
    ("win_sink", 4, 1, 128, 900, "pi", 200, 4, 1),
    ("win0_sink3", 2, 1, 64, 300, "ntk", 0, 3, 1),
    ("win_tiles", 4, 2, 64, 1000, "plain", 127, 70, 1),
    ("pairs_d128", 4, 1, 128, 400, "pair_factors", -1, 0, 1),
]


def _pair_factors(d, seed):
    return tuple(np.exp(np.random.default_rng(seed).uniform(0.0, np.log(64.0), d // 2)))


def _w(name, Hq, Hkv, d, n, scheme, window, n_sink, B):
    return W.Workload(name, B, Hq, Hkv, d, n, scheme, 10000.0 if d == 64 else 500000.0, 64, 256,
                      cur_len=256, window=window, n_sink=n_sink, seed=300 + n,
                      factors=_pair_factors(d, n) if scheme == "pair_factors" else None)


@pytest.mark.parametrize("name,Hq,Hkv,d,n,scheme,window,n_sink,B", SMALL)
def test_backward_small_shapes(lcx, name, Hq, Hkv, d, n, scheme, window, n_sink, B):
    w = _w(name, Hq, Hkv, d, n, scheme, window, n_sink, B)
    U.log(f"bwd case {name}")
    q, k, v = U.inputs(w)
    dout = _dout(w, n)
    ref = oracle_grads(w, q, k, v, dout)
    got = gpu_grads(lcx, w, q, k, v, dout)
    check_grads(got, ref, name)


def test_backward_offsets_and_empty_rows(lcx):
    # rows at 300.. over keys 0..499; then keys starting at 50 for rows 0..99
    # (rows 0..49 keep no key: zero dq; keys past every row: zero dk, dv)
    w = W.TINY.with_(Hq=4, Hkv=2, d=128, base=500000.0, seed=11)
    q, _, _ = U.inputs(w, n_q=200)
    _, k, v = U.inputs(w, n_kv=500)
    dout = _dout(w, 200)
    ref = oracle_grads(w, q, k, v, dout, q_pos0=300)
    check_grads(gpu_grads(lcx, w, q, k, v, dout, q_pos0=300), ref, "q_pos0=300")
    q2, dout2 = q[:, :, :100], dout[:, :, :100]
    _, k2, v2 = U.inputs(w, n_kv=200)
    ref = oracle_grads(w, q2, k2, v2, dout2, k_pos0=50)
    got = gpu_grads(lcx, w, q2, k2, v2, dout2, k_pos0=50)
    assert np.all(got[0][:, :, :50] == 0)
    assert np.all(got[1][:, :, 50:] == 0) and np.all(got[2][:, :, 50:] == 0)
    check_grads(got, ref, "k_pos0=50")


def test_backward_bf16_gradients_and_rotated_frame(lcx):
    w = W.TINY.with_(Hq=8, Hkv=2, d=128, base=500000.0, n=450, seed=12, scheme="yarn", L_train=64,
                     L_target=512)
    q, k, v = U.inputs(w)
    dout = _dout(w, w.n)
    ref = oracle_grads(w, q, k, v, dout)
    # bf16 outputs add one rounding (2^-9 relative) per element
    check_grads(gpu_grads(lcx, w, q, k, v, dout, grad_dtype=torch.bfloat16), ref, "bf16-out",
                rel_fro=REL_FRO + 4e-3, rel_max=REL_MAX + 4e-3)
    # unrotate = 0: gradients of q~ = R(p) q and k~, i.e. the oracle's raw
    # gradients turned forward by R(p)
    th, pf, _ = U.oracle_freqs(w)
    pos = np.arange(w.n)
    rot = []
    for g in ref:
        x = g.reshape(-1, w.d)
        rows = np.tile(pos, x.shape[0] // w.n)
        rot.append(oracle.rope_rotate(x, rows, th, pf).reshape(g.shape))
    rot[2] = ref[2]
    check_grads(gpu_grads(lcx, w, q, k, v, dout, unrotate=False), tuple(rot), "rotated-frame")


def test_backward_strided_inputs(lcx):
    w = W.TINY.with_(Hq=4, Hkv=1, d=64, n=260, seed=13, window=40, n_sink=2)
    q, k, v = U.inputs(w)
    dout = _dout(w, w.n)
    ref = oracle_grads(w, q, k, v, dout)
    check_grads(gpu_grads(lcx, w, q, k, v, dout, strided=True), ref, "strided")


def test_backward_empty_inputs(lcx):
    # no keys: every row is empty (O = 0, LSE = -inf) and dq = 0; no rows: dk = dv = 0
    B, Hq, Hkv, d = 1, 2, 1, 64
    dv_ = U.dev()
    q = torch.randn((B, Hq, 70, d), device=dv_).to(torch.bfloat16)
    k0 = torch.empty((B, Hkv, 0, d), dtype=torch.bfloat16, device=dv_)
    o = torch.zeros((B, Hq, 70, d), dtype=torch.bfloat16, device=dv_)
    lse = torch.full((B, Hq, 70), float("-inf"), device=dv_)
    dq, dk, dv = lcx.attn_bwd(q, k0, k0, o, lse, q.clone())
    torch.cuda.synchronize()
    assert dq.shape == (B, Hq, 70, d) and torch.all(dq == 0)
    q0 = torch.empty((B, Hq, 0, d), dtype=torch.bfloat16, device=dv_)
    k = torch.randn((B, Hkv, 90, d), device=dv_).to(torch.bfloat16)
    lse0 = torch.empty((B, Hq, 0), device=dv_)
    dq, dk, dv = lcx.attn_bwd(q0, k, k.clone(), q0, lse0, q0)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


@pytest.mark.parametrize("Hq,Hkv,d,n,window,n_sink,B", [(8, 2, 128, 700, -1, 0, 1), (4, 4, 64, 333, 100, 4, 2),
                                                       (64, 8, 128, 8192, -1, 0, 1)])
def test_backward_work_order_gives_identical_gradients(lcx, Hq, Hkv, d, n, window, n_sink, B):
    # every dq row block and dk/dv key block is computed whole by the
    # workgroup that takes it, so the dynamic order must reproduce the static
    # order's gradients bit for bit (sched buffer reused, then a fresh one)
    w = W.TINY.with_(B=B, Hq=Hq, Hkv=Hkv, d=d, n=n, window=window, n_sink=n_sink, seed=23,
                     base=500000.0)
    q, k, v = U.inputs(w)
    qd, kd, vd, gd = U.to_dev(q), U.to_dev(k), U.to_dev(v), U.to_dev(_dout(w, n))
    cfg = _cfg(lcx, w)
    cos, sin = lcx.rope_tables(cfg, n, device=U.dev())
    _, kf = lcx.rope_apply_qk(None, kd, cos, sin, out_dtype=torch.float16)
    o, lse = lcx.attn_fwd(qd, kf, vd, rope_q=True, cos=cos, sin=sin, rope=cfg, window=window, n_sink=n_sink)
    qr, kr = lcx.rope_apply_qk(qd, kd, cos, sin, out_dtype=torch.bfloat16)
    sched = torch.empty(lcx.SCHED_BYTES // 8, dtype=torch.int64, device=U.dev())
    res = []
    for order in (False, sched, sched, True):
        grads = lcx.attn_bwd(qr, kr, vd, o, lse, gd, unrotate=True, cos=cos, sin=sin, rope=cfg,
                             window=window, n_sink=n_sink, sched=order)
        torch.cuda.synchronize()
        res.append(grads)
    for grads in res[1:]:
        for a, b in zip(res[0], grads):
            assert torch.equal(a, b)


def test_backward_deterministic(lcx):
    w = W.TINY.with_(Hq=8, Hkv=2, d=128, base=500000.0, n=1100, seed=15)
    q, k, v = U.inputs(w)
    dout = _dout(w, w.n)
    a = gpu_grads(lcx, w, q, k, v, dout)
    b = gpu_grads(lcx, w, q, k, v, dout)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
