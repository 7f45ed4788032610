"""Shared helpers of the GPU parity tests: seeded inputs on the device, sampled
rows, the oracle on those rows, and the tolerance checks."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import fixtures
import oracle

# tolerances stated for the attention path (O against the fp64 oracle, LSE)
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3
TABLE_MAX_ABS = 1e-6


def log(msg: str):
    sys.stderr.write(f"[{time.strftime('%H:%M:%S')}] {msg}\n")
    sys.stderr.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def inputs(w, n_q=None, n_kv=None):
    """Host bf16 bit arrays Q [B,Hq,n_q,d], K, V [B,Hkv,n_kv,d] of workload w."""
    n_q = w.n if n_q is None else n_q
    n_kv = w.n if n_kv is None else n_kv
    q = fixtures.normal_bf16(w.seed, fixtures.Q_ID, (w.B, w.Hq, n_q, w.d))
    k = fixtures.normal_bf16(w.seed, fixtures.K_ID, (w.B, w.Hkv, n_kv, w.d))
    v = fixtures.normal_bf16(w.seed, fixtures.V_ID, (w.B, w.Hkv, n_kv, w.d))
    return q, k, v


def oracle_freqs(w):
    return oracle.rope_freqs(w.scheme, w.base, w.d, w.L_train, w.L_target, w.cur_len, w.alpha, w.beta,
                             factors=w.factors)


def sample_rows(w, count=4096, seed=0, n_q=None, extra_pos=()):
    """(batch, head, row) triples: edge rows on every head plus seeded uniform rows."""
    n = w.n if n_q is None else n_q
    edge = {0, 1, 2, 3, 4, 5, 31, 32, 63, 64, 65, 127, 128, 129, 255, 256, n - 1, n - 2, n - 3,
            n - 64, n - 65, n - 128, n - 129}
    if w.window >= 0:
        for dlt in range(-2, 8):
            edge.add(w.window + dlt)
            edge.add(w.window + w.n_sink + dlt)
    if w.chunk:
        for c in (1, 2, 3, n // w.chunk // 2, n // w.chunk - 1):
            edge.update({c * w.chunk - 1, c * w.chunk, c * w.chunk + 1})
    edge.update(extra_pos)
    edge = sorted(p for p in edge if 0 <= p < n)
    trip = [(b, h, p) for b in range(w.B) for h in range(w.Hq) for p in edge[:: max(1, len(edge) // 8)]]
    trip += [(0, h % w.Hq, p) for h, p in enumerate(edge)]
    rng = np.random.default_rng(seed)
    while len(trip) < count:
        trip.append((int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(n))))
    trip = sorted(set(trip))[:count]
    a = np.array(trip, dtype=np.int64)
    return a[:, 0].astype(np.int32), a[:, 1].astype(np.int32), a[:, 2]


def oracle_rows(w, q, k, v, bb, hh, rr, q_pos0=0, k_pos0=0, rope=True, sm_scale=None):
    th, pf, lm = oracle_freqs(w)
    if sm_scale is None:
        sm_scale = lm / np.sqrt(w.d)
    qrows = q[bb, hh, rr]
    return oracle.attn_rows(qrows, rr + q_pos0, hh, bb, k, v, w.Hq, th if rope else None, pf, sm_scale,
                            True, w.window, w.n_sink, k_pos0=k_pos0)


def check(o_gpu: np.ndarray, l_gpu: np.ndarray, o_ref: np.ndarray, l_ref: np.ndarray, what: str):
    """The stated bar: O max-abs <= 2e-2, mean-abs <= 2e-3, LSE max-abs <= 1e-3
    (both -inf together for empty rows)."""
    o_gpu = o_gpu.astype(np.float64)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    inf_g, inf_r = np.isneginf(l_gpu), np.isneginf(l_ref)
    assert np.array_equal(inf_g, inf_r), f"{what}: empty rows differ"
    eo = np.abs(o_gpu - o_ref)
    el = np.abs(l_gpu[~inf_r] - l_ref[~inf_r]) if (~inf_r).any() else np.zeros(1)
    log(f"{what}: O max-abs {eo.max():.3e} mean-abs {eo.mean():.3e}; LSE max-abs {el.max():.3e} "
        f"({o_ref.shape[0]} rows)")
    assert eo.max() <= O_MAX_ABS, f"{what}: O max-abs {eo.max()}"
    assert eo.mean() <= O_MEAN_ABS, f"{what}: O mean-abs {eo.mean()}"
    assert el.max() <= LSE_MAX_ABS, f"{what}: LSE max-abs {el.max()}"
    return eo.max(), eo.mean(), el.max()
