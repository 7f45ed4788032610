"""Sizing arithmetic: the KV-cache bytes the pages print, and the pair / FLOP
counters behind every throughput figure, against brute force.

KV cache per token of the 70B GQA model and its totals: tests/golden/kv_cache_70b.txt
(page "上下文擴充套件（Context Extension）", KV Cache 的視訊記憶體架構).  The FLOP
counter counts 4·d per kept (query, key) pair per query head (QK^T and PV);
the kept pairs follow the mask of "上下文窗口扩展技术：从 4K 到 1M" §4.1-§4.2
(causal, window [i-w, i], sinks j < n_sink)."""
import pathlib

import numpy as np
import pytest

import bench
from fixtures import workloads as W

GOLDEN = pathlib.Path(__file__).parent / "golden"


def _kv_golden():
    vals, rows = {}, []
    for line in (GOLDEN / "kv_cache_70b.txt").read_text().splitlines():
        line = line.split("#")[0].strip()
        if not line:
            continue
        a, b = line.split()
        if a.isdigit():
            rows.append((int(a), float(b)))
        else:
            vals[a] = int(b)
    return vals, rows


def test_kv_cache_bytes_per_token_matches_the_page():
    v, rows = _kv_golden()
    per_tok = bench.kv_cache_bytes_per_token(v["n_layers"], v["n_kv_heads"], v["head_dim"], v["dtype_bytes"])
    assert per_tok == v["bytes_per_token"]
    for tokens, approx_gb in rows:
        total_gib = per_tok * tokens / 2**30
        # the page rounds (1.25 -> 1.2, 40.0 -> 40, 320 -> 300)
        assert abs(total_gib - approx_gb) <= 0.1 * approx_gb, (tokens, total_gib, approx_gb)


def test_kv_cache_of_one_layer_is_the_decode_bytes():
    # the decode bench reads one layer's cache: K and V of the 8 KV heads, 128K keys
    w = W.LLAMA70B_128K
    assert bench.kv_cache_bytes_per_token(1, w.Hkv, w.d) * w.n == 536_870_912


def _pairs_brute(n, window, n_sink):
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    keep = j <= i
    if window >= 0:
        keep &= (j >= i - window) | (j < n_sink)
    return int(keep.sum())


@pytest.mark.parametrize("n,window,n_sink", [(1, -1, 0), (64, -1, 0), (300, -1, 0), (300, 0, 0), (300, 0, 3),
                                             (517, 40, 4), (517, 600, 4), (1000, 127, 70), (1000, 5, 999)])
def test_allowed_pairs_equal_brute_force(n, window, n_sink):
    w = W.TINY.with_(n=n, window=window, n_sink=n_sink)
    assert w.allowed_pairs() == _pairs_brute(n, window, n_sink)


def test_flop_counters_of_the_workloads():
    w = W.LLAMA70B_128K
    assert w.flop() == 4 * 128 * 64 * (131072 * 131073 // 2) == 281_477_124_194_304
    assert bench.backward_flop(w) == 2.5 * w.flop()
    # window 4096 + 4 sinks over 64K: each row keeps min(i+1, 4097) keys plus the
    # sinks below its window
    s = W.SWA_SINK_64K
    n, wd, ns = s.n, s.window, s.n_sink
    closed = sum(min(i + 1, wd + 1) for i in range(n)) + sum(min(ns, max(0, i - wd)) for i in range(n))
    assert s.allowed_pairs() == closed
    assert s.flop() == 4 * s.d * s.Hq * closed
