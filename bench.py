"""Benchmark of the scaled-RoPE causal GQA attention path on one MI355X.

One step = the whole hot path over one batch of synthetic input that is
already resident in HBM:
  1. lcx_rope_freqs     frequencies (host, fp64) + cos/sin tables (GPU)
  2. lcx_rope_apply_qk  K rotated once into f16
     lcx_attn_pack_v    V copied into 64-key tiles (PV operand layout)
  3. lcx_attn_fwd       causal GQA attention, RoPE fused into the Q load,
                        O (bf16) + LSE (fp32)
on the Llama-3-70B-shaped layer: B=1, 64 query / 8 KV heads, d=128,
n=131072, dynamic NTK (base 500000, L_train 8192, l=131072).

Prints ONE JSON line.  `value` is algorithmic causal-attention TFLOP/s of the
whole step (4·d·Hq·n(n+1)/2 FLOP; masked work never counted).
`roofline` is for the dominant kernel (attention), timed with HIP events on
the stream it runs on.  `cpu_baseline` times the fp64 oracle on a bounded
sample of rows of the same layer.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense bf16/f16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "causal attn TFLOP/s + % bf16 MFMA peak, 70B-shape GQA layer at 128K ctx"
PMC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_llama3_70b_128k_pmc.json")
KERNEL_SRC = [os.path.join(ROOT, "long_context_attention_rope_amd", "csrc", f)
              for f in ("attn_fwd.hip", "attn_tile.h")]  # the attention kernel's source text


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRC:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


BWD_PMC_FILE = os.path.join(ROOT, "profiles", "attn_bwd_llama3_70b_128k_pmc.json")
BWD_SRC = os.path.join(ROOT, "long_context_attention_rope_amd", "csrc", "attn_bwd.hip")


def bwd_kernel_hash() -> str:
    h = hashlib.sha256()
    for f in (BWD_SRC, KERNEL_SRC[1]):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def bwd_traffic_from_profile():
    """HBM bytes of one lcx_attn_bwd call (its three kernels) from the committed
    counter runs, only if they were taken on the current backward source."""
    try:
        rec = json.load(open(BWD_PMC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != bwd_kernel_hash():
        return None
    return rec.get("hbm_bytes_per_backward")


DEC_PMC_FILE = os.path.join(ROOT, "profiles", "attn_decode_llama3_70b_128k_pmc.json")
DEC_SRC = [os.path.join(ROOT, "long_context_attention_rope_amd", "csrc", f)
           for f in ("attn_fwd.hip", "attn_tile.h", "attn_merge.hip")]  # decode + combine kernels


def decode_kernel_hash() -> str:
    h = hashlib.sha256()
    for f in DEC_SRC:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def decode_traffic_from_profile(new_rows, splits):
    """HBM bytes of one lcx_attn_decode call (decode + combine kernels) from the
    committed counter runs, only for the same source, new rows and splits."""
    try:
        rec = json.load(open(DEC_PMC_FILE))
    except (OSError, ValueError):
        return None
    if (rec.get("kernel_source_sha256_16") != decode_kernel_hash() or rec.get("new_rows") != new_rows
            or rec.get("splits_per_kv_head") != splits):
        return None
    return rec.get("hbm_bytes_per_call")


def traffic_from_profile(launch_flop_bytes):
    """HBM bytes per attention launch from the committed rocprofv3 counter runs,
    only if they were taken on the current kernel source."""
    try:
        rec = json.load(open(PMC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def kv_cache_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int, dtype_bytes: int = 2) -> int:
    """KV cache per token: K and V of every layer and KV head."""
    return 2 * n_layers * n_kv_heads * head_dim * dtype_bytes


def backward_flop(w) -> float:
    """Algorithmic FLOP of the backward pass: five products (S, dP, dV, dK, dQ)
    of 2·d FLOP per kept pair per query head, i.e. 2.5 times the forward's."""
    return 2.5 * w.flop()


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _single_core(fn, flop_scale):
    """Rate of fn() on one thread (fn returns (flop, seconds)); threads restored after."""
    import oracle
    n = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        flop, dt = fn()
    finally:
        oracle.set_num_threads(n)
    return flop * flop_scale / dt / 1e12


def cpu_baseline(w, rows: int):
    import numpy as np
    import fixtures
    import oracle
    th, pf, lm = oracle.rope_freqs(w.scheme, w.base, w.d, w.L_train, w.L_target, w.cur_len,
                                   w.alpha, w.beta)
    rng = np.random.default_rng(12345)
    heads = rng.integers(0, w.Hq, rows).astype(np.int32)
    pos = rng.integers(0, w.n, rows).astype(np.int64)
    flat = heads.astype(np.int64) * w.n + pos
    q_rows = fixtures.rows_bf16(w.seed, fixtures.Q_ID, flat, w.d)
    k = fixtures.normal_bf16(w.seed, fixtures.K_ID, (w.B, w.Hkv, w.n, w.d))
    v = fixtures.normal_bf16(w.seed, fixtures.V_ID, (w.B, w.Hkv, w.n, w.d))
    def run(n_rows):
        t0 = time.perf_counter()
        oracle.attn_rows(q_rows[:n_rows], pos[:n_rows], heads[:n_rows], np.zeros(n_rows, np.int32), k, v,
                         w.Hq, th, pf, lm / np.sqrt(w.d), True, w.window, w.n_sink)
        return 4 * w.d * int(np.sum(pos[:n_rows] + 1)), time.perf_counter() - t0

    flop, dt = run(rows)
    one = _single_core(lambda: run(max(1, rows // 16)), 1.0)
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 3), "cpu_model": cpu_model(),
            "single_core_value": one, "extrapolated_full_layer_s": round(w.flop() / (flop / dt), 1),
            "sample": f"{rows} seeded rows (uniform head, uniform position) of the same layer, "
                      f"fp64, {flop:.3e} algorithmic FLOP, K rotation of the needed heads included; "
                      f"single core on the first {max(1, rows // 16)} of them"}


def copy_calibration(gib: float = 1.0, reps: int = 5):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = int(gib * (1 << 30)) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "reps": reps}))


def bench_chunked(args, w):
    """The million-token layer as the one-GPU share of ring attention: KV in
    chunks of w.chunk keys, one attention call per chunk, partials merged by
    LSE.  A step = tables + K rotation + V packing + the chunked driver with the
    merge fused into each call's epilogue; the separate-merge form (attention
    into a partial, then lcx_attn_merge) is timed once after the steps."""
    import numpy as np
    import torch

    import fixtures
    import long_context_attention_rope_amd as lcx

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q = to_dev(fixtures.normal_bf16(w.seed, fixtures.Q_ID, (w.B, w.Hq, w.n, w.d)))
    k = to_dev(fixtures.normal_bf16(w.seed, fixtures.K_ID, (w.B, w.Hkv, w.n, w.d)))
    v = to_dev(fixtures.normal_bf16(w.seed, fixtures.V_ID, (w.B, w.Hkv, w.n, w.d)))
    cfg = lcx.rope_cfg(w.scheme, w.base, w.d, w.L_train, w.L_target, w.cur_len, w.alpha, w.beta)
    cos = torch.empty((w.n, w.d // 2), dtype=torch.float32, device=dev)
    sin = torch.empty_like(cos)
    k_rot = torch.empty(k.shape, dtype=torch.float16, device=dev)
    v_tiles = torch.empty((w.B, w.Hkv, (w.n + 63) // 64, w.d, 64), dtype=torch.float16, device=dev)
    acc_o = torch.empty((w.B, w.Hq, w.n, w.d), dtype=torch.float32, device=dev)
    acc_l = torch.empty((w.B, w.Hq, w.n), dtype=torch.float32, device=dev)
    o = torch.empty((w.B, w.Hq, w.n, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, w.n), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sched = torch.empty(lcx.SCHED_BYTES // 8, dtype=torch.int64, device=dev) \
        if args.work_order == "dynamic" else False

    def step(ev=None, o_part=None, lse_part=None):
        if ev: ev[0].record(stream)
        lcx.rope_freqs(cfg, cos, sin, 0)
        lcx.rope_apply_qk(None, k, cos, sin, k_out=k_rot)
        lcx.pack_v(v, out=v_tiles)
        if ev: ev[1].record(stream)
        lcx.attn_fwd_chunked(q, k_rot, v_tiles, w.chunk, acc_o, acc_l, o, lse, o_part=o_part,
                             lse_part=lse_part, rope_q=True, cos=cos, sin=sin, rope=cfg, sched=sched)
        if ev: ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prep_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    drv_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    # separate merge pass, timed once
    o_part = torch.empty_like(acc_o)
    lse_part = torch.empty_like(acc_l)
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    step(sev, o_part, lse_part)
    torch.cuda.synchronize()
    sep_ms = sev[1].elapsed_time(sev[2])

    flop = w.flop()
    ms_step = wall * 1e3 / args.steps
    drv_tflops = flop / (drv_ms * 1e-3) / 1e12
    n_chunks = (w.n + w.chunk - 1) // w.chunk
    out = {
        "metric": "causal attn TFLOP/s, 1M-token GQA layer as 128 KV chunks + LSE merge (one GPU's ring share)",
        "value": round(flop / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
                   "seq_len": w.n, "rope": w.scheme, "rope_base": w.base, "L_train": w.L_train,
                   "L_target": w.L_target, "causal": True, "kv_chunk": w.chunk, "chunks": n_chunks,
                   "merge": "fused into each chunk's epilogue (accumulate)", "v_layout": "tiles",
                   "work_order": args.work_order},
        "pct_bf16_peak": round(100 * flop / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "tokens_per_s": round(w.B * w.n / (ms_step * 1e-3), 1),
        "kernels_ms": {"tables_rotate_pack": round(prep_ms, 3), "chunked_attention_fused_merge": round(drv_ms, 1),
                       "chunked_attention_separate_merge": round(sep_ms, 1)},
        "roofline": {"kernel": "attn_fwd (128 chunk launches)", "bound": "mfma", "achieved": round(drv_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(drv_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
    }
    if args.cpu_rows > 0:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    print(json.dumps(out), flush=True)


def bench_decode(args, w):
    """Split-KV decode on the layer's KV cache: N new rows (positions n-N .. n-1)
    of all query heads against the n cached keys.  A step = the RoPE table rows
    of the new positions (the base for the current length) + lcx_attn_decode.
    HBM-bound: the cache (K pre-rotated f16, V f16 tiles) is read once per step."""
    import numpy as np
    import torch

    import fixtures
    import long_context_attention_rope_amd as lcx

    n_q = args.decode
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q = to_dev(fixtures.normal_bf16(w.seed, fixtures.Q_ID, (w.B, w.Hq, n_q, w.d)))
    k = to_dev(fixtures.normal_bf16(w.seed, fixtures.K_ID, (w.B, w.Hkv, w.n, w.d)))
    v = to_dev(fixtures.normal_bf16(w.seed, fixtures.V_ID, (w.B, w.Hkv, w.n, w.d)))
    cfg = lcx.rope_cfg(w.scheme, w.base, w.d, w.L_train, w.L_target, w.cur_len, w.alpha, w.beta)
    # the cache: K rotated once (when it was written), V in tiles
    cos_all, sin_all = lcx.rope_tables(cfg, w.n, device=dev)
    _, k_rot = lcx.rope_apply_qk(None, k, cos_all, sin_all)
    v_tiles = lcx.pack_v(v)
    del k, v, cos_all, sin_all
    q_pos0 = w.n - n_q
    cos = torch.empty((n_q, w.d // 2), dtype=torch.float32, device=dev)
    sin = torch.empty_like(cos)
    n_splits = args.splits or lcx.decode_splits(w.B, w.Hkv, w.n, w.d)
    o = torch.empty((w.B, w.Hq, n_q, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, n_q), dtype=torch.float32, device=dev)
    o_part = torch.empty((n_splits, w.B, w.Hq, n_q, w.d), dtype=torch.float32, device=dev)
    lse_part = torch.empty((n_splits, w.B, w.Hq, n_q), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev: ev[0].record(stream)
        lcx.rope_freqs(cfg, cos, sin, q_pos0)
        if ev: ev[1].record(stream)
        lcx.attn_decode(q, k_rot, v_tiles, o, lse, n_splits=n_splits, o_part=o_part, lse_part=lse_part,
                        rope_q=True, cos=cos, sin=sin, tab_pos0=q_pos0, rope=cfg, window=w.window,
                        n_sink=w.n_sink, q_pos0=q_pos0)
        if ev: ev[2].record(stream)

    steps = max(args.steps, 50)
    for _ in range(max(args.warmup, 5)):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = float(np.median([e[0].elapsed_time(e[2]) for e in evs]))
    tab_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    dec_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    # one layer's cache: K rows (f16) and V tiles (f16, the last tile padded to 64 keys)
    cache_bytes = w.B * (w.n + 64 * ((w.n + 63) // 64)) * kv_cache_bytes_per_token(1, w.Hkv, w.d) // 2
    io_bytes = w.B * w.Hq * n_q * w.d * (2 + 2) + 2 * n_splits * w.B * w.Hq * n_q * (w.d + 1) * 4
    gbs = (cache_bytes + io_bytes) / (ms * 1e-3) / 1e9
    dec_gbs = (cache_bytes + io_bytes) / (dec_ms * 1e-3) / 1e9
    out = {
        "metric": "split-KV decode HBM GB/s (K and V cache, 2 B per element, read once per step)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": max(args.warmup, 5),
        "ms_per_step": round(ms, 4), "wall_ms_per_step": round(wall * 1e3 / steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name + "_decode", "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.d, "cached_keys": w.n, "new_rows": n_q, "splits_per_kv_head": n_splits,
                   "rope": w.scheme, "v_layout": "tiles"},
        "tokens_per_s": round(w.B * n_q / (ms * 1e-3), 1),
        "kernels_ms": {"rope_table (new rows)": round(tab_ms, 4), "attn_decode + combine": round(dec_ms, 4)},
        "roofline": {"kernel": "attn_decode + combine (one lcx_attn_decode call)", "bound": "hbm",
                     "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                     "traffic": decode_traffic_from_profile(n_q, n_splits)
                     if w.name == "llama3_70b_128k_dynntk" else None},
    }
    print(json.dumps(out), flush=True)


def bench_table(args, w):
    """The cos/sin table pass alone (lcx_rope_freqs for the layer's n positions):
    HBM write-bound, 8 bytes per (position, pair)."""
    import numpy as np
    import torch

    import long_context_attention_rope_amd as lcx

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = lcx.rope_cfg(w.scheme, w.base, w.d, w.L_train, w.L_target, w.cur_len, w.alpha, w.beta)
    half = w.d // 2
    cos = torch.empty((w.n, half), dtype=torch.float32, device=dev)
    sin = torch.empty_like(cos)
    stream = torch.cuda.current_stream(dev)
    steps = max(args.steps, 20)
    for _ in range(max(args.warmup, 3)):
        lcx.rope_freqs(cfg, cos, sin, 0)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        lcx.rope_freqs(cfg, cos, sin, 0)
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    nbytes = w.n * half * 8
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "RoPE cos/sin table HBM GB/s (fp32 cos and sin per position and pair, written once)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": max(args.warmup, 3),
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64", "data": "synthetic",
        "config": {"workload": w.name + "_rope_table", "positions": w.n, "pairs": half, "rope": w.scheme},
        "roofline": {"kernel": "rope_table_kernel", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": None},
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_bwd(w, m: int):
    """The oracle's backward pass (dq, dk, dv, every element) on the first m
    positions of every head of the layer: a causal prefix of the same shape."""
    import numpy as np
    import fixtures
    import oracle
    th, pf, lm = oracle.rope_freqs(w.scheme, w.base, w.d, w.L_train, w.L_target, w.cur_len,
                                   w.alpha, w.beta)
    def prefix(tid, H):
        # rows 0..m-1 of every (batch, head) of a [B, H, n, d] tensor
        flat = (np.arange(w.B * H, dtype=np.int64)[:, None] * w.n + np.arange(m)[None, :]).reshape(-1)
        return fixtures.rows_bf16(w.seed, tid, flat, w.d).reshape(w.B, H, m, w.d)
    q, g = prefix(fixtures.Q_ID, w.Hq), prefix(fixtures.DO_ID, w.Hq)
    k, v = prefix(fixtures.K_ID, w.Hkv), prefix(fixtures.V_ID, w.Hkv)
    def run(mm):
        t0 = time.perf_counter()
        oracle.attn_bwd(q[:, :, :mm], k[:, :, :mm], v[:, :, :mm], g[:, :, :mm], th, pf, lm / np.sqrt(w.d),
                        True, w.window, w.n_sink)
        return backward_flop(w.with_(n=mm)), time.perf_counter() - t0

    flop, dt = run(m)
    one = _single_core(lambda: run(max(1, m // 4)), 1.0)
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 3), "cpu_model": cpu_model(),
            "single_core_value": one, "extrapolated_full_layer_s": round(backward_flop(w) / (flop / dt), 1),
            "sample": f"the first {m} positions of all {w.Hq} query heads of the same layer (dq, dk, dv "
                      f"in full), fp64, {flop:.3e} algorithmic FLOP (5 products per kept pair); single "
                      f"core on the first {max(1, m // 4)} positions"}


def bench_backward(args, w):
    """The backward pass of the layer: a step = lcx_attn_bwd (row statistics,
    dq kernel, dk/dv kernel) with its inputs resident in HBM: q~ and k~ rotated
    to bf16, V rows, the forward's O (bf16) and LSE, a synthetic dL/dO; the
    gradients of the raw q, k (inverse rotation in the epilogues) in fp32."""
    import numpy as np
    import torch

    import fixtures
    import long_context_attention_rope_amd as lcx

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q = to_dev(fixtures.normal_bf16(w.seed, fixtures.Q_ID, (w.B, w.Hq, w.n, w.d)))
    k = to_dev(fixtures.normal_bf16(w.seed, fixtures.K_ID, (w.B, w.Hkv, w.n, w.d)))
    v = to_dev(fixtures.normal_bf16(w.seed, fixtures.V_ID, (w.B, w.Hkv, w.n, w.d)))
    g = to_dev(fixtures.normal_bf16(w.seed, fixtures.DO_ID, (w.B, w.Hq, w.n, w.d)))
    cfg = lcx.rope_cfg(w.scheme, w.base, w.d, w.L_train, w.L_target, w.cur_len, w.alpha, w.beta)
    cos, sin = lcx.rope_tables(cfg, w.n, device=dev)
    _, kf = lcx.rope_apply_qk(None, k, cos, sin)
    o, lse = lcx.attn_fwd(q, kf, lcx.pack_v(v), rope_q=True, cos=cos, sin=sin, rope=cfg,
                          window=w.window, n_sink=w.n_sink)
    del kf
    qr, kr = lcx.rope_apply_qk(q, k, cos, sin, out_dtype=torch.bfloat16)
    del q, k
    dq = torch.empty((w.B, w.Hq, w.n, w.d), dtype=torch.float32, device=dev)
    dk = torch.empty((w.B, w.Hkv, w.n, w.d), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    ws = torch.empty((w.B, w.Hq, w.n, 2), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sched = torch.empty(lcx.SCHED_BYTES // 8, dtype=torch.int64, device=dev) \
        if args.work_order == "dynamic" else False

    def step():
        lcx.attn_bwd(qr, kr, v, o, lse, g, dq=dq, dk=dk, dv=dv, workspace=ws, sched=sched, unrotate=True,
                     cos=cos, sin=sin, rope=cfg, window=w.window, n_sink=w.n_sink)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        step()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    bwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    ms_step = wall * 1e3 / args.steps
    flop = backward_flop(w)   # S, dP, dV, dK, dQ: five products per kept pair
    value = flop / (ms_step * 1e-3) / 1e12
    ach = flop / (bwd_ms * 1e-3) / 1e12
    out = {
        "metric": "causal attn backward TFLOP/s (5 products per kept pair) + % bf16 MFMA peak, "
                  "70B-shape GQA layer at 128K ctx",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name + "_backward", "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.d, "seq_len": w.n, "rope": w.scheme, "causal": True,
                   "window": w.window, "n_sink": w.n_sink, "grads": "dq, dk, dv fp32 (raw q, k)",
                   "mfma": "bf16 operands (q~, k~, V, dO, P, dS), fp32 accumulate",
                   "executed_products_per_pair": 7, "work_order": args.work_order},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "tokens_per_s": round(w.B * w.n / (ms_step * 1e-3), 1),
        "kernels_ms": {"attn_bwd (stats + dq + dk/dv)": round(bwd_ms, 3)},
        "roofline": {"kernel": "attn_bwd (stats + dq + dk/dv launches)", "bound": "mfma",
                     "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                     "traffic": bwd_traffic_from_profile()
                     if w.name == "llama3_70b_128k_dynntk" and args.work_order == "dynamic" else None},
    }
    if args.cpu_rows > 0:
        out["cpu_baseline"] = cpu_baseline_bwd(w, args.cpu_rows)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 10; 1 for the chunked workload)")
    ap.add_argument("--warmup", type=int, default=None, help="warm-up steps (default 3; 1 for the chunked workload)")
    ap.add_argument("--workload", default="llama3_70b_128k_dynntk")
    ap.add_argument("--k-mode", choices=["prerotate", "fused", "precise"], default="prerotate",
                    help="K rotated once by lcx_rope_apply_qk (default), inside the attention tile load, or "
                         "inside the tile load with the precise QK^T form (f16 high/low parts, three products)")
    ap.add_argument("--work-order", choices=["dynamic", "static"], default="dynamic",
                    help="forward work order: per-XCD queues with stealing (lcx_attn_args.sched), "
                         "or one fixed unit per workgroup")
    ap.add_argument("--v-layout", choices=["tiles", "rows"], default="tiles",
                    help="V packed into 64-key tiles by lcx_attn_pack_v inside the step (default) or read as rows")
    ap.add_argument("--cpu-rows", type=int, default=None,
                    help="oracle rows for the CPU baseline (default 16384; 640 for the chunked workload; 0: skip)")
    ap.add_argument("--decode", type=int, default=0, metavar="N",
                    help="time split-KV decode of N new rows (1..8) against this layer's cache instead")
    ap.add_argument("--splits", type=int, default=None, help="decode: workgroups per KV head")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward pass (lcx_attn_bwd) of this layer instead; --cpu-rows is then "
                         "the length of the prefix the oracle differentiates (default 5120)")
    ap.add_argument("--table", action="store_true",
                    help="time the cos/sin table pass (lcx_rope_freqs) for this layer's positions instead")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-merge-check", dest="merge_check", action="store_false",
                    help="skip timing the merge pass on this layer's partial sizes")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path would shard by KV head group, or by sequence as a ring of KV chunks).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    import fixtures
    import long_context_attention_rope_amd as lcx
    from fixtures import workloads as W

    w = W.BY_NAME[args.workload]
    if args.steps is None:
        args.steps = 1 if w.chunk else 10
    if args.warmup is None:
        args.warmup = 1 if w.chunk else 3
    if args.cpu_rows is None:
        args.cpu_rows = 640 if w.chunk else (5120 if args.bwd else 16384)
    if args.table:
        return bench_table(args, w)
    if args.bwd:
        return bench_backward(args, w)
    if w.chunk:
        return bench_chunked(args, w)
    if args.decode:
        return bench_decode(args, w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # synthetic inputs, generated on the host from the seeded generator, then resident in HBM
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q = to_dev(fixtures.normal_bf16(w.seed, fixtures.Q_ID, (w.B, w.Hq, w.n, w.d)))
    k = to_dev(fixtures.normal_bf16(w.seed, fixtures.K_ID, (w.B, w.Hkv, w.n, w.d)))
    v = to_dev(fixtures.normal_bf16(w.seed, fixtures.V_ID, (w.B, w.Hkv, w.n, w.d)))
    cfg = lcx.rope_cfg(w.scheme, w.base, w.d, w.L_train, w.L_target, w.cur_len, w.alpha, w.beta)
    half = w.d // 2
    cos = torch.empty((w.n, half), dtype=torch.float32, device=dev)
    sin = torch.empty((w.n, half), dtype=torch.float32, device=dev)
    k_rot = torch.empty(k.shape, dtype=torch.float16, device=dev)
    v_tiles = torch.empty((w.B, w.Hkv, (w.n + 63) // 64, w.d, 64), dtype=torch.float16, device=dev)
    tiled = args.v_layout == "tiles"
    o = torch.empty((w.B, w.Hq, w.n, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, w.n), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sched = torch.empty(lcx.SCHED_BYTES // 8, dtype=torch.int64, device=dev) \
        if args.work_order == "dynamic" else False

    def step(ev=None):
        if ev: ev[0].record(stream)
        lcx.rope_freqs(cfg, cos, sin, 0)
        if ev: ev[1].record(stream)
        if args.k_mode == "prerotate":
            lcx.rope_apply_qk(None, k, cos, sin, k_out=k_rot)
        if ev: ev[2].record(stream)
        vv = lcx.pack_v(v, out=v_tiles) if tiled else v
        if ev: ev[3].record(stream)
        lcx.attn_fwd(q, k_rot if args.k_mode == "prerotate" else k, vv, o, lse, rope_q=True,
                     rope_k=args.k_mode != "prerotate", cos=cos, sin=sin, rope=cfg,
                     window=w.window, n_sink=w.n_sink, precise_qk=args.k_mode == "precise",
                     sched=sched)
        if ev: ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the merge pass (chunked / ring form) on partials of this layer's size, timed
    # on its own after the step loop: reads two fp32 (O, LSE), writes one
    merge_gbs = None
    if args.merge_check:
        del o, k_rot
        oa = torch.zeros((w.B, w.Hq, w.n, w.d), dtype=torch.float32, device=dev)
        ob = torch.zeros_like(oa)
        la = torch.zeros((w.B, w.Hq, w.n), dtype=torch.float32, device=dev)
        lb = torch.zeros_like(la)
        lcx.attn_merge(oa, la, ob, lb)
        m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        m0.record(stream)
        for _ in range(3):
            lcx.attn_merge(oa, la, ob, lb)
        m1.record(stream)
        torch.cuda.synchronize()
        merge_ms = m0.elapsed_time(m1) / 3
        merge_bytes = 3 * (oa.numel() + la.numel()) * 4
        merge_gbs = round(merge_bytes / (merge_ms * 1e-3) / 1e9, 1)
        del oa, ob, la, lb

    tab_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    rot_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    pack_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    attn_ms = float(np.mean([e[3].elapsed_time(e[4]) for e in evs]))
    ms_step = wall * 1e3 / args.steps
    flop = w.flop()
    tokens = w.B * w.n
    value = flop / (ms_step * 1e-3) / 1e12
    attn_tflops = flop / (attn_ms * 1e-3) / 1e12
    # the committed counter runs cover the default configuration of the 70B layer only
    profiled = w.name == W.LLAMA70B_128K.name and args.k_mode == "prerotate" and args.v_layout == "tiles" \
        and args.work_order == "dynamic"
    traffic = traffic_from_profile(flop) if profiled else None

    tab_bytes = w.n * half * 8
    rot_bytes = w.B * w.Hkv * w.n * w.d * 4 + tab_bytes
    pack_bytes = w.B * w.Hkv * w.d * 2 * (w.n + 64 * ((w.n + 63) // 64))

    out = {
        "metric": METRIC if w.name == W.LLAMA70B_128K.name else
                  f"causal attn TFLOP/s + % bf16 MFMA peak, {w.name} layer",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.d, "seq_len": w.n, "rope": w.scheme, "rope_base": w.base,
                   "L_train": w.L_train, "cur_len": w.cur_len, "causal": True,
                   "k_rope": args.k_mode, "v_layout": args.v_layout, "work_order": args.work_order,
                   "mfma": (("QK^T as three f16 products of high/low parts" if args.k_mode == "precise"
                             else "QK^T f16 operands") + ", PV " + ("f16" if args.v_layout == "tiles" else "bf16")
                            + " operands, fp32 accumulate")},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "tokens_per_s": round(tokens / (ms_step * 1e-3), 1),
        "kernels_ms": {"rope_table": round(tab_ms, 4), "rope_apply_k": round(rot_ms, 4),
                       "pack_v": round(pack_ms, 4), "attn_fwd": round(attn_ms, 3)},
        "hbm_gbs": {"rope_table": round(tab_bytes / (tab_ms * 1e-3) / 1e9, 1),
                    "rope_apply_k": round(rot_bytes / (rot_ms * 1e-3) / 1e9, 1)
                    if args.k_mode == "prerotate" else None,
                    "pack_v": round(pack_bytes / (pack_ms * 1e-3) / 1e9, 1) if tiled else None,
                    "attn_merge": merge_gbs, "peak": PEAK_HBM_GBS},
        "roofline": {"kernel": "attn_fwd", "bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
    }
    if args.cpu_rows > 0:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
