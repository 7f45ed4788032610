"""The five synthetic workloads (shapes, RoPE scheme parameters, masks, seeds).

Plain data only.  Q/K/V are bf16 N(0,1) from ``fixtures.normal_bf16`` with
tensor ids Q=0, K=1, V=2, layout [B, H, n, d] contiguous, flat index = C order.
Positions are 0..n-1.  The schemes are named by string; each side maps the
name to its own enum.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    n: int
    scheme: str           # plain | pi | ntk | ntk_parts | yarn | dynamic_ntk | pair_factors
    base: float
    L_train: int
    L_target: int
    cur_len: int = 0      # dynamic NTK length l (0: use L_target)
    alpha: float = 1.0
    beta: float = 32.0
    causal: bool = True
    window: int = -1      # -1: none; else keys j >= i - window allowed
    n_sink: int = 0
    chunk: int = 0        # >0: KV processed in chunks of this many keys + merge
    seed: int = 1
    factors: tuple = None # pair_factors: the d/2 per-pair frequency divisors

    @property
    def s(self) -> float:
        return self.L_target / self.L_train

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def allowed_pairs(self) -> int:
        """Number of (query, key) pairs the mask keeps, per (batch, q head)."""
        import numpy as np
        n, w, ns = self.n, self.window, self.n_sink
        if w < 0:
            return n * (n + 1) // 2
        # row i keeps the window [max(0, i-w), i] plus sinks j < n_sink below it
        i = np.arange(n, dtype=np.int64)
        return int(np.sum(np.minimum(i + 1, w + 1) + np.minimum(ns, np.maximum(0, i - w))))

    def flop(self) -> int:
        """Algorithmic FLOP: 4 d per allowed pair per query head (QK^T + PV)."""
        return 4 * self.d * self.Hq * self.B * self.allowed_pairs()


TINY = Workload("tiny", 1, 4, 1, 64, 512, "ntk", 10000.0, 128, 512, seed=1)
LLAMA8B_32K = Workload("llama3_8b_32k_yarn", 1, 32, 8, 128, 32768, "yarn", 500000.0, 8192, 32768,
                       alpha=1.0, beta=32.0, seed=2)
LLAMA70B_128K = Workload("llama3_70b_128k_dynntk", 1, 64, 8, 128, 131072, "dynamic_ntk", 500000.0,
                         8192, 131072, cur_len=131072, seed=3)
SWA_SINK_64K = Workload("swa4096_sink4_64k_pi", 1, 32, 8, 128, 65536, "pi", 500000.0, 8192, 65536,
                        window=4096, n_sink=4, seed=4)
MILLION = Workload("million_1m_ntk_chunked", 1, 64, 8, 128, 1048576, "ntk", 500000.0, 8192, 1048576,
                   chunk=8192, seed=5)

ALL = [TINY, LLAMA8B_32K, LLAMA70B_128K, SWA_SINK_64K, MILLION]
BY_NAME = {w.name: w for w in ALL}
