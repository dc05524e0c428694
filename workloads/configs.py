"""The workloads, by shape.

Shapes follow the pages' setting (64-token blocks, 8B-class heads: 32 query
heads, 8 KV heads, head_dim 128, hidden 4096; 128K contexts; a 2048-token
local window in prefill) -- "SparDA: a fourth projection that lets sparse
attention prefetch its own KV cache", "One Forecast head per GQA group"
(closing paragraph on the evaluated configuration) and "Three speedups, three
different baselines" (128K decode, batch sweep).
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "decode" | "prefill" | "offload"
    dtype: str                # "f32" | "bf16": K, V, Q (and x, W) element type
    B: int
    Hq: int
    Hkv: int
    d: int
    hidden: int | None        # None: the Forecast vector is given directly
    T: int
    block: int
    topk: int
    n_init: int
    n_local: int
    layers: int
    seed: int
    chunk: int | None = None         # prefill query-chunk length
    plant_frac: float | None = None  # prefill: fraction of blocks with an offset
    host_layers: int | None = None   # offload: distinct host KV layers (layer l uses l % host_layers)
    plant: int | None = None         # decode: planted blocks per (b, g) (None: topk)
    drift: float | None = None       # steady-state offload: random-walk step of the Forecast input per decode step

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def NB(self) -> int:
        return self.T // self.block

    @property
    def U(self) -> int:
        return self.topk + self.n_init + self.n_local

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)


_ALL = [
    Workload("tiny-decode-fp32", "decode", "f32", B=1, Hq=4, Hkv=1, d=64, hidden=None,
            T=4096, block=64, topk=8, n_init=1, n_local=2, layers=1, seed=0),
    Workload("decode-B4-32K", "decode", "bf16", B=4, Hq=32, Hkv=8, d=128, hidden=4096,
            T=32768, block=64, topk=32, n_init=1, n_local=2, layers=1, seed=1),
    Workload("decode-B8-128K-32L", "decode", "bf16", B=8, Hq=32, Hkv=8, d=128, hidden=4096,
            T=131072, block=64, topk=64, n_init=1, n_local=4, layers=32, seed=2),
    Workload("prefill-B4-128K", "prefill", "bf16", B=4, Hq=32, Hkv=8, d=128, hidden=None,
            T=131072, block=64, topk=64, n_init=1, n_local=32, layers=1, seed=3,
            chunk=2048, plant_frac=0.05),
    Workload("offload-decode-B16-128K-32L", "offload", "bf16", B=16, Hq=32, Hkv=8, d=128,
            hidden=4096, T=131072, block=64, topk=64, n_init=1, n_local=4, layers=32, seed=4,
            host_layers=4),
    Workload("offload-steady-B16-128K-32L", "offload", "bf16", B=16, Hq=32, Hkv=8, d=128, hidden=4096,
            T=131072, block=64, topk=64, n_init=1, n_local=4, layers=32, seed=5, host_layers=4, plant=32,
            drift=0.05),
]

# the workloads by name
WORKLOADS = {w.name: w for w in _ALL}
