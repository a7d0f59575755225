"""The five synthetic layer workloads, named by what they are.

Each entry pairs a draw recipe with the selection policy applied after
scoring. Shapes follow the model families the pages measure on (a 1.5B-class
Qwen2.5 layer, a Qwen3-8B layer, a Qwen2.5-14B layer) and the KVpop
future-attention setting on causal self-attention.

Selection:
* ``keep_k`` / ``keep_pct``: per KV head, keep the k highest-scoring keys among
  the non-window keys (k = floor(pct * n / 100) in integer arithmetic), plus the
  window of the last ``window`` keys.
* ``tau``: keep non-window keys whose score is >= tau, plus the window.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

from . import Recipe


@dataclass(frozen=True)
class Workload:
    name: str
    recipe: Recipe
    score_mode: str            # "max" (repeat pass) or "sum" (future mass)
    window: int
    keep_pcts: tuple = ()      # top-k percentages
    keep_k: int = -1           # explicit top-k
    tau: float = -1.0          # threshold (linear score space)
    seed: int = 0

    def ks(self) -> list[int]:
        n = self.recipe.n_ctx
        if self.keep_k >= 0:
            return [self.keep_k]
        return [(p * n) // 100 for p in self.keep_pcts]


TINY_KVZIP = Workload(
    name="tiny-kvzip-d64-256",
    recipe=Recipe(Hq=4, Hkv=2, D=64, n_ctx=256, n_q=256, mask="repeat", chunk=256,
                  scale=1.0, q_prescale=1.0 / 8.0),
    score_mode="max", window=32, keep_k=64, seed=0)

QWEN25_1P5B_2K = Workload(
    name="qwen2.5-1.5b-layer-kvzip+-2k",
    recipe=Recipe(Hq=12, Hkv=2, D=128, n_ctx=2048, n_q=2048, mask="repeat", chunk=2048,
                  lowrank_rank=8, lowrank_scale=2.0, value_norms=True, d_hidden=1536),
    score_mode="max", window=128, keep_pcts=(30, 50, 70), seed=1)

QWEN3_8B_32K = Workload(
    name="qwen3-8b-layer-kvzip+-32k",
    recipe=Recipe(Hq=32, Hkv=8, D=128, n_ctx=32768, n_q=32768, mask="repeat", chunk=2048,
                  lowrank_rank=8, lowrank_scale=2.0, value_norms=True, d_hidden=4096),
    score_mode="max", window=128, tau=math.exp(-6.0), seed=2)

KVPOP_CAUSAL_16K = Workload(
    name="kvpop-future-mass-causal-16k",
    recipe=Recipe(Hq=32, Hkv=8, D=128, n_ctx=16384, n_q=16384, mask="causal",
                  sinks=4, sink_mult=4.0),
    score_mode="sum", window=128, keep_pcts=(12, 25), seed=3)

QWEN25_14B_120K = Workload(
    name="qwen2.5-14b-layer-kvzip+-120k",
    recipe=Recipe(Hq=40, Hkv=8, D=128, n_ctx=120000, n_q=120000, mask="repeat", chunk=2048,
                  lowrank_rank=8, lowrank_scale=2.0, value_norms=True, d_hidden=5120,
                  dup_frac=0.01),
    score_mode="max", window=128, keep_pcts=(25,), seed=4)

ALL = [TINY_KVZIP, QWEN25_1P5B_2K, QWEN3_8B_32K, KVPOP_CAUSAL_16K, QWEN25_14B_120K]
BY_NAME = {w.name: w for w in ALL}
