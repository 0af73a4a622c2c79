"""Workload shapes: layers, batch, sequence, heads, head size, input dtype and the
per-layer (n_K, n_V) angle-bin counts (per-layer early boost: a leading subset of
layers gets finer codebooks, as the TurboAngle abstract describes)."""

from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    seq: int
    hkv: int
    hq: int
    d: int
    dtype: str  # "f32" or "f16"
    recipe: str  # "tiny", "gqa" or "gqa_drift"
    boosted_layers: int = 0  # layers [0, boosted_layers) use boost_n for K and V
    boost_n: int = 256
    n_k: int = 128
    n_v: int = 64

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    def bins(self, layer: int) -> tuple[int, int]:
        if layer < self.boosted_layers:
            return self.boost_n, self.boost_n
        return self.n_k, self.n_v


CONFIGS = {
    "tiny": Workload("tiny", 1, 1, 256, 1, 1, 64, "f32", "tiny"),
    "tinyllama": Workload("tinyllama", 22, 1, 4096, 4, 32, 64, "f16", "gqa"),
    "mistral7b": Workload("mistral7b", 32, 4, 32768, 8, 32, 128, "f16", "gqa",
                          boosted_layers=4),
    "llama3_8b_long": Workload("llama3_8b_long", 32, 1, 131072, 8, 32, 128, "f16",
                               "gqa_drift"),
    "llama70b_batch": Workload("llama70b_batch", 80, 64, 8192, 8, 64, 128, "f16", "gqa",
                               boosted_layers=8),
}


def get(name: str) -> Workload:
    return CONFIGS[name]
