"""Seeded generators for K, V and query tensors (no codec arithmetic here).

tiny recipe: NumPy default_rng(0) draws K, V, q (that order) as float64 standard
normals, cast to float32; K channels 3 and 17 are scaled by 8.

gqa recipe (torch Philox/CPU generator, seeded per (seed, layer, tensor)):
  K ~ N(0, 1) with 4 distinct outlier channels per (layer, kv head) scaled by 10,
  times a per-token factor exp(0.25 N(0, 1)) shared by all heads; V ~ N(0, 1);
  q ~ N(0, 1); all stored as fp16.
gqa_drift recipe: gqa plus 0.5 sin(2 pi t / 4096 + phi[kv head, channel]) added to K
  after the scaling, phi ~ U[0, 2 pi) per (layer, kv head, channel).
"""

from __future__ import annotations

import math

import numpy as np
import torch

from .configs import Workload

_TAGS = {"k": 1, "v": 2, "q": 3, "outlier": 4, "scale": 5, "phase": 6}


def _gen(device, seed: int, layer: int, tag: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + layer * 101 + _TAGS[tag]) & ((1 << 63) - 1))
    return g


def tiny_inputs() -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The tiny workload: K, V [1, 256, 1, 64] and q [1, 1, 64], float32."""
    rng = np.random.default_rng(0)
    k = rng.standard_normal((1, 256, 1, 64))
    v = rng.standard_normal((1, 256, 1, 64))
    q = rng.standard_normal((1, 1, 64))
    k[..., 3] *= 8.0
    k[..., 17] *= 8.0
    return k.astype(np.float32), v.astype(np.float32), q.astype(np.float32)


def layer_kv(cfg: Workload, layer: int, device="cpu", seed: int = 0,
             seq: int | None = None, batch: int | None = None):
    """K and V of one layer, [batch, seq, hkv, d] in the workload's input dtype.

    seq / batch may be given smaller than the workload's to draw a prefix-shaped
    sample with the same recipe (used by CPU-sized tests)."""
    if cfg.recipe == "tiny":
        k, v, _ = tiny_inputs()
        return (torch.from_numpy(k).to(device), torch.from_numpy(v).to(device))
    bsz = cfg.batch if batch is None else batch
    t = cfg.seq if seq is None else seq
    shape = (bsz, t, cfg.hkv, cfg.d)
    k = torch.randn(shape, generator=_gen(device, seed, layer, "k"), device=device)
    go = _gen(device, seed, layer, "outlier")
    for h in range(cfg.hkv):
        ch = torch.randperm(cfg.d, generator=go, device=device)[:4]
        k[:, :, h, ch] *= 10.0
    scale = torch.exp(0.25 * torch.randn((bsz, t, 1, 1), device=device,
                                         generator=_gen(device, seed, layer, "scale")))
    k *= scale
    if cfg.recipe == "gqa_drift":
        phi = 2 * math.pi * torch.rand((cfg.hkv, cfg.d), device=device,
                                       generator=_gen(device, seed, layer, "phase"))
        pos = torch.arange(t, device=device, dtype=torch.float32)
        drift = 0.5 * torch.sin(2 * math.pi * pos[:, None, None] / 4096.0 + phi[None])
        k += drift[None]
    v = torch.randn(shape, generator=_gen(device, seed, layer, "v"), device=device)
    dt = torch.float16 if cfg.dtype == "f16" else torch.float32
    return k.to(dt), v.to(dt)


def query(cfg: Workload, layer: int, device="cpu", seed: int = 0,
          batch: int | None = None):
    """Decode-step query, [batch, hq, d] in the workload's input dtype."""
    if cfg.recipe == "tiny":
        _, _, q = tiny_inputs()
        return torch.from_numpy(q).to(device)
    bsz = cfg.batch if batch is None else batch
    q = torch.randn((bsz, cfg.hq, cfg.d), generator=_gen(device, seed, layer, "q"),
                    device=device)
    dt = torch.float16 if cfg.dtype == "f16" else torch.float32
    return q.to(dt)
