"""Synthetic fidelity of the angle codec: bits per element against reconstruction,
softmax and attention-output error, for chosen (n_K, n_V), on seeded synthetic K/V
shaped like a workload's layers.

"TurboAngle: Near-Lossless KV Cache Compression via Uniform Angle Quantization"
(arXiv 2603.27467), Abstract, reports the trade-off of per-layer codebook sizes on real
models (bits per element against perplexity, with K- or V-dominated layers). Models and
corpora are not available here, so this measures the same kind of trade-off on synthetic
tensors: how each (n_K, n_V) moves the error of the reconstructed keys and values, of
the softmax weights (KL divergence) and of the attention output.

Every quantised quantity comes from libkvq (encode, dequantise, decode attention); the
exact side is plain float64 PyTorch on the CPU over the unquantised inputs.

    python -m rotated_angle_quantization_amd.fidelity --workload tinyllama --layer 0
"""

from __future__ import annotations

import argparse
import json
import math

import torch

from . import _lib as kvq


def bits_per_element(d: int, n_k: int, n_v: int) -> float:
    """Cache bits per K or V element (record bytes of a token-head over its 2d values)."""
    return kvq.tile_bytes(d, n_k, n_v) * 8.0 / (64 * 2 * d)


def _attention64(q, k, v, scale):
    """Exact decode attention in float64: q [B, Hq, d], k/v [B, T, Hkv, d]; returns the
    output [B, Hq, d] and the softmax weights [B, Hq, T]."""
    g = q.shape[1] // k.shape[2]
    kk = k.repeat_interleave(g, dim=2).permute(0, 2, 1, 3)  # [B, Hq, T, d]
    vv = v.repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    s = torch.matmul(kk, q.unsqueeze(-1)).squeeze(-1) * scale
    p = torch.softmax(s, dim=-1)
    return torch.matmul(p.unsqueeze(-2), vv).squeeze(-2), p


def layer_fidelity(k: torch.Tensor, v: torch.Tensor, q: torch.Tensor, n_k: int, n_v: int,
                   layer: int = 0, seed: int = 0) -> dict:
    """Errors of one layer coded with (n_k, n_v). k, v: device [B, T, Hkv, d]; q: device
    [B, Hq, d]. Returns bits per element, key / value normalised squared error, the mean
    KL divergence of the softmax weights and the attention-output relative L2 error
    (mean and max over (batch, query head))."""
    bsz, t, hkv, d = k.shape
    desc = kvq.make_desc(d, hkv, bsz, t, n_k, n_v, layer, seed)
    cache = kvq.alloc_cache(desc, k.device)
    kvq.encode(desc, cache, k, v, 0)
    kh, vh = kvq.decode(desc, cache, 0, t, out_dtype=torch.float32)
    out = kvq.attn_decode(desc, cache, q, t, out_dtype=torch.float32)
    torch.cuda.synchronize(k.device)
    k64, v64, q64 = (x.detach().to("cpu", torch.float64) for x in (k, v, q))
    kh64, vh64, out64 = (x.detach().to("cpu", torch.float64) for x in (kh, vh, out))
    scale = 1.0 / math.sqrt(d)
    o_ref, p_ref = _attention64(q64, k64, v64, scale)
    _, p_hat = _attention64(q64, kh64, vh64, scale)
    kl = (p_ref * (torch.log(p_ref.clamp_min(1e-300)) - torch.log(p_hat.clamp_min(1e-300)))).sum(-1)
    rel = (out64 - o_ref).norm(dim=-1) / o_ref.norm(dim=-1).clamp_min(1e-300)
    return {
        "n_k": n_k, "n_v": n_v,
        "bits_per_element": bits_per_element(d, n_k, n_v),
        "key_nmse": float(((kh64 - k64) ** 2).sum() / (k64 ** 2).sum()),
        "value_nmse": float(((vh64 - v64) ** 2).sum() / (v64 ** 2).sum()),
        "softmax_kl_mean": float(kl.mean()),
        "attn_rel_l2_mean": float(rel.mean()),
        "attn_rel_l2_max": float(rel.max()),
    }


def sweep(k, v, q, grid, layer=0, seed=0, extra=()) -> list[dict]:
    """K-side sweep (n_V held at its largest value), V-side sweep (n_K held at its
    largest), the diagonal n_K = n_V, then any extra (n_K, n_V) pairs."""
    top = max(grid)
    cases = [(n, top) for n in grid] + [(top, n) for n in grid if n != top] + \
            [(n, n) for n in grid if n != top]
    cases += [c for c in extra if c not in cases]
    return [layer_fidelity(k, v, q, nk, nv, layer, seed) for nk, nv in cases]


def main():
    from synthetic import get, layer_kv, query  # seeded input generators

    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="tinyllama")
    ap.add_argument("--layer", type=int, default=0)
    ap.add_argument("--tokens", type=int, default=4096)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--grid", default="64,128,256",
                    help="codebook sizes (n in [2, 256]; n <= 32 is attended through a 6-bit copy)")
    ap.add_argument("--json", action="store_true")
    args = ap.parse_args()
    cfg = get(args.workload)
    dev = torch.device("cuda:0")
    k, v = layer_kv(cfg, args.layer, dev, seq=args.tokens, batch=args.batch)
    q = query(cfg, args.layer, dev, batch=args.batch)
    rows = sweep(k, v, q, [int(x) for x in args.grid.split(",")], args.layer,
                 extra=[tuple(cfg.bins(args.layer))])
    if args.json:
        print(json.dumps({"workload": cfg.name, "layer": args.layer, "tokens": args.tokens,
                          "batch": args.batch, "rows": rows}))
        return
    print(f"{cfg.name} layer {args.layer}, {args.batch} x {args.tokens} tokens, "
          f"{cfg.hkv}/{cfg.hq} heads, d {cfg.d}")
    print("| n_K | n_V | bits/elem | key NMSE | value NMSE | softmax KL | attn rel-L2 mean | max |")
    print("|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['n_k']} | {r['n_v']} | {r['bits_per_element']:.3f} | {r['key_nmse']:.2e} | "
              f"{r['value_nmse']:.2e} | {r['softmax_kl_mean']:.2e} | "
              f"{r['attn_rel_l2_mean']:.2e} | {r['attn_rel_l2_max']:.2e} |")


if __name__ == "__main__":
    main()
