"""Per-layer timing of encode and decode attention on single layers of a synthetic
workload, for shapes whose every layer does not fit beside its inputs (the 80-layer
large-batch workload) or to compare layers. HIP events on the library's stream.

    python -m rotated_angle_quantization_amd.layerbench --workload llama70b_batch --layers 0,40
"""

from __future__ import annotations

import argparse
import json

import torch

from . import _lib as kvq

HBM_PEAK_GBPS = 8000.0


def time_layer(cfg, layer: int, reps: int = 20, seed: int = 0) -> dict:
    from synthetic import layer_kv, query  # seeded input generators

    dev = torch.device("cuda:0")
    B, T, Hkv, Hq, d = cfg.batch, cfg.seq, cfg.hkv, cfg.hq, cfg.d
    nk, nv = cfg.bins(layer)
    desc = kvq.make_desc(d, Hkv, B, T, nk, nv, layer, seed)
    cache = kvq.alloc_cache(desc, dev)
    k, v = layer_kv(cfg, layer, dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    kvq.encode(desc, cache, k, v, 0)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(3):
        kvq.encode(desc, cache, k, v, 0)
    e1.record()
    torch.cuda.synchronize()
    enc_us = e0.elapsed_time(e1) * 1e3 / 3
    del k, v
    q = query(cfg, layer, dev)
    ws = kvq.alloc_workspace(desc, Hq, T, dev)
    out = torch.empty((B, Hq, d), dtype=torch.float16, device=dev)
    for _ in range(3):
        kvq.attn_decode(desc, cache, q, T, workspace=ws, out=out)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        kvq.attn_decode(desc, cache, q, T, workspace=ws, out=out)
    e1.record()
    torch.cuda.synchronize()
    att_us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = B * Hkv * T * kvq.tile_bytes(d, nk, nv) // 64
    return {
        "workload": cfg.name, "layer": layer, "n_k": nk, "n_v": nv, "batch": B, "seq": T,
        "group": Hq // Hkv, "attn_us": round(att_us, 2),
        "attn_GBps": round(nbytes / (att_us * 1e-6) / 1e9, 1),
        "attn_hbm_frac": round(nbytes / (att_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "encode_us": round(enc_us, 2),
        "encode_tokens_per_s_this_layer": round(B * T / (enc_us * 1e-6), 1),
    }


def main():
    from synthetic import get

    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama70b_batch")
    ap.add_argument("--layers", default="0,40")
    ap.add_argument("--reps", type=int, default=20)
    args = ap.parse_args()
    cfg = get(args.workload)
    for layer in (int(x) for x in args.layers.split(",")):
        print(json.dumps(time_layer(cfg, layer, args.reps)), flush=True)
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
