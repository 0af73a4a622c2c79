"""Benchmark of the angle-quantised KV-cache hot path on one MI355X.

One step = the whole path over one batch of synthetic input, all layers:
  encode   K/V [B, T, Hkv, d] fp16 -> packed cache (kvq_encode), every layer
  attend   one decode query per sequence over the full compressed cache
           (kvq_attn_decode: one kernel launch), every layer
  dequant  packed cache -> fp16 K/V (kvq_decode), every layer
After the timed steps, a ragged-batch decode loop is timed on the same caches (append one
token per sequence at its own slot, attend with per-sequence lengths) and reported under
`decode_loop`; multi-query attention (kvq_attn_multi, several query tokens per sequence
on the matrix cores) is timed on them and reported under `multi_query`; a read-only
streaming probe over the same buffers gives the achievable read bandwidth
(`roofline.stream_probe`); last, the triplet codec is run on the same K/V and queries
(`triplet`). Inputs and
caches are resident in HBM before timing starts. `value` is decode-attention
throughput in GB/s of compressed cache read per second over the attention phase of a
step (all layers, every launch and gap included). Phase times come from HIP events on
the stream the library launches on. Each attention launch (the dominant kernel) is
also bracketed by its own events for the roofline figure.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mistral7b]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed-KV decode attn cache GB/s (% HBM peak); encode tokens/s"
HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="mistral7b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager-attention", action="store_true",
                    help="launch the per-layer attention calls one by one with HIP events "
                         "around each (default: the 32-layer sweep is captured once in a "
                         "HIP graph and replayed)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="approximate oracle CPU time (all cores together) of the baseline "
                         "sample")
    ap.add_argument("--no-triplet", action="store_true",
                    help="skip the triplet-codec sub-record")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (used to "
                         "scale rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes) and exit")
    return ap.parse_args()


def copy_calibration(mib):
    """A plain copy of known size: reads and writes exactly mib MiB once."""
    import torch
    n = mib * 1024 * 1024
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def attn_lds_bytes(d, group, bk, bv, mode):
    """LDS bytes of one decode-attention variant (the library's own layout: cos/sin
    tables, rotated query, flag word, then the score table and the waves' fp16 value
    rows, or the merge buffers; with a score table and matrix-core values the query
    lives in that union instead)."""
    p = d // 2
    nw = (12 if mode == 7 and d == 128 else 8) if mode & 3 == 3 else (12 if mode & 3 and group <= 4 else 8)
    hg = group // 4 if group > 4 else 1
    tab = {1: p * (1 << bk) * group * 4, 2: p * (1 << (bk - 1)) * group * 4}.get(mode & 3, 0)
    rows = nw * (hg * 4 * 64 + 64 * 16) * 2 if mode & 4 else 0
    qb = group * d * 4
    qu = tab > 0 and bool(mode & 4)
    merge = nw * group * (d + 2) * 4 + (qb if qu else 0)
    return (1 << bk) * 8 + (1 << bv) * 8 + (0 if qu else qb) + 16 + max(tab + rows, merge)


def attn_kernel_name(d, group, n_k, n_v):
    """Name of the attention-kernel instantiation the library launches for this shape:
    for up to four query heads per kv head the score table with the value sum on the
    matrix cores when both fit in 160 KiB of LDS (the half table, mode 6, for
    power-of-two n_k at three or four heads, else the full table, mode 5), else for key
    codes under 8 bits the score table with the vector value sum (mode 1 / 2) when it
    fits; otherwise matrix-core products for both (mode 7)."""
    bk, bv = (n_k - 1).bit_length(), (n_v - 1).bit_length()
    pow2 = n_k == 1 << bk
    cap = 160 * 1024
    mode = 7
    if group <= 4:
        tab = 2 if pow2 else 1
        full = attn_lds_bytes(d, group, bk, bv, 5) <= cap
        half = pow2 and attn_lds_bytes(d, group, bk, bv, 6) <= cap
        if full and (group <= 2 or not half):
            mode = 5
        elif half:
            mode = 6
        elif bk < 8 and attn_lds_bytes(d, group, bk, bv, tab) <= cap:
            mode = tab
    return f"attn_decode_kernel<{d}, {group}, {bk}, {bv}, {mode}>"


def attn_traffic(cfg):
    """Calibrated HBM bytes per attention launch from the committed rocprofv3 counter
    record, or None if the record is for another workload or the kernel source has
    changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"attn_decode_{cfg.name}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = open(os.path.join(ROOT, rec["kernel_source"]), "rb").read()
    if hashlib.sha256(src).hexdigest() != rec["source_sha256"]:
        return None
    total = 0.0
    for layer in range(cfg.layers):
        name = attn_kernel_name(cfg.d, cfg.group, *cfg.bins(layer))
        if name not in rec["per_kernel"]:
            return None
        total += rec["per_kernel"][name]["bytes"]
    return total / cfg.layers


def record_bytes(d, n_k, n_v, tokens):
    """Algorithmic compressed bytes of `tokens` token-heads (one record per token-head)."""
    import rotated_angle_quantization_amd as kvq
    return tokens * kvq.tile_bytes(d, n_k, n_v) // 64


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_slice(args):
    """One (layer, batch, kv head) slice of the oracle baseline: encode its K/V token
    sample, pack the codes into tiles, then decode attention for the G query heads of
    that kv head from the packed bytes (unpack + dequantise + attention). Runs in a
    worker process with one BLAS thread."""
    import time as _time

    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import codec as oc
    from oracle import layout as ol
    from synthetic import get, layer_kv, query

    name, layer, b, h, tokens = args
    cfg = get(name)
    n_k, n_v = cfg.bins(layer)
    d, g = cfg.d, cfg.group
    with threadpool_limits(limits=1):
        torch.set_num_threads(1)
        k, v = layer_kv(cfg, layer, "cpu", seq=tokens, batch=b + 1)
        q = query(cfg, layer, "cpu", batch=b + 1)
        xk = k[b, :, h].double().numpy()
        xv = v[b, :, h].double().numpy()
        qn = q[b:b + 1, h * g:(h + 1) * g].double().numpy()
        sg = oc.layer_signs(0, layer, d)
        t0 = _time.perf_counter()
        ek, ev = oc.encode_k(xk, sg, n_k), oc.encode_v(xv, sg, n_v)
        enc_s = _time.perf_counter() - t0
        tiles = []
        for t in range(tokens // 64):
            s = slice(t * 64, t * 64 + 64)
            tiles.append(ol.pack_tile(d, n_k, n_v, ek["angle"][s], ek["radius"][s],
                                      ek["scale"][s], ev["angle"][s], ev["radius"][s],
                                      ev["s_min"][s], ev["s_max"][s]))
        cache = np.stack(tiles)
        t0 = _time.perf_counter()
        u = ol.unpack_tiles(cache, d, n_k, n_v)
        u = {kk: vv.reshape((tokens,) + vv.shape[2:]) for kk, vv in u.items()}
        kh = oc.dequant_k(u["k_angle"], u["k_radius"], u["k_scale"], n_k, sg)
        vh = oc.dequant_v(u["v_angle"], u["v_radius"], u["v_smin"], u["v_smax"], n_v, sg)
        oc.attention(qn, kh[None, :, None], vh[None, :, None])
        att_s = _time.perf_counter() - t0
    return enc_s, att_s, cache.nbytes


def cpu_baseline(cfg, budget_s):
    """The oracle (as it stands) on the host cores, over a bounded sample of the parity
    subset of the workload: layers {0, first non-boosted, last}, batch entries
    {0, B - 1}, every kv head, the first `tokens` tokens of each sequence; one worker
    process per core over independent (layer, batch, kv head) slices. Encode and decode
    attention (from packed bytes) are timed separately inside each slice; throughputs
    are the slices' totals over the pool's wall time, scaled by the share of it each
    phase took."""
    import multiprocessing as mp

    cores = len(os.sched_getaffinity(0))
    layers = sorted({0, min(cfg.boosted_layers, cfg.layers - 1), cfg.layers - 1})
    batches = sorted({0, cfg.batch - 1})
    # budget_s of oracle CPU time in total: encode and decode attention together cost
    # the oracle about 25 us per token-head (d = 128, measured on these hosts)
    slices = len(layers) * len(batches) * cfg.hkv
    tokens = max(64, min(cfg.seq, int(budget_s / 25e-6 / slices)) // 64 * 64)
    work = [(cfg.name, layer, b, h, tokens) for layer in layers for b in batches
            for h in range(cfg.hkv)]
    t0 = time.perf_counter()
    with mp.get_context("spawn").Pool(processes=cores) as pool:
        res = pool.map(_oracle_slice, work)
    wall = time.perf_counter() - t0
    enc_s = sum(r[0] for r in res)
    att_s = sum(r[1] for r in res)
    nbytes = sum(r[2] for r in res)
    token_heads = tokens * len(work)
    # independent slices on `cores` workers: the pool's rate is the per-core rate times
    # the cores (input generation and process start-up are not the oracle's work)
    enc_wall = enc_s / cores
    att_wall = att_s / cores
    return {
        "value": nbytes / att_wall / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"{cfg.name}: layers {layers}, batch entries {batches}, all {cfg.hkv} kv "
                   f"heads, first {tokens} tokens each ({len(work)} slices, "
                   f"{token_heads} token-heads); oracle decode attention from packed bytes "
                   f"(unpack + dequant + attention for G={cfg.group} query heads) and "
                   f"oracle encode, one worker process per core; {enc_s + att_s:.1f} s of "
                   f"oracle CPU time in {wall:.1f} s wall (incl. worker start-up and input "
                   f"generation); rates = slice totals / (CPU time / cores)"),
        "decode_token_heads_per_s": token_heads / att_wall,
        "encode_token_heads_per_s": token_heads / enc_wall,
        "cpu_seconds": enc_s + att_s,
        "wall_s": wall,
    }


def decode_loop(kvq, cfg, descs, caches, ws, dev, iters=8):
    """Decode steps of a ragged batch on the resident caches: per layer, append one new
    token per sequence at its own slot (kvq_append), then attend with a length per
    sequence (kvq_attn_decode_varlen). Timed with HIP events on the library's stream."""
    import torch

    L, B, T, Hkv, Hq, d = cfg.layers, cfg.batch, cfg.seq, cfg.hkv, cfg.hq, cfg.d
    lens0 = [T - iters - (T // 3) * b // max(B - 1, 1) for b in range(B)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    new_k = torch.randn((B, Hkv, d), generator=gen, device=dev).half()
    new_v = torch.randn((B, Hkv, d), generator=gen, device=dev).half()
    qd = torch.randn((B, Hq, d), generator=gen, device=dev).half()
    pos = [torch.tensor(lens0, dtype=torch.int32, device=dev) + i for i in range(iters + 1)]
    out = torch.empty((B, Hq, d), dtype=torch.float16, device=dev)
    Ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def run(record):
        for i in range(iters):
            for layer in range(L):
                ev = (Ev(), Ev(), Ev()) if record is not None else None
                if ev:
                    ev[0].record()
                kvq.append(descs[layer], caches[layer], new_k, new_v, pos[i])
                if ev:
                    ev[1].record()
                kvq.attn_decode_varlen(descs[layer], caches[layer], qd, pos[i + 1], T,
                                       workspace=ws, out=out)
                if ev:
                    ev[2].record()
                    record.append((layer, i, ev))

    run(None)
    torch.cuda.synchronize()
    recs = []
    t0, t1 = Ev(), Ev()
    t0.record()
    run(recs)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    app_us = sum(ev[0].elapsed_time(ev[1]) for _, _, ev in recs) * 1e3 / len(recs)
    att_us = sum(ev[1].elapsed_time(ev[2]) for _, _, ev in recs) * 1e3 / len(recs)
    att_bytes = sum(record_bytes(d, *cfg.bins(layer), Hkv * (sum(lens0) + B * (i + 1)))
                    for layer, i, _ in recs) / len(recs)

    # the same steps with the append fused into the attention launch (rewriting the same
    # tokens into the same slots)
    def run_fused(record):
        for i in range(iters):
            for layer in range(L):
                ev = (Ev(), Ev()) if record is not None else None
                if ev:
                    ev[0].record()
                kvq.attn_decode_append(descs[layer], caches[layer], new_k, new_v, pos[i], qd, T,
                                       workspace=ws, out=out)
                if ev:
                    ev[1].record()
                    record.append(ev)

    run_fused(None)
    torch.cuda.synchronize()
    frecs = []
    f0, f1 = Ev(), Ev()
    f0.record()
    run_fused(frecs)
    f1.record()
    torch.cuda.synchronize()
    fused_ms = f0.elapsed_time(f1)
    fused_us = sum(e[0].elapsed_time(e[1]) for e in frecs) * 1e3 / len(frecs)
    return {
        "what": "per layer: kvq_append of one token per sequence at its own slot, then "
                "kvq_attn_decode_varlen over each sequence's length; fused: both in one "
                "kvq_attn_decode_append launch",
        "batch_lengths_start": lens0,
        "iterations": iters,
        "ms_per_token_all_layers": round(total_ms / iters, 4),
        "append_us_per_layer": round(app_us, 2),
        "attend_us_per_layer": round(att_us, 2),
        "attend_GBps": round(att_bytes / (att_us * 1e-6) / 1e9, 2),
        "fused_ms_per_token_all_layers": round(fused_ms / iters, 4),
        "fused_us_per_layer": round(fused_us, 2),
    }


def multi_query(kvq, cfg, descs, caches, dev, nqs=(4, 8), reps=5):
    """Multi-query attention (kvq_attn_multi) on the resident caches: NQ query tokens per
    sequence attending causally over the full context, every layer; HIP events."""
    import torch

    L, B, T, Hkv, Hq, d = cfg.layers, cfg.batch, cfg.seq, cfg.hkv, cfg.hq, cfg.d
    gen = torch.Generator(device=dev)
    gen.manual_seed(4321)
    Ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    res = {}
    for nq in nqs:
        if nq * (Hq // Hkv) > 32:
            continue
        q = torch.randn((B, nq, Hq, d), generator=gen, device=dev).half()
        out = torch.empty_like(q)
        ws = torch.zeros(max(kvq.attn_multi_workspace_bytes(dd, Hq, nq, T) for dd in descs),
                         dtype=torch.uint8, device=dev)

        def sweep():
            for layer in range(L):
                kvq.attn_multi(descs[layer], caches[layer], q, T, workspace=ws, out=out)

        sweep()
        torch.cuda.synchronize()
        e0, e1 = Ev(), Ev()
        e0.record()
        for _ in range(reps):
            sweep()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * L)
        nbytes = sum(record_bytes(d, *cfg.bins(x), B * Hkv * T) for x in range(L)) / L
        flops = 2 * 2 * B * Hq * nq * T * d  # scores and value sum, per layer
        res[f"nq{nq}"] = {
            "rows_per_kv_head": nq * (Hq // Hkv),
            "us_per_layer": round(us, 2),
            "cache_GBps": round(nbytes / (us * 1e-6) / 1e9, 2),
            "mfma_TFLOPs": round(flops / (us * 1e-6) / 1e12, 2),
            "mfma_frac_of_fp16_dense_peak": round(flops / (us * 1e-6) / 2.5e15, 4),
        }
    return res


def fixed_and_streaming(kvq, cfg, descs, caches, qs, dev, reps=16):
    """Per-launch time of decode attention on one 7/6-bit layer at a quarter and at the
    full sequence length (each launch over the same cache, replayed from a HIP graph of
    `reps` calls): the difference gives the streaming rate once a launch is under way,
    and the intercept the fixed cost of a launch (set-up, the split merge, launch and
    ramp), which no amount of streaming hides."""
    import torch

    layer = min(cfg.boosted_layers, cfg.layers - 1)
    desc, cache, q = descs[layer], caches[layer], qs[layer]
    T = cfg.seq
    out = torch.empty((cfg.batch, cfg.hq, cfg.d), dtype=torch.float16, device=dev)
    times = {}
    for L in (T // 4, T):
        ws = kvq.alloc_workspace(desc, cfg.hq, L, dev)
        kvq.attn_decode(desc, cache, q, L, workspace=ws, out=out)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for _ in range(reps):
                    kvq.attn_decode(desc, cache, q, L, workspace=ws, out=out)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times[L] = e0.elapsed_time(e1) * 1e3 / reps
    per_tok = record_bytes(cfg.d, *cfg.bins(layer), cfg.batch * cfg.hkv)  # bytes per token
    lo, hi = T // 4, T
    slope_us = (times[hi] - times[lo]) / (hi - lo)
    return {
        "layer": layer, "seq_lens": [lo, hi],
        "us_per_launch": [round(times[lo], 2), round(times[hi], 2)],
        "streaming_GBps": round(per_tok / (slope_us * 1e-6) / 1e9, 1),
        "fixed_us_per_launch": round(times[hi] - slope_us * hi, 2),
    }


def stream_probe(kvq, caches, dev, reps=3):
    """Read-only streaming probe (kvq_probe_read) over the same cache buffers the
    attention sweep reads, one launch per layer, HIP events around the sweep: the
    bandwidth a plain read of this memory reaches on this GPU (context for the
    roofline, no codec work). The sweep is also timed over the first quarter of each
    buffer: the two sweep times give the probe's own streaming rate (bytes over the
    difference in time) and its fixed time per launch, as `launch_breakdown` does for
    attention."""
    import torch

    sink = torch.zeros(256, dtype=torch.uint8, device=dev)

    def timed(bufs):
        def sweep():
            for c in bufs:
                kvq.probe_read(c, sink)
        sweep()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            sweep()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    quarter = [c[: (c.numel() // 4) // 16 * 16] for c in caches]
    nbytes = sum(c.numel() for c in caches)
    qbytes = sum(c.numel() for c in quarter)
    s, sq = timed(caches), timed(quarter)
    stream = (nbytes - qbytes) / (s - sq) if s > sq else float("nan")
    return {"GBps": round(nbytes / s / 1e9, 2), "bytes_per_sweep": nbytes,
            "launches_per_sweep": len(caches), "frac_of_peak": round(nbytes / s / 1e9 / HBM_PEAK_GBPS, 4),
            "quarter_GBps": round(qbytes / sq / 1e9, 2),
            "streaming_GBps": round(stream / 1e9, 1),
            "fixed_us_per_launch": round((s - nbytes / stream) / len(caches) * 1e6, 2)}


TRIPLET_BITS = (4, 2, 3)  # (bits per square coordinate, per triplet norm, per leftover)


def triplet_sub(kvq, cfg, ks, vs, qs, dev, reps=3):
    """The triplet (octahedral) codec on the same K/V and queries, every layer: encode
    all tokens, then one decode attention launch pair (splits + merge) per layer; HIP
    events around each sweep. Cache bytes per attention launch are the records read
    (both planes, whole 32-bit words)."""
    import torch

    L, B, T, Hkv, Hq, d = cfg.layers, cfg.batch, cfg.seq, cfg.hkv, cfg.hq, cfg.d
    descs = [kvq.make_tri_desc(d, Hkv, B, T, *TRIPLET_BITS, layer, 0) for layer in range(L)]
    table = kvq.tri_codebook_device(descs[0], dev)  # depends on (d, bits) only
    caches = [kvq.alloc_tri_cache(dd, dev) for dd in descs]
    ws = torch.empty(kvq.tri_attn_workspace_bytes(descs[0], Hq, T), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.float16, device=dev)
    Ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def enc():
        for layer in range(L):
            kvq.tri_encode(descs[layer], caches[layer], table, ks[layer], vs[layer], 0)

    def att():
        for layer in range(L):
            kvq.tri_attn_decode(descs[layer], caches[layer], table, qs[layer], T, workspace=ws,
                                out=out)

    enc()
    att()
    torch.cuda.synchronize()
    e = [Ev() for _ in range(3)]
    e[0].record()
    for _ in range(reps):
        enc()
    e[1].record()
    for _ in range(reps):
        att()
    e[2].record()
    torch.cuda.synchronize()
    enc_ms = e[0].elapsed_time(e[1]) / reps
    att_ms = e[1].elapsed_time(e[2]) / reps
    words = kvq.tri_record_words(descs[0])
    rec_bytes = B * Hkv * T * words * 4 * 2
    del caches
    torch.cuda.empty_cache()
    return {
        "what": "triplet codec (octahedral directions + Lloyd-Max norms): encode every "
                "layer, then decode attention every layer (split + merge launches)",
        "bits": {"dir": TRIPLET_BITS[0], "norm": TRIPLET_BITS[1], "rest": TRIPLET_BITS[2],
                 "record_words": words, "bits_per_element": words * 32 / d},
        "encode_tokens_per_s": round(B * T / (enc_ms * 1e-3), 1),
        "encode_ms_all_layers": round(enc_ms, 4),
        "attn_ms_all_layers": round(att_ms, 4),
        "attn_us_per_layer": round(att_ms * 1e3 / L, 2),
        "attn_cache_GBps": round(rec_bytes * L / (att_ms * 1e-3) / 1e9, 2),
        "attn_hbm_frac": round(rec_bytes * L / (att_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "bytes_per_launch": rec_bytes,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode "
              "(no sharding or collectives); use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return

    import torch

    import rotated_angle_quantization_amd as kvq
    from synthetic import get, layer_kv, query

    cfg = get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L, B, T, Hkv, Hq, d = cfg.layers, cfg.batch, cfg.seq, cfg.hkv, cfg.hq, cfg.d
    print(f"[bench] workload {cfg.name}: L={L} B={B} T={T} Hkv={Hkv} Hq={Hq} d={d}",
          file=sys.stderr, flush=True)

    descs, caches, ks, vs, qs = [], [], [], [], []
    for layer in range(L):
        n_k, n_v = cfg.bins(layer)
        desc = kvq.make_desc(d, Hkv, B, T, n_k, n_v, layer, 0)
        descs.append(desc)
        caches.append(kvq.alloc_cache(desc, dev))
        k, v = layer_kv(cfg, layer, dev)
        ks.append(k)
        vs.append(v)
        qs.append(query(cfg, layer, dev))
    ws_bytes = max(kvq.attn_workspace_bytes(dd, Hq, T) for dd in descs)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)  # zero-filled once, reused
    outs = torch.empty((B, Hq, d), dtype=torch.float16, device=dev)
    kd = torch.empty((B, T, Hkv, d), dtype=torch.float16, device=dev)
    vd = torch.empty_like(kd)
    torch.cuda.synchronize()
    cache_bytes_total = sum(c.numel() for c in caches)
    attn_bytes = sum(record_bytes(d, *cfg.bins(layer), B * Hkv * T) for layer in range(L))
    print(f"[bench] inputs ready: cache {cache_bytes_total / 1e9:.2f} GB "
          f"({attn_bytes / 1e9:.3f} GB algorithmic per attention sweep)", file=sys.stderr,
          flush=True)

    Ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def attention_sweep():
        for layer in range(L):
            kvq.attn_decode(descs[layer], caches[layer], qs[layer], T, workspace=ws, out=outs)

    graph = [None]  # the captured attention sweep, once captured

    def step(record):
        e = [Ev() for _ in range(4)]
        attn_ev = []
        e[0].record()
        for layer in range(L):
            kvq.encode(descs[layer], caches[layer], ks[layer], vs[layer], 0)
        e[1].record()
        if graph[0] is not None:
            graph[0].replay()
        else:
            for layer in range(L):
                ev = (Ev(), Ev())
                ev[0].record()
                kvq.attn_decode(descs[layer], caches[layer], qs[layer], T, workspace=ws,
                                out=outs)
                ev[1].record()
                attn_ev.append(ev)
        e[2].record()
        for layer in range(L):
            kvq.decode(descs[layer], caches[layer], 0, T, out=(kd, vd))
        e[3].record()
        if record is not None:
            record.append((e, attn_ev))

    # eager warm-up steps (the library's one-time set-up runs here), then the attention
    # sweep is captured; the last warm-up step already replays the graph
    for _ in range(args.warmup - (0 if args.eager_attention else 1)):
        step(None)
    torch.cuda.synchronize()
    if not args.eager_attention:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                attention_sweep()
        torch.cuda.synchronize()
        graph[0] = g
        if args.warmup > 0:
            step(None)
    torch.cuda.synchronize()
    recs = []
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    # the timed output (fp16, from the replayed graph, last layer) against an eager fp32
    # call on the same cache: the benchmarked configuration computes what is tested
    ref32 = kvq.attn_decode(descs[L - 1], caches[L - 1], qs[L - 1], T, out_dtype=torch.float32)
    torch.cuda.synchronize()
    diff = (outs.float() - ref32).norm(dim=-1) / ref32.norm(dim=-1).clamp_min(1e-30)
    timed_vs_fp32 = float(diff.max())
    loop = decode_loop(kvq, cfg, descs, caches, ws, dev)
    mq = multi_query(kvq, cfg, descs, caches, dev)
    probe = stream_probe(kvq, caches, dev)
    fixed = fixed_and_streaming(kvq, cfg, descs, caches, qs, dev)
    tri = None if args.no_triplet else triplet_sub(kvq, cfg, ks, vs, qs, dev)

    enc_ms = sum(e[0].elapsed_time(e[1]) for e, _ in recs) / args.steps
    att_ms = sum(e[1].elapsed_time(e[2]) for e, _ in recs) / args.steps
    deq_ms = sum(e[2].elapsed_time(e[3]) for e, _ in recs) / args.steps
    step_ms = sum(e[0].elapsed_time(e[3]) for e, _ in recs) / args.steps
    if graph[0] is None:
        launch_ms = [a.elapsed_time(b) for _, sp in recs for a, b in sp]
        launch_avg_ms = sum(launch_ms) / len(launch_ms)
    else:
        # graph replay: the sweep's time over its launches (the gaps between the kernels
        # inside the graph count as kernel time, so this errs low)
        launch_avg_ms = att_ms / L
    launch_bytes_avg = attn_bytes / L

    att_steps = sorted(e[1].elapsed_time(e[2]) for e, _ in recs)

    def pct(xs, f):  # nearest-rank percentile of a sorted list
        return xs[min(len(xs) - 1, max(0, int(round(f * (len(xs) - 1)))))]

    attn_gbps = attn_bytes / (att_ms * 1e-3) / 1e9
    achieved = launch_bytes_avg / (launch_avg_ms * 1e-3) / 1e9
    tokens = B * T
    result = {
        "metric": METRIC,
        "value": round(attn_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: {L} layers, batch {B}, seq {T}, {Hkv} kv heads, "
                         f"{Hq} query heads, d={d}, fp16 K/V, per-layer (n_K, n_V) = "
                         f"{sorted(set(cfg.bins(x) for x in range(L)))}"),
            "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)",
            "encode_decisions": "f64",
            "attention_arithmetic": "f32 (value products on the matrix cores: fp16 operands, "
                                    "fp32 sums)",
        },
        "hbm_frac": round(attn_gbps / HBM_PEAK_GBPS, 4),
        "encode_tokens_per_s": round(tokens / (enc_ms * 1e-3), 1),
        "encode_ms": round(enc_ms, 4),
        "attn_ms": round(att_ms, 4),
        "attn_ms_p10_median_p90": [round(pct(att_steps, f), 4) for f in (0.1, 0.5, 0.9)],
        "dequant_ms": round(deq_ms, 4),
        "dequant_out_GBps": round(2 * L * B * T * Hkv * d * 2 / (deq_ms * 1e-3) / 1e9, 2),
        "wall_s_timed": round(wall, 3),
        "timed_output_vs_eager_fp32_rel_l2": timed_vs_fp32,
        "decode_loop": loop,
        "multi_query": mq,
        "triplet": tri,
        "roofline": {
            "kernel": "attn_decode_kernel (kvq_attn_decode)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": attn_traffic(cfg),
            "avg_launch_ms": round(launch_avg_ms, 5),
            "timing": ("HIP events around each launch" if graph[0] is None else
                       f"HIP events around the replayed graph of the {L} launches, / {L}"),
            "bytes_per_launch": launch_bytes_avg,
            "stream_probe": probe,
            "achieved_over_probe": round(achieved / probe["GBps"], 4),
            "launch_breakdown": fixed,
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle CPU baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
