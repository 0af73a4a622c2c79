"""GPU parity of the triplet (octahedral) codec: the library's encode, dequantise and
decode attention (through the C ABI) against the float64 oracle in oracle/triplet.py.

Rules (the same bars as the angle codec's):
  codes      bit-exact. A square-coordinate, norm or leftover code may differ only where
             the oracle's float64 quantity lies within 1e-9 of a decision boundary (the
             two sides fit their Lloyd-Max tables independently and agree to ~1e-11).
             The fp16 scale bits always match.
  dequant    ||x_hat_gpu - x_hat_oracle|| <= 1e-3 ||x|| per (token, kv head), both decoding
             the same code bytes (fp16 outputs also get the fp16 subnormal half-spacing).
  attention  rel-L2 <= 2e-3 per (batch, query head) against the plain definition on the
             oracle's dequantisation of the same bytes.
"""

import numpy as np
import pytest
import torch

from oracle import codec as oc
from oracle import layout as ol
from oracle import triplet as ot
from parity import compare_attention, compare_dequant, note
from synthetic import get, layer_kv, query

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("rotated_angle_quantization_amd")

NEAR = 1e-9
_CODEBOOKS = {}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def codebook(d, bits) -> ot.Codebook:
    key = (d, *bits)
    if key not in _CODEBOOKS:
        _CODEBOOKS[key] = ot.Codebook(d, *bits)
    return _CODEBOOKS[key]


def plane_codes(got: dict, name: str) -> dict:
    return {"s_code": got[f"{name}_s_code"], "t_code": got[f"{name}_t_code"],
            "norm_code": got[f"{name}_norm_code"], "rest_code": got[f"{name}_rest_code"],
            "scale": got[f"{name}_scale"]}


def compare_tri_codes(got: dict, name: str, want: dict, cb: ot.Codebook) -> int:
    """Every code bit-exact except the near-boundary exemptions; returns their count."""
    g = plane_codes(got, name)
    np.testing.assert_array_equal(g["scale"], want["scale"], err_msg=f"{name} fp16 scale")
    exempt = 0
    for key, vals, bounds in (("s_code", want["st"][..., 0], cb.dir_bounds),
                              ("t_code", want["st"][..., 1], cb.dir_bounds),
                              ("norm_code", want["rho"], cb.norm_bounds),
                              ("rest_code", want["rest"], cb.rest_bounds)):
        bad = g[key] != want[key]
        if bad.any():
            near = ot.near_boundary(vals, bounds, NEAR)
            off = bad & ~near
            if off.any():
                i = np.argwhere(off)[:5]
                raise AssertionError(f"{name} {key} mismatch at {i.tolist()}: gpu "
                                     f"{g[key][off][:5]}, oracle {want[key][off][:5]}, "
                                     f"value {vals[off][:5]}")
            exempt += int(bad.sum())
    return exempt


def tri_full_check(dev, k, v, q, bits, layer=0, seed=0, capacity=None, seq_len=None, tag="",
                   fp16_dequant=True):
    bsz, t, hkv, d = k.shape
    capacity = capacity or t
    seq_len = seq_len or t
    note(f"[tri] {tag} B={bsz} T={t} Hkv={hkv} d={d} bits={bits} cap={capacity} "
         f"seq={seq_len}")
    desc = kvq.make_tri_desc(d, hkv, bsz, capacity, *bits, layer, seed)
    table = kvq.tri_codebook_device(desc, dev)
    cache = torch.zeros(kvq.tri_cache_bytes(desc), dtype=torch.uint8, device=dev)
    kvq.tri_encode(desc, cache, table, k, v, 0)
    torch.cuda.synchronize()
    got = ol.tri_unpack_cache(cache.cpu().numpy(), d, *bits, bsz, hkv, capacity, 0, t)
    cb = codebook(d, bits)
    sg = oc.layer_signs(seed, layer, d)
    xk, xv = np64(k), np64(v)
    exempt = 0
    for name, x in (("k", xk), ("v", xv)):
        exempt += compare_tri_codes(got, name, ot.encode(x, sg, cb), cb)
    kh_ref = ot.dequant(plane_codes(got, "k"), sg, cb)
    vh_ref = ot.dequant(plane_codes(got, "v"), sg, cb)
    stats = {"exempt": exempt}
    for dt in (torch.float32, torch.float16) if fp16_dequant else (torch.float32,):
        kh, vh = kvq.tri_decode(desc, cache, table, 0, t, out_dtype=dt)
        torch.cuda.synchronize()
        f16 = dt == torch.float16
        stats[f"k_{dt}"] = compare_dequant(np64(kh), kh_ref, xk, f"{tag} keys {dt}", fp16_out=f16)
        stats[f"v_{dt}"] = compare_dequant(np64(vh), vh_ref, xv, f"{tag} values {dt}",
                                           fp16_out=f16)
    if q is not None:
        ref = oc.attention(np64(q), kh_ref[:, :seq_len], vh_ref[:, :seq_len])
        out = kvq.tri_attn_decode(desc, cache, table, q, seq_len, out_dtype=torch.float32)
        out16 = kvq.tri_attn_decode(desc, cache, table, q, seq_len, out_dtype=torch.float16)
        torch.cuda.synchronize()
        stats["attn"] = compare_attention(np64(out), ref, f"{tag} attention")
        stats["attn_f16"] = compare_attention(np64(out16), ref, f"{tag} attention fp16 out")
    note(f"[tri] {tag} ok {stats}")
    return desc, table, cache


# ------------------------------------------------------------------ small, compared in full


@pytest.mark.parametrize("d,bits", [(d, b) for d in (64, 128)
                                    for b in ((4, 2, 3), (2, 2, 2), (3, 3, 3), (6, 6, 7),
                                              (1, 1, 1))] + [(128, (2, 1, 8))])
def test_codec_configurations(dev, d, bits):
    torch.manual_seed(d + 10 * sum(bits))
    hkv, bsz, t = 2, 2, 150
    k = (torch.randn(bsz, t, hkv, d, device=dev) * 2).half()
    v = torch.randn(bsz, t, hkv, d, device=dev).half()
    q = torch.randn(bsz, hkv * 4, d, device=dev).half()
    tri_full_check(dev, k, v, q, bits, layer=1, capacity=200, tag=f"d{d} bits{bits}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_attention_group_sizes(dev, d, g):
    torch.manual_seed(g * 10 + d)
    hkv, bsz, t = 2, 2, 333
    k = torch.randn(bsz, t, hkv, d, device=dev).half()
    v = torch.randn(bsz, t, hkv, d, device=dev).half()
    q = torch.randn(bsz, hkv * g, d, device=dev).half()
    tri_full_check(dev, k, v, q, (4, 2, 3), layer=3, capacity=400, tag=f"G{g} d{d}")


@pytest.mark.parametrize("seq_len", [1, 63, 64, 65, 999, 1000])
def test_attention_sequence_lengths(dev, seq_len):
    torch.manual_seed(seq_len)
    d, hkv, g = 128, 2, 4
    k = torch.randn(1, 1000, hkv, d, device=dev).half()
    v = torch.randn(1, 1000, hkv, d, device=dev).half()
    q = torch.randn(1, hkv * g, d, device=dev).half()
    tri_full_check(dev, k, v, q, (4, 2, 3), capacity=1000, seq_len=seq_len,
                   tag=f"seq {seq_len}")


def test_workload_inputs_and_float32(dev):
    """Keys with the outlier channels and per-token scales of the synthetic workloads, in
    fp16; then fp32 strided views with an fp32 query."""
    cfg = get("mistral7b")
    k, v = layer_kv(cfg, 6, dev, seq=300, batch=2)
    q = query(cfg, 6, dev, batch=2)
    tri_full_check(dev, k, v, q, (4, 2, 3), layer=6, capacity=320, tag="mistral-shaped")
    torch.manual_seed(5)
    big = torch.randn(2, 130, 3, 256, device=dev) * 2
    kf, vf = big[..., :128], big[..., 128:]
    assert kf.stride(2) == 256
    qf = torch.randn(2, 6, 128, device=dev)
    tri_full_check(dev, kf, vf, qf, (3, 3, 4), layer=2, tag="f32 strided")


def test_degenerate_vectors(dev):
    d = 128
    torch.manual_seed(11)
    k = torch.randn(1, 70, 2, d, device=dev)
    v = torch.randn(1, 70, 2, d, device=dev)
    k[0, 0] = 0.0      # zero vectors: scale 0, codes of the zero direction
    v[0, 1] = 0.0
    v[0, 2] = 1.0      # constant vector: all energy on one rotated coordinate
    sg = torch.tensor(oc.layer_signs(0, 0, d), device=dev, dtype=torch.float32)
    h = torch.tensor(oc.hadamard(d), device=dev, dtype=torch.float32)
    k[0, 3, 0] = sg * h[:, 9]      # rotates to one-hot coordinates: triplet on an axis
    k[0, 4, 1] = sg * h[:, 127]    # one-hot on the last leftover coordinate
    v[0, 5, 0] = sg * (h[:, 0] - h[:, 2])  # a triplet in the lower hemisphere
    k[0, 6] = 1e-6     # tiny: scale in the fp16 subnormal range
    k[0, 7] = 10000.0  # norm beyond the fp16 range: scale saturates at 65504
    q = torch.randn(1, 4, d, device=dev)
    _, _, cache = tri_full_check(dev, k.half(), v.half(), q.half(), (4, 2, 3),
                                 tag="degenerate", fp16_dequant=False)
    got = ol.tri_unpack_cache(cache.cpu().numpy(), d, 4, 2, 3, 1, 2, 70, 0, 70)
    assert got["k_scale"][0, 0, 0] == 0.0
    assert got["k_scale"][0, 7, 0] == 65504.0


def test_chunked_encode_equals_one_shot(dev):
    rng = np.random.default_rng(3)
    cfg = get("mistral7b")
    k, v = layer_kv(cfg, 5, dev, seq=700, batch=2)
    bits = (4, 2, 3)
    desc = kvq.make_tri_desc(128, cfg.hkv, 2, 704, *bits, 5, 0)
    table = kvq.tri_codebook_device(desc, dev)
    one = torch.zeros(kvq.tri_cache_bytes(desc), dtype=torch.uint8, device=dev)
    kvq.tri_encode(desc, one, table, k, v, 0)
    for trial in range(2):
        cuts = np.sort(rng.choice(np.arange(1, 700), size=int(rng.integers(3, 10)),
                                  replace=False))
        edges = [0, *cuts.tolist(), 700]
        chunked = torch.zeros_like(one)
        for lo, hi in zip(edges[:-1], edges[1:]):
            kvq.tri_encode(desc, chunked, table, k[:, lo:hi], v[:, lo:hi], lo)
        torch.cuda.synchronize()
        assert torch.equal(one, chunked), (trial, edges)
    # appends write only their own slots: a garbage-filled cache ends with the same codes
    garbage = torch.randint(0, 256, one.shape, dtype=torch.uint8, device=dev)
    for j in range(0, 130):
        kvq.tri_encode(desc, garbage, table, k[:, j:j + 1], v[:, j:j + 1], j)
    torch.cuda.synchronize()
    a = ol.tri_unpack_cache(garbage.cpu().numpy(), 128, *bits, 2, cfg.hkv, 704, 0, 130)
    r = ol.tri_unpack_cache(one.cpu().numpy(), 128, *bits, 2, cfg.hkv, 704, 0, 130)
    for key in r:
        np.testing.assert_array_equal(a[key], r[key], err_msg=key)


def test_attention_workspace_reuse_and_scale(dev):
    cfg = get("mistral7b")
    k, v = layer_kv(cfg, 9, dev, seq=1500, batch=2)
    q = query(cfg, 9, dev, batch=2)
    bits = (4, 2, 3)
    desc = kvq.make_tri_desc(128, cfg.hkv, 2, 1536, *bits, 9, 0)
    table = kvq.tri_codebook_device(desc, dev)
    cache = kvq.alloc_tri_cache(desc, dev)
    kvq.tri_encode(desc, cache, table, k, v, 0)
    lens = [1500, 600, 64, 1000]
    fresh = [kvq.tri_attn_decode(desc, cache, table, q, n) for n in lens]
    ws = torch.full((kvq.tri_attn_workspace_bytes(desc, cfg.hq, 1500),), 255,
                    dtype=torch.uint8, device=dev)
    for n, ref in zip(lens, fresh):
        got = kvq.tri_attn_decode(desc, cache, table, q, n, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), n
    out = kvq.tri_attn_decode(desc, cache, table, q, 600, softmax_scale=0.05,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    cb = codebook(128, bits)
    sg = oc.layer_signs(0, 9, 128)
    got = ol.tri_unpack_cache(cache.cpu().numpy(), 128, *bits, 2, cfg.hkv, 1536, 0, 600)
    kh = ot.dequant(plane_codes(got, "k"), sg, cb)
    vh = ot.dequant(plane_codes(got, "v"), sg, cb)
    compare_attention(np64(out), oc.attention(np64(q), kh, vh, scale=0.05), "scale 0.05")


# ------------------------------------------------------------------ full size, sampled


def test_mistral7b_full_size_sampled(dev):
    """The Mistral-7B-shaped layer (B 4, 32768 tokens, 8 KV heads, 32 query heads, d 128)
    at 3.5 bits per element, in the launch configuration the benchmark times: codes on
    sampled tiles, attention on sampled (batch, query head) rows over the full sequence."""
    cfg = get("mistral7b")
    bits = (4, 2, 3)
    layer = 4
    d, bsz, t, hkv = cfg.d, cfg.batch, cfg.seq, cfg.hkv
    k, v = layer_kv(cfg, layer, dev)
    q = query(cfg, layer, dev)
    desc = kvq.make_tri_desc(d, hkv, bsz, t, *bits, layer, 0)
    table = kvq.tri_codebook_device(desc, dev)
    cache = kvq.alloc_tri_cache(desc, dev)
    kvq.tri_encode(desc, cache, table, k, v, 0)
    out = kvq.tri_attn_decode(desc, cache, table, q, t, out_dtype=torch.float32)
    out16 = kvq.tri_attn_decode(desc, cache, table, q, t, out_dtype=torch.float16)
    torch.cuda.synchronize()
    cb = codebook(d, bits)
    sg = oc.layer_signs(0, layer, d)
    rng = np.random.default_rng(23)
    tiles_per_seq = t // 64
    tb = kvq.tri_tile_bytes(desc)
    cache4 = cache.view(bsz, hkv, tiles_per_seq, tb)
    for b, h in {(0, 0), (bsz - 1, hkv - 1), (int(rng.integers(bsz)), int(rng.integers(hkv)))}:
        tiles = sorted({0, tiles_per_seq - 1, *rng.integers(0, tiles_per_seq, 5).tolist()})
        for tile in tiles:
            got = ol.tri_unpack_cache(cache4[b, h, tile].cpu().numpy(), d, *bits, 1, 1, 64, 0,
                                      64)
            xs = slice(tile * 64, tile * 64 + 64)
            for name, x in (("k", np64(k[b:b + 1, xs, h:h + 1])),
                            ("v", np64(v[b:b + 1, xs, h:h + 1]))):
                compare_tri_codes(got, name, ot.encode(x, sg, cb), cb)
    worst = worst16 = 0.0
    for _ in range(2):
        b, hq = int(rng.integers(bsz)), int(rng.integers(cfg.hq))
        h = hq // cfg.group
        got = ol.tri_unpack_cache(cache4[b, h].cpu().numpy(), d, *bits, 1, 1, t, 0, t)
        kh = ot.dequant(plane_codes(got, "k"), sg, cb)
        vh = ot.dequant(plane_codes(got, "v"), sg, cb)
        ref = oc.attention(np64(q[b:b + 1, hq:hq + 1]), kh, vh)
        worst = max(worst, compare_attention(np64(out[b:b + 1, hq:hq + 1]), ref, f"b{b} h{hq}"))
        worst16 = max(worst16, compare_attention(np64(out16[b:b + 1, hq:hq + 1]), ref,
                                                 f"b{b} h{hq} fp16 out"))
    note(f"[tri sampled] ok, attention worst rel {worst:.2e} (fp16 out {worst16:.2e})")
    del k, v, cache
    torch.cuda.empty_cache()


def test_long_sequence_many_splits(dev):
    """One 32768-token sequence over eight kv heads: 128 splits per (batch, kv head), so
    the merge's lane-parallel pass over the splits' (max, sum) runs more than one round
    of 64 and its accumulator loop several rounds of sixteen. Attention on sampled query
    heads against the oracle's dequantisation of the same bytes."""
    cfg = get("llama3_8b_long")
    bits = (4, 2, 3)
    layer, t = 2, 32768
    d, hkv = cfg.d, cfg.hkv
    k, v = layer_kv(cfg, layer, dev, seq=t, batch=1)
    q = query(cfg, layer, dev)
    desc = kvq.make_tri_desc(d, hkv, 1, t, *bits, layer, 0)
    table = kvq.tri_codebook_device(desc, dev)
    cache = kvq.alloc_tri_cache(desc, dev)
    kvq.tri_encode(desc, cache, table, k, v, 0)
    out = kvq.tri_attn_decode(desc, cache, table, q, t, out_dtype=torch.float32)
    torch.cuda.synchronize()
    cb = codebook(d, bits)
    sg = oc.layer_signs(0, layer, d)
    cache3 = cache.view(hkv, t // 64, kvq.tri_tile_bytes(desc))
    rng = np.random.default_rng(41)
    worst = 0.0
    for hq in sorted({0, cfg.hq - 1, int(rng.integers(cfg.hq))}):
        h = hq // cfg.group
        got = ol.tri_unpack_cache(cache3[h].cpu().numpy(), d, *bits, 1, 1, t, 0, t)
        kh = ot.dequant(plane_codes(got, "k"), sg, cb)
        vh = ot.dequant(plane_codes(got, "v"), sg, cb)
        ref = oc.attention(np64(q[:, hq:hq + 1]), kh, vh)
        worst = max(worst, compare_attention(np64(out[:, hq:hq + 1]), ref, f"h{hq}"))
    note(f"[tri long] ok, attention worst rel {worst:.2e}")
    del k, v, cache
    torch.cuda.empty_cache()
