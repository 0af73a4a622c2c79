"""GPU parity: the HIP library (through its C ABI) against the oracle on the same seeded
inputs. Small workloads are compared in full; the full-size workloads run in the same
launch configuration the benchmark uses and are compared on sampled tiles and heads."""

import math

import numpy as np
import pytest
import torch

from oracle import codec as oc
from parity import (compare_attention, compare_codes, compare_dequant, note, oracle_dequant,
                    oracle_encode, unpack)
from synthetic import get, layer_kv, query

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("rotated_angle_quantization_amd")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def run_full_check(dev, k, v, q, d, n_k, n_v, layer=0, seed=0, capacity=None, seq_len=None,
                   attn_checks=True, tag="", fp16_dequant=True):
    """Encode k/v [B, T, Hkv, d] on the GPU, then compare every code, every dequantised
    vector and every attention output against the oracle."""
    bsz, t, hkv, _ = k.shape
    capacity = capacity or t
    seq_len = seq_len or t
    note(f"[full] {tag} B={bsz} T={t} Hkv={hkv} d={d} n=({n_k},{n_v}) layer={layer}")
    desc = kvq.make_desc(d, hkv, bsz, capacity, n_k, n_v, layer, seed)
    cache = torch.zeros(kvq.cache_bytes(desc), dtype=torch.uint8, device=dev)
    kvq.encode(desc, cache, k, v, 0)
    torch.cuda.synchronize()
    got = unpack(cache.cpu().numpy(), d, n_k, n_v, bsz, hkv, capacity, 0, t)
    sg = oc.layer_signs(seed, layer, d)
    xk, xv = np64(k), np64(v)
    ek, ev = oracle_encode(xk, xv, sg, n_k, n_v)
    stats = compare_codes(got, ek, ev)
    # dequant: both sides decode the same bytes
    kh_ref, vh_ref = oracle_dequant(got, sg, n_k, n_v)
    for dt in (torch.float32, torch.float16) if fp16_dequant else (torch.float32,):
        kh, vh = kvq.decode(desc, cache, 0, t, out_dtype=dt)
        torch.cuda.synchronize()
        f16 = dt == torch.float16
        compare_dequant(np64(kh), kh_ref, xk, f"{tag} keys {dt}", fp16_out=f16)
        compare_dequant(np64(vh), vh_ref, xv, f"{tag} values {dt}", fp16_out=f16)
    if attn_checks and q is not None:
        ref = oc.attention(np64(q), kh_ref[:, :seq_len], vh_ref[:, :seq_len])
        # both output types; fp16 is the one the benchmark times (its rounding adds at
        # most 2^-11 relative per element, inside the 2e-3 bound)
        out16 = kvq.attn_decode(desc, cache, q, seq_len, out_dtype=torch.float16)
        out = kvq.attn_decode(desc, cache, q, seq_len, out_dtype=torch.float32)
        torch.cuda.synchronize()
        stats["attn_rel"] = compare_attention(np64(out), ref, f"{tag} attention")
        stats["attn_rel_f16out"] = compare_attention(np64(out16), ref, f"{tag} attention fp16 out")
        # end to end against an independent oracle encode (reported, not gated)
        kh_o = oc.dequant_k(ek["angle"], ek["radius"], ek["scale"], n_k, sg)
        vh_o = oc.dequant_v(ev["angle"], ev["radius"], ev["s_min"], ev["s_max"], n_v, sg)
        ref_o = oc.attention(np64(q), kh_o[:, :seq_len], vh_o[:, :seq_len])
        e2e = np.linalg.norm(np64(out) - ref_o, axis=-1) / np.linalg.norm(ref_o, axis=-1)
        stats["attn_rel_e2e"] = float(e2e.max())
    note(f"[full] {tag} ok {stats}")
    return desc, cache, stats


# ----------------------------------------------------------------- small workloads in full


def test_tiny_workload_full(dev):
    cfg = get("tiny")
    k, v = layer_kv(cfg, 0, dev)
    q = query(cfg, 0, dev)
    run_full_check(dev, k, v, q, 64, 128, 64, tag="tiny")


@pytest.mark.parametrize("layer", [0, 21])
def test_tinyllama_layer_full(dev, layer):
    cfg = get("tinyllama")
    k, v = layer_kv(cfg, layer, dev)
    q = query(cfg, layer, dev)
    run_full_check(dev, k, v, q, 64, 128, 64, layer=layer, tag=f"tinyllama L{layer}")


# ----------------------------------------------------------------- full sizes, sampled


def sampled_check(dev, name, layer, n_heads_attn=2, n_tiles=6, seed=0):
    cfg = get(name)
    n_k, n_v = cfg.bins(layer)
    d, bsz, t, hkv = cfg.d, cfg.batch, cfg.seq, cfg.hkv
    note(f"[sampled] {name} layer {layer} n=({n_k},{n_v}) B={bsz} T={t} Hkv={hkv}")
    k, v = layer_kv(cfg, layer, dev)
    q = query(cfg, layer, dev)
    desc = kvq.make_desc(d, hkv, bsz, t, n_k, n_v, layer, seed)
    cache = kvq.alloc_cache(desc, dev)
    kvq.encode(desc, cache, k, v, 0)
    out = kvq.attn_decode(desc, cache, q, t, out_dtype=torch.float32)
    out16 = kvq.attn_decode(desc, cache, q, t, out_dtype=torch.float16)  # as benchmarked
    torch.cuda.synchronize()
    sg = oc.layer_signs(seed, layer, d)
    rng = np.random.default_rng(layer + 17)
    tiles_per_seq = t // 64
    tb = kvq.tile_bytes(d, n_k, n_v)
    cache4 = cache.view(bsz, hkv, tiles_per_seq, tb)
    # codes and dequant on sampled tiles (first, last and random tiles)
    for b, h in {(0, 0), (bsz - 1, hkv - 1), (int(rng.integers(bsz)), int(rng.integers(hkv)))}:
        tiles = sorted({0, tiles_per_seq - 1, *rng.integers(0, tiles_per_seq, n_tiles).tolist()})
        for tile in tiles:
            got = unpack(cache4[b, h, tile].cpu().numpy(), d, n_k, n_v, 1, 1, 64, 0, 64)
            xs = slice(tile * 64, tile * 64 + 64)
            xk = np64(k[b:b + 1, xs, h:h + 1])
            xv = np64(v[b:b + 1, xs, h:h + 1])
            ek, ev = oracle_encode(xk, xv, sg, n_k, n_v)
            compare_codes(got, ek, ev)
            kh, vh = kvq.decode(desc, cache, tile * 64, 64, out_dtype=torch.float32)
            kh_ref, vh_ref = oracle_dequant(got, sg, n_k, n_v)
            compare_dequant(np64(kh[b:b + 1, :, h:h + 1]), kh_ref, xk, f"{name} keys")
            compare_dequant(np64(vh[b:b + 1, :, h:h + 1]), vh_ref, xv, f"{name} values")
    # attention on sampled (b, query head) over the full sequence
    worst = worst16 = 0.0
    g = cfg.group
    for _ in range(n_heads_attn):
        b, hq = int(rng.integers(bsz)), int(rng.integers(cfg.hq))
        h = hq // g
        got = unpack(cache4[b, h].cpu().numpy(), d, n_k, n_v, 1, 1, t, 0, t)
        kh_ref, vh_ref = oracle_dequant(got, sg, n_k, n_v)
        ref = oc.attention(np64(q[b:b + 1, hq:hq + 1]), kh_ref, vh_ref)
        worst = max(worst, compare_attention(np64(out[b:b + 1, hq:hq + 1]), ref,
                                             f"{name} b{b} h{hq}"))
        worst16 = max(worst16, compare_attention(np64(out16[b:b + 1, hq:hq + 1]), ref,
                                                 f"{name} b{b} h{hq} fp16 out"))
    note(f"[sampled] {name} layer {layer} ok, attention worst rel {worst:.2e} "
         f"(fp16 out {worst16:.2e})")
    del k, v, cache
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layer", [0, 4])
def test_mistral7b_full_size_sampled(dev, layer):
    sampled_check(dev, "mistral7b", layer)


def test_llama3_8b_long_full_size_sampled(dev):
    sampled_check(dev, "llama3_8b_long", 7)


@pytest.mark.parametrize("layer", [3, 40])
def test_llama70b_batch_full_size_sampled(dev, layer):
    sampled_check(dev, "llama70b_batch", layer)


# ----------------------------------------------------------------- kernel variants


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_attention_group_sizes(dev, d, g):
    cfg = get("mistral7b")
    torch.manual_seed(g * 10 + d)
    hkv, bsz, t = 2, 2, 333
    k = torch.randn(bsz, t, hkv, d, device=dev).half()
    v = torch.randn(bsz, t, hkv, d, device=dev).half()
    q = torch.randn(bsz, hkv * g, d, device=dev).half()
    del cfg
    run_full_check(dev, k, v, q, d, 128, 64, layer=3, capacity=400, tag=f"G{g} d{d}")


@pytest.mark.parametrize("nk", [33, 64, 100, 128, 200, 256])
@pytest.mark.parametrize("nv", [40, 64, 128, 256])
def test_attention_code_widths(dev, nk, nv):
    torch.manual_seed(nk + nv)
    d = 128 if (nk + nv) % 2 == 0 else 64
    k = (torch.randn(1, 150, 2, d, device=dev) * 3).half()
    v = torch.randn(1, 150, 2, d, device=dev).half()
    q = torch.randn(1, 8, d, device=dev).half()
    run_full_check(dev, k, v, q, d, nk, nv, layer=1, tag=f"n=({nk},{nv}) d{d}")


@pytest.mark.parametrize("nk,nv,d,g", [(2, 3, 128, 4), (5, 17, 64, 2), (16, 8, 128, 8),
                                        (31, 32, 128, 1), (32, 64, 128, 4), (200, 5, 64, 4)])
def test_small_codebooks(dev, nk, nv, d, g):
    """Codebooks of at most 32 bins (1- to 5-bit codes, K only, V only or both): codes,
    dequantisation and attention (through the 6-bit widened copy) against the oracle,
    over 100 tokens (a ragged second tile)."""
    torch.manual_seed(nk * nv + d)
    k = torch.randn(1, 100, 3, d, device=dev).half()
    v = torch.randn(1, 100, 3, d, device=dev).half()
    q = torch.randn(1, 3 * g, d, device=dev).half()
    run_full_check(dev, k, v, q, d, nk, nv, tag=f"n=({nk},{nv}) d={d} G={g}")


def test_small_codebooks_varlen_static_and_paged(dev):
    """Narrow codebooks through the ragged-batch and allocation-free entry points (against
    the oracle per sequence), and the paged form's UNSUPPORTED."""
    d, hkv, g, nk, nv, t = 128, 2, 4, 24, 12, 200
    torch.manual_seed(5)
    k = torch.randn(3, t, hkv, d, device=dev).half()
    v = torch.randn(3, t, hkv, d, device=dev).half()
    q = torch.randn(3, hkv * g, d, device=dev).half()
    desc = kvq.make_desc(d, hkv, 3, t, nk, nv)
    cache = torch.zeros(kvq.cache_bytes(desc), dtype=torch.uint8, device=dev)
    kvq.encode(desc, cache, k, v, 0)
    torch.cuda.synchronize()
    got = unpack(cache.cpu().numpy(), d, nk, nv, 3, hkv, t, 0, t)
    kh, vh = oracle_dequant(got, oc.layer_signs(0, 0, d), nk, nv)
    lens = [200, 65, 1]
    out = kvq.attn_decode_varlen(desc, cache, q, torch.tensor(lens, dtype=torch.int32,
                                                              device=dev), t,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        ref = oc.attention(np64(q[b:b + 1]), kh[b:b + 1, :n], vh[b:b + 1, :n])
        compare_attention(np64(out[b:b + 1]), ref, f"narrow varlen b={b} len={n}")
    st = kvq.attn_decode_static(desc, cache, q, 150, out_dtype=torch.float32)
    torch.cuda.synchronize()
    compare_attention(np64(st), oc.attention(np64(q), kh[:, :150], vh[:, :150]),
                      "narrow static 150")
    pages = torch.arange(12, dtype=torch.int32, device=dev).reshape(3, 4)
    pool = torch.zeros(kvq.paged_pool_bytes(desc, 12), dtype=torch.uint8, device=dev)
    with pytest.raises(kvq.KvqError, match="UNSUPPORTED"):
        kvq.attn_decode_paged(desc, pool, kvq.make_paging(pages, 12), q, t,
                              seq_lens=torch.tensor(lens, dtype=torch.int32, device=dev))


@pytest.mark.parametrize("seq_len", [1, 63, 64, 65, 999, 1000])
def test_attention_sequence_lengths(dev, seq_len):
    torch.manual_seed(seq_len)
    d, hkv, g = 128, 2, 4
    k = torch.randn(1, 1000, hkv, d, device=dev).half()
    v = torch.randn(1, 1000, hkv, d, device=dev).half()
    q = torch.randn(1, hkv * g, d, device=dev).half()
    run_full_check(dev, k, v, q, d, 128, 64, capacity=1000, seq_len=seq_len,
                   tag=f"seq {seq_len}")


def test_float32_inputs_d128_and_strided_views(dev):
    torch.manual_seed(5)
    big = torch.randn(2, 130, 3, 256, device=dev) * 2
    k, v = big[..., :128], big[..., 128:]
    assert k.stride(2) == 256
    q = torch.randn(2, 6, 128, device=dev)
    run_full_check(dev, k, v, q, 128, 128, 64, layer=2, tag="f32 strided")
    kh, vh = big.half()[..., :128], big.half()[..., 128:]
    run_full_check(dev, kh, vh, q.half(), 128, 256, 256, layer=2, tag="f16 strided")


def test_degenerate_vectors(dev):
    d = 128
    k = torch.randn(1, 70, 2, d, device=dev)
    v = torch.randn(1, 70, 2, d, device=dev)
    k[0, 0] = 0.0  # zero key: scale 0, all codes 0
    v[0, 1] = 0.0  # zero value: s_max = 0 <= s_min, all codes 0
    v[0, 2] = 1.0  # constant value vector: rotated energy on one coordinate
    k[0, 3] = 30000.0  # key whose largest rotated radius exceeds the fp16 range
    k[0, 4] = 1e-6  # tiny radii below the fp16 normal range
    v[0, 5] = 3e-6
    sg = torch.tensor(oc.layer_signs(0, 0, d), device=dev, dtype=torch.float32)
    h = torch.tensor(oc.hadamard(d), device=dev, dtype=torch.float32)
    k[0, 6, 0] = sg * h[:, 9]  # rotates to a one-hot: angles on bin centres
    # fp16 inputs near the top of the range: one-hot rotations whose radius (6000
    # sqrt(128) = 67,882) is past the fp16 range, so the key scale and s_max are clipped
    # at 65504 and the level estimates run past the last level (clamped on both sides),
    # while the reconstructed elements (65504 / sqrt(128)) stay inside fp16; and +-4000
    # sign vectors (large radii in every pair)
    k[0, 7, 0] = sg * h[:, 5] * 6000.0
    v[0, 7, 1] = sg * h[:, 12] * 6000.0
    k[0, 8] = 4000.0 * torch.sign(torch.randn(2, d, device=dev))
    v[0, 8] = 4000.0 * torch.sign(torch.randn(2, d, device=dev))
    q = torch.randn(1, 4, d, device=dev)
    run_full_check(dev, k.half(), v.half(), q.half(), d, 128, 64, tag="degenerate")


def test_degenerate_vectors_fp32_extremes(dev):
    """fp32 inputs at the ends of the range: pairs whose fp32 values are subnormal or
    round to zero (the angle estimate would divide by a flushed reciprocal) and pairs
    that overflow fp32 after the rotation get the codes of the binary64 definition."""
    d = 128
    torch.manual_seed(9)
    k = torch.randn(1, 70, 2, d, device=dev)
    v = torch.randn(1, 70, 2, d, device=dev)
    sg = torch.tensor(oc.layer_signs(0, 0, d), device=dev, dtype=torch.float32)
    h = torch.tensor(oc.hadamard(d), device=dev, dtype=torch.float32)
    k[0, 0, 0] = sg * h[:, 9] * 1e-41   # rotates to (0, tiny) in pair 4: code n/4
    k[0, 1, 0] = sg * h[:, 8] * 1e-41   # (tiny, 0): code 0
    v[0, 0, 1] = sg * h[:, 11] * 1e-40
    k[0, 2] = torch.randn(2, d, device=dev) * 1e-39  # subnormal fp32 inputs
    v[0, 3] = torch.randn(2, d, device=dev) * 1e-38
    k[0, 4] = torch.randn(2, d, device=dev) * 1e-30
    k[0, 5, 0] = sg * h[:, 3] * 1e38    # rotates to 1.1e39 > the fp32 range
    v[0, 5, 1] = sg * h[:, 6] * 1e38
    k[0, 6] = torch.randn(2, d, device=dev) * 2e37
    v[0, 7] = torch.randn(2, d, device=dev) * 2e37
    q = torch.randn(1, 4, d, device=dev)
    # dequantised elements of the saturated vectors exceed the fp16 range (a radius of
    # 65504 in every pair), so only the fp32 output is compared for them
    _, cache, _ = run_full_check(dev, k, v, q, d, 128, 64, tag="fp32 extremes",
                                 fp16_dequant=False)
    got = unpack(cache.cpu().numpy(), d, 128, 64, 1, 2, 70, 0, 70)
    assert got["k_angle"][0, 0, 0, 4] == 32 and got["k_angle"][0, 1, 0, 4] == 0
    assert got["v_angle"][0, 0, 1, 5] == 16


# ----------------------------------------------------------------- online / determinism


@pytest.mark.parametrize("d,nk,nv", [(128, 128, 64), (128, 100, 100), (64, 256, 33),
                                     (128, 200, 128)])
def test_random_chunkings_equal_one_shot(dev, d, nk, nv):
    """Encoding a sequence in seeded random chunks (partial tiles at both ends, value words
    of odd widths shared across chunk edges) leaves the one-shot bytes."""
    rng = np.random.default_rng(d + nk + nv)
    cfg = get("mistral7b")
    k, v = layer_kv(cfg, 5, dev, seq=700, batch=2)
    if d == 64:
        k, v = k[..., :64].contiguous(), v[..., :64].contiguous()
    desc = kvq.make_desc(d, cfg.hkv, 2, 704, nk, nv, 5, 0)
    one = torch.zeros(kvq.cache_bytes(desc), dtype=torch.uint8, device=dev)
    kvq.encode(desc, one, k, v, 0)
    for trial in range(3):
        cuts = np.sort(rng.choice(np.arange(1, 700), size=int(rng.integers(3, 12)), replace=False))
        edges = [0, *cuts.tolist(), 700]
        chunked = torch.zeros_like(one)
        for lo, hi in zip(edges[:-1], edges[1:]):
            kvq.encode(desc, chunked, k[:, lo:hi], v[:, lo:hi], lo)
        torch.cuda.synchronize()
        assert torch.equal(one, chunked), (trial, edges)


def test_chunked_append_equals_one_shot(dev):
    cfg = get("tinyllama")
    k, v = layer_kv(cfg, 2, dev, seq=300)
    desc = kvq.make_desc(64, cfg.hkv, 1, 320, 128, 64, 2, 0)
    one = torch.zeros(kvq.cache_bytes(desc), dtype=torch.uint8, device=dev)
    kvq.encode(desc, one, k, v, 0)
    chunked = torch.zeros_like(one)
    for lo, hi in [(0, 1), (1, 70), (70, 128), (128, 129), (129, 250), (250, 300)]:
        kvq.encode(desc, chunked, k[:, lo:hi], v[:, lo:hi], lo)
    torch.cuda.synchronize()
    assert torch.equal(one, chunked)
    # token-by-token appends through a tile boundary, onto a garbage-filled cache
    garbage = torch.randint(0, 256, one.shape, dtype=torch.uint8, device=dev)
    kvq.encode(desc, garbage, k[:, :60], v[:, :60], 0)
    for j in range(60, 130):
        kvq.encode(desc, garbage, k[:, j:j + 1], v[:, j:j + 1], j)
    ref = torch.zeros_like(one)
    kvq.encode(desc, ref, k[:, :130], v[:, :130], 0)
    torch.cuda.synchronize()
    a = unpack(garbage.cpu().numpy(), 64, 128, 64, 1, cfg.hkv, 320, 0, 130)
    r = unpack(ref.cpu().numpy(), 64, 128, 64, 1, cfg.hkv, 320, 0, 130)
    for key in r:
        np.testing.assert_array_equal(a[key], r[key], err_msg=key)


def test_deterministic_across_runs_and_seeds(dev):
    cfg = get("mistral7b")
    k, v = layer_kv(cfg, 5, dev, seq=512, batch=2)
    desc = kvq.make_desc(128, cfg.hkv, 2, 512, 128, 64, 5, 0)
    c1 = kvq.alloc_cache(desc, dev)
    c2 = kvq.alloc_cache(desc, dev)
    kvq.encode(desc, c1, k, v, 0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        kvq.encode(desc, c2, k, v, 0)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    other = kvq.make_desc(128, cfg.hkv, 2, 512, 128, 64, 5, 1)
    c3 = kvq.alloc_cache(other, dev)
    kvq.encode(other, c3, k, v, 0)
    torch.cuda.synchronize()
    assert not torch.equal(c1, c3)
    q = query(cfg, 5, dev, batch=2)
    o1 = kvq.attn_decode(desc, c1, q, 512)
    o2 = kvq.attn_decode(desc, c1, q, 512)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_attention_workspace_reuse_and_explicit_scale(dev):
    """One zero-filled workspace serves a sequence of calls of different shapes and
    split counts: results equal those with fresh workspaces, and the split counters at
    its start are back at zero afterwards."""
    cfg = get("mistral7b")
    k, v = layer_kv(cfg, 9, dev, seq=2048, batch=2)
    q = query(cfg, 9, dev, batch=2)
    desc = kvq.make_desc(128, cfg.hkv, 2, 2048, 128, 64, 9, 0)
    cache = kvq.alloc_cache(desc, dev)
    kvq.encode(desc, cache, k, v, 0)
    lens = [2048, 600, 64, 1500, 2048]
    assert len({kvq.attn_num_splits(desc, cfg.hq, n) for n in lens}) >= 3
    fresh = [kvq.attn_decode(desc, cache, q, n, workspace=kvq.alloc_workspace(desc, cfg.hq, n, dev))
             for n in lens]
    ws = kvq.alloc_workspace(desc, cfg.hq, 2048, dev)
    for _ in range(2):
        for n, ref in zip(lens, fresh):
            got = kvq.attn_decode(desc, cache, q, n, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(got, ref), n
    assert int(ws[: 4 * 2 * cfg.hkv].count_nonzero()) == 0
    desc1 = kvq.make_desc(128, cfg.hkv, 1, 640, 128, 64, 9, 0)
    cache1 = kvq.alloc_cache(desc1, dev)
    kvq.encode(desc1, cache1, k[:1, :640].contiguous(), v[:1, :640].contiguous(), 0)
    q1 = q[:1].contiguous()
    out = kvq.attn_decode(desc1, cache1, q1, 600, softmax_scale=0.05, workspace=ws)
    torch.cuda.synchronize()
    # an explicit softmax scale is honoured
    sg = oc.layer_signs(0, 9, 128)
    got = unpack(cache1.cpu().numpy(), 128, 128, 64, 1, cfg.hkv, 640, 0, 600)
    kh, vh = oracle_dequant(got, sg, 128, 64)
    ref = oc.attention(np64(q1), kh, vh, scale=0.05)
    compare_attention(np64(out), ref, "scale 0.05")
    assert math.isclose(kvq.default_scale(128), 128 ** -0.5)
