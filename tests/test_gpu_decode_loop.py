"""GPU parity of the decode-loop entry points: attention with a length per sequence
(kvq_attn_decode_varlen) and one-token appends at per-sequence slots (kvq_append),
against the oracle on the same seeded inputs."""

import numpy as np
import pytest
import torch

from oracle import codec as oc
from parity import compare_attention, note, oracle_dequant, unpack
from synthetic import get, layer_kv, query

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("rotated_angle_quantization_amd")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_varlen(cache, desc, q, lens):
    """Oracle attention of entry b over its first lens[b] tokens, from the oracle's own
    dequantisation of the library's bytes; a zero length gives a zero row."""
    d, hkv, bsz = desc.head_dim, desc.num_kv_heads, desc.batch
    top = max(max(lens), 1)
    got = unpack(cache.cpu().numpy(), d, desc.n_bins_k, desc.n_bins_v, bsz, hkv,
                 desc.capacity, 0, top)
    # slots past a sequence's length may hold no record (all-zero bytes); they are
    # dequantised here but never attended
    with np.errstate(invalid="ignore", divide="ignore"):
        kh, vh = oracle_dequant(got, oc.layer_signs(desc.seed, desc.layer, d),
                                desc.n_bins_k, desc.n_bins_v)
    qn = np64(q)
    out = np.zeros(qn.shape)
    for b, n in enumerate(lens):
        if n:
            out[b] = oc.attention(qn[b:b + 1], kh[b:b + 1, :n], vh[b:b + 1, :n])[0]
    return out


@pytest.mark.parametrize("d,g,nk,nv", [(128, 4, 128, 64), (64, 8, 128, 64), (128, 4, 256, 256),
                                       (128, 8, 256, 256), (128, 2, 100, 40)])
def test_attention_varlen_matches_oracle(dev, d, g, nk, nv):
    torch.manual_seed(d + g + nk)
    hkv, cap = 2, 2048
    lens = [1, 700, 0, 2048, 65, 1999]
    bsz = len(lens)
    note(f"[varlen] d={d} G={g} n=({nk},{nv}) lens={lens}")
    k = torch.randn(bsz, cap, hkv, d, device=dev).half()
    v = torch.randn(bsz, cap, hkv, d, device=dev).half()
    q = torch.randn(bsz, hkv * g, d, device=dev).half()
    desc = kvq.make_desc(d, hkv, bsz, cap, nk, nv, 3, 0)
    cache = kvq.alloc_cache(desc, dev)
    kvq.encode(desc, cache, k, v, 0)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    ws = kvq.alloc_workspace(desc, hkv * g, cap, dev)
    ref = oracle_varlen(cache, desc, q, lens)
    for dt in (torch.float32, torch.float16):
        out = kvq.attn_decode_varlen(desc, cache, q, seq_lens, cap, out_dtype=dt, workspace=ws)
        torch.cuda.synchronize()
        got = np64(out)
        assert not np.any(got[2]), "a zero-length sequence gives a zero output"
        rel = compare_attention(np.delete(got, 2, 0), np.delete(ref, 2, 0),
                                f"varlen d{d} G{g} {dt}")
        note(f"[varlen] {dt} worst rel-L2 {rel:.2e}")
    assert int(ws[: 4 * bsz * hkv].count_nonzero()) == 0, "split counters back at zero"


def test_attention_varlen_uniform_equals_fixed_length_and_clamps(dev):
    """Every entry at max_seq_len gives the bits of kvq_attn_decode; entries above the
    bound count as the bound; fp16 output as well."""
    cfg = get("mistral7b")
    k, v = layer_kv(cfg, 6, dev, seq=1536, batch=3)
    q = query(cfg, 6, dev, batch=3)
    desc = kvq.make_desc(128, cfg.hkv, 3, 1536, 128, 64, 6, 0)
    cache = kvq.alloc_cache(desc, dev)
    kvq.encode(desc, cache, k, v, 0)
    ws = kvq.alloc_workspace(desc, cfg.hq, 1536, dev)
    for dt in (torch.float16, torch.float32):
        fixed = kvq.attn_decode(desc, cache, q, 1200, out_dtype=dt, workspace=ws)
        same = kvq.attn_decode_varlen(desc, cache, q,
                                      torch.full((3,), 1200, dtype=torch.int32, device=dev),
                                      1200, out_dtype=dt, workspace=ws)
        over = kvq.attn_decode_varlen(desc, cache, q,
                                      torch.tensor([1200, 5000, 1 << 30], dtype=torch.int32,
                                                   device=dev), 1200, out_dtype=dt, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(fixed, same)
        assert torch.equal(fixed, over)
    assert int(ws[: 4 * 3 * cfg.hkv].count_nonzero()) == 0


@pytest.mark.parametrize("f32", [False, True])
def test_append_at_per_sequence_slots_gives_one_shot_bytes(dev, f32):
    """Encoding data with some tokens replaced, then appending the true tokens at those
    slots, gives the bytes of encoding the true data at once: the appended token's codes
    are those of the encoder, and its neighbours (which share value words) are kept."""
    torch.manual_seed(11 + f32)
    d, hkv, cap = 128, 3, 1024
    pos = [5, 64, 127, 1000, 0, 1023]
    bsz = len(pos)
    dt = torch.float32 if f32 else torch.float16
    k = (torch.randn(bsz, cap, hkv, d, device=dev) * 2).to(dt)
    v = torch.randn(bsz, cap, hkv, d, device=dev).to(dt)
    desc = kvq.make_desc(d, hkv, bsz, cap, 128, 64, 4, 0)
    truth = kvq.alloc_cache(desc, dev)
    kvq.encode(desc, truth, k, v, 0)
    k2, v2 = k.clone(), v.clone()
    for b, p in enumerate(pos):
        k2[b, p] = torch.randn(hkv, d, device=dev).to(dt)
        v2[b, p] = torch.randn(hkv, d, device=dev).to(dt)
    cache = kvq.alloc_cache(desc, dev)
    kvq.encode(desc, cache, k2, v2, 0)
    torch.cuda.synchronize()
    assert not torch.equal(cache, truth)
    positions = torch.tensor(pos, dtype=torch.int32, device=dev)
    rows = torch.arange(bsz, device=dev)
    kvq.append(desc, cache, k[rows, positions.long()], v[rows, positions.long()], positions)
    torch.cuda.synchronize()
    assert torch.equal(cache, truth)
    # a slot past the capacity writes nothing
    before = cache.clone()
    junk = torch.randn(bsz, hkv, d, device=dev).to(dt)
    kvq.append(desc, cache, junk, junk, torch.full((bsz,), cap, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert torch.equal(cache, before)


def test_ragged_decode_loop(dev):
    """A ragged batch decodes a few steps: each step appends one token per sequence at
    its own length and attends over the new lengths; every step matches the oracle."""
    cfg = get("mistral7b")
    bsz, cap = 4, 1024
    k, v = layer_kv(cfg, 10, dev, seq=cap, batch=bsz)
    desc = kvq.make_desc(128, cfg.hkv, bsz, cap, 128, 64, 10, 0)
    cache = kvq.alloc_cache(desc, dev)
    lens = [100, 257, 1, 640]
    # prefixes of different lengths: one encode of the longest, with other data in every
    # slot past a sequence's own length (the appends must overwrite those)
    k0, v0 = k[:, :max(lens)].clone(), v[:, :max(lens)].clone()
    for b, n in enumerate(lens):
        k0[b, n:] = -k0[b, n:]
        v0[b, n:] = v0[b, n:].flip(-1)
    kvq.encode(desc, cache, k0, v0, 0)
    ws = kvq.alloc_workspace(desc, cfg.hq, cap, dev)
    rows = torch.arange(bsz, device=dev)
    for step in range(3):
        positions = torch.tensor(lens, dtype=torch.int32, device=dev)
        kvq.append(desc, cache, k[rows, positions.long()], v[rows, positions.long()], positions)
        lens = [n + 1 for n in lens]
        q = query(cfg, 10, dev, batch=bsz, seed=step)
        out = kvq.attn_decode_varlen(desc, cache, q, positions + 1, cap,
                                     out_dtype=torch.float32, workspace=ws)
        out16 = kvq.attn_decode_varlen(desc, cache, q, positions + 1, cap,
                                       out_dtype=torch.float16, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle_varlen(cache, desc, q, lens)
        rel = compare_attention(np64(out), ref, f"decode step {step}")
        rel16 = compare_attention(np64(out16), ref, f"decode step {step} fp16 out")
        note(f"[decode loop] step {step} lens {lens} rel-L2 {rel:.2e} (fp16 out {rel16:.2e})")
    # the appended caches equal a one-shot encode of the same tokens
    truth = kvq.alloc_cache(desc, dev)
    kvq.encode(desc, truth, k[:, :max(lens)], v[:, :max(lens)], 0)
    torch.cuda.synchronize()
    a = unpack(cache.cpu().numpy(), 128, 128, 64, bsz, cfg.hkv, cap, 0, max(lens))
    r = unpack(truth.cpu().numpy(), 128, 128, 64, bsz, cfg.hkv, cap, 0, max(lens))
    for key in r:
        for b, n in enumerate(lens):
            np.testing.assert_array_equal(a[key][b, :n], r[key][b, :n], err_msg=f"{key} b{b}")
