"""GPU parity of multi-query attention over the compressed cache (kvq_attn_multi):
num_queries query tokens per sequence, query j attending causally to the first
seq_len - num_queries + j + 1 cached tokens, against the oracle's attention over its own
dequantisation of the library's bytes."""

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


def oracle_multi(cache, desc, q, seq_len, scale=None):
    d, hkv, bsz = desc.head_dim, desc.num_kv_heads, desc.batch
    got = unpack(cache.cpu().numpy(), d, desc.n_bins_k, desc.n_bins_v, bsz, hkv,
                 desc.capacity, 0, seq_len)
    kh, vh = oracle_dequant(got, oc.layer_signs(desc.seed, desc.layer, d), desc.n_bins_k,
                            desc.n_bins_v)
    qn = np64(q)  # [B, NQ, Hq, d]
    nq = qn.shape[1]
    out = np.zeros(qn.shape)
    for j in range(nq):
        n = seq_len - nq + j + 1
        out[:, j] = oc.attention(qn[:, j], kh[:, :n], vh[:, :n], scale=scale)
    return out


def run_multi(dev, d, g, nq, seq_len, nk=128, nv=64, hkv=2, bsz=2, cap=None, q_dt=torch.float16,
              out_dt=torch.float32, seed=0, scale=0.0):
    torch.manual_seed(seed + 7 * d + g + nq)
    cap = cap or seq_len
    k = (torch.randn(bsz, cap, hkv, d, device=dev) * 1.5).half()
    v = torch.randn(bsz, cap, hkv, d, device=dev).half()
    q = torch.randn(bsz, nq, hkv * g, d, device=dev).to(q_dt)
    desc = kvq.make_desc(d, hkv, bsz, cap, nk, nv, 2, 0)
    cache = kvq.alloc_cache(desc, dev)
    kvq.encode(desc, cache, k, v, 0)
    out = kvq.attn_multi(desc, cache, q, seq_len, softmax_scale=scale, out_dtype=out_dt)
    torch.cuda.synchronize()
    ref = oracle_multi(cache, desc, q, seq_len, scale=scale if scale > 0 else None)
    got = np64(out)
    rel = compare_attention(got.reshape(-1, d), ref.reshape(-1, d),
                            f"multi d{d} G{g} NQ{nq} L{seq_len}")
    note(f"[multi] d={d} G={g} NQ={nq} L={seq_len} n=({nk},{nv}) worst rel-L2 {rel:.2e}")
    return out, desc, cache, q


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g,nq", [(1, 1), (1, 16), (1, 32), (2, 8), (4, 1), (4, 4), (4, 8),
                                  (8, 2), (8, 4), (2, 3), (4, 5)])
def test_multi_query_matches_oracle(dev, d, g, nq):
    run_multi(dev, d, g, nq, 777, cap=800)


@pytest.mark.parametrize("seq_len", [1, 5, 64, 65, 200, 4096])
def test_multi_query_sequence_lengths_and_splits(dev, seq_len):
    nq = min(4, seq_len)
    run_multi(dev, 128, 4, nq, seq_len, cap=max(seq_len, 64), bsz=3, hkv=2)


@pytest.mark.parametrize("nk,nv", [(256, 256), (100, 40), (64, 128)])
def test_multi_query_code_widths_dtypes_and_scale(dev, nk, nv):
    run_multi(dev, 128, 4, 8, 1000, nk=nk, nv=nv, q_dt=torch.float32, out_dt=torch.float16,
              scale=0.07)


@pytest.mark.parametrize("d,g,nq,nk,nv", [(128, 4, 4, 32, 64), (64, 2, 8, 128, 5),
                                           (128, 8, 3, 3, 17), (128, 1, 16, 24, 12)])
def test_multi_query_narrow_codebooks(dev, d, g, nq, nk, nv):
    """Codebooks of at most 32 bins (1- to 5-bit codes) through the 6-bit widened copy."""
    run_multi(dev, d, g, nq, 333, nk=nk, nv=nv, cap=400)


def test_multi_query_one_query_agrees_with_decode_attention(dev):
    """With one query token the result is single-query decode attention (fp16 matrix
    operands against the decode kernel's fp32 arithmetic: close, not bitwise)."""
    cfg = get("mistral7b")
    k, v = layer_kv(cfg, 7, dev, seq=3000, batch=2)
    q = query(cfg, 7, dev, batch=2)
    desc = kvq.make_desc(128, cfg.hkv, 2, 3000, 128, 64, 7, 0)
    cache = kvq.alloc_cache(desc, dev)
    kvq.encode(desc, cache, k, v, 0)
    o1 = kvq.attn_decode(desc, cache, q, 3000, out_dtype=torch.float32)
    om = kvq.attn_multi(desc, cache, q[:, None].contiguous(), 3000, out_dtype=torch.float32)
    torch.cuda.synchronize()
    compare_attention(np64(om[:, 0]).reshape(-1, 128), np64(o1).reshape(-1, 128),
                      "multi vs decode")


def test_multi_query_workspace_reuse(dev):
    cfg = get("mistral7b")
    k, v = layer_kv(cfg, 8, dev, seq=4096, batch=2)
    desc = kvq.make_desc(128, cfg.hkv, 2, 4096, 128, 64, 8, 0)
    cache = kvq.alloc_cache(desc, dev)
    kvq.encode(desc, cache, k, v, 0)
    ws = torch.zeros(kvq.attn_multi_workspace_bytes(desc, cfg.hq, 8, 4096), dtype=torch.uint8,
                     device=dev)
    torch.manual_seed(3)
    q = torch.randn(2, 8, cfg.hq, 128, device=dev).half()
    ref = kvq.attn_multi(desc, cache, q, 4096)
    for n in (4096, 700, 4096):
        got = kvq.attn_multi(desc, cache, q, n, workspace=ws)
        fresh = kvq.attn_multi(desc, cache, q, n)
        torch.cuda.synchronize()
        assert torch.equal(got, fresh), n
    assert torch.equal(kvq.attn_multi(desc, cache, q, 4096, workspace=ws), ref)
    assert int(ws[: 4 * 2 * cfg.hkv].count_nonzero()) == 0


@pytest.mark.parametrize("g,nq", [(4, 4), (4, 8), (1, 32), (8, 3)])
def test_multi_query_ragged_batch(dev, g, nq):
    """Per-sequence lengths (kvq_attn_multi_varlen): query j of sequence b attends to the
    first L_b - NQ + j + 1 tokens (none: a zero row); lengths above the bound are clamped;
    with every length at the bound the result is that of the fixed-length call."""
    torch.manual_seed(11 + g + nq)
    d, hkv, cap = 128, 2, 1000
    lens = [1000, 3, 0, 640, 65, 1500]  # 1500 is clamped to the bound (1000)
    bsz = len(lens)
    k = (torch.randn(bsz, cap, hkv, d, device=dev) * 1.5).half()
    v = torch.randn(bsz, cap, hkv, d, device=dev).half()
    q = torch.randn(bsz, nq, hkv * g, d, device=dev).half()
    desc = kvq.make_desc(d, hkv, bsz, cap, 128, 64, 2, 0)
    cache = kvq.alloc_cache(desc, dev)
    kvq.encode(desc, cache, k, v, 0)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    out = kvq.attn_multi(desc, cache, q, cap, seq_lens=sl, out_dtype=torch.float32)
    full = torch.full_like(sl, cap)
    same = kvq.attn_multi(desc, cache, q, cap, seq_lens=full, out_dtype=torch.float32)
    ref_fixed = kvq.attn_multi(desc, cache, q, cap, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(same, ref_fixed)
    got = unpack(cache.cpu().numpy(), d, 128, 64, bsz, hkv, cap, 0, cap)
    kh, vh = oracle_dequant(got, oc.layer_signs(0, 2, d), 128, 64)
    qn, on = np64(q), np64(out)
    worst = 0.0
    for b, length in enumerate(min(x, cap) for x in lens):
        for j in range(nq):
            n = length - nq + j + 1
            if n <= 0:
                assert not np.any(on[b, j]), (b, j)
                continue
            ref = oc.attention(qn[b:b + 1, j], kh[b:b + 1, :n], vh[b:b + 1, :n])
            worst = max(worst, compare_attention(on[b:b + 1, j].reshape(-1, d),
                                                 ref.reshape(-1, d), f"ragged b={b} j={j}"))
    note(f"[multi] ragged batch G={g} NQ={nq}: worst rel-L2 {worst:.2e}")
