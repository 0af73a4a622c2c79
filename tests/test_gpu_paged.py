"""Paged caches: a pool of pages shared by the sequences and a page table per sequence.
Every paged entry point must give the bytes and results of its contiguous counterpart on
the same data (pages scattered in a shuffled order), and pages mapped to no page must be
left alone by encode and append and dropped by attention (checked against the oracle)."""

import numpy as np
import pytest
import torch

from oracle import codec as oc
from parity import compare_attention, note, oracle_dequant, unpack

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("rotated_angle_quantization_amd")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def setup(dev, d=128, g=4, nk=128, nv=64, bsz=3, hkv=2, cap=1000, seed=0):
    torch.manual_seed(seed)
    desc = kvq.make_desc(d, hkv, bsz, cap, nk, nv, 5, 0)
    tiles = (cap + 63) // 64
    num_pages = bsz * tiles + 7
    perm = torch.randperm(num_pages)[: bsz * tiles].to(torch.int32)
    table = perm.view(bsz, tiles).contiguous().to(dev)
    k = torch.randn(bsz, cap, hkv, d, device=dev).half()
    v = torch.randn(bsz, cap, hkv, d, device=dev).half()
    q = torch.randn(bsz, hkv * g, d, device=dev).half()
    return desc, tiles, num_pages, table, k, v, q


def scatter(cache, desc, tiles, table, num_pages):
    """The pool holding a contiguous cache's tiles at the pages of the table."""
    tb = kvq.tile_bytes(desc.head_dim, desc.n_bins_k, desc.n_bins_v)
    b, h = desc.batch, desc.num_kv_heads
    c = cache.view(b, h, tiles, tb).permute(0, 2, 1, 3).reshape(b * tiles, h, tb)
    pool = torch.zeros(num_pages, h, tb, dtype=torch.uint8, device=cache.device)
    pool[table.flatten().long()] = c
    return pool.flatten()


@pytest.mark.parametrize("d,g,nk,nv", [(128, 4, 128, 64), (64, 8, 128, 64), (128, 8, 256, 256),
                                     (128, 4, 100, 40)])
def test_paged_paths_equal_contiguous(dev, d, g, nk, nv):
    desc, tiles, num_pages, table, k, v, q = setup(dev, d, g, nk, nv)
    paging = kvq.make_paging(table, num_pages)
    assert kvq.paged_pool_bytes(desc, num_pages) == num_pages * desc.num_kv_heads * \
        kvq.tile_bytes(d, nk, nv)
    # zero-filled, like the pool: slots past the capacity are never written on either side
    cont = torch.zeros(kvq.cache_bytes(desc), dtype=torch.uint8, device=dev)
    kvq.encode(desc, cont, k, v, 0)
    pool = torch.zeros(kvq.paged_pool_bytes(desc, num_pages), dtype=torch.uint8, device=dev)
    kvq.encode_paged(desc, pool, paging, k[:, :600], v[:, :600], 0)
    kvq.encode_paged(desc, pool, paging, k[:, 600:], v[:, 600:], 600)
    torch.cuda.synchronize()
    assert torch.equal(pool, scatter(cont, desc, tiles, table, num_pages))
    for dt in (torch.float16, torch.float32):
        assert torch.equal(torch.stack(kvq.decode_paged(desc, pool, paging, 37, 900, dt)),
                           torch.stack(kvq.decode(desc, cont, 37, 900, out_dtype=dt)))
    for n in (1000, 333, 64):
        ref = kvq.attn_decode(desc, cont, q, n, out_dtype=torch.float32)
        got = kvq.attn_decode_paged(desc, pool, paging, q, n, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), n
    lens = torch.tensor([1000, 5, 640], dtype=torch.int32, device=dev)
    ref = kvq.attn_decode_varlen(desc, cont, q, lens, 1000, out_dtype=torch.float32)
    got = kvq.attn_decode_paged(desc, pool, paging, q, 1000, seq_lens=lens,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    # one-token appends at per-sequence slots
    pos = torch.tensor([999, 0, 500], dtype=torch.int32, device=dev)
    nk_, nv_ = torch.randn(3, desc.num_kv_heads, d, device=dev).half(), \
        torch.randn(3, desc.num_kv_heads, d, device=dev).half()
    kvq.append(desc, cont, nk_, nv_, pos)
    kvq.append_paged(desc, pool, paging, nk_, nv_, pos)
    torch.cuda.synchronize()
    assert torch.equal(pool, scatter(cont, desc, tiles, table, num_pages))


def test_pages_mapped_to_no_page(dev):
    desc, tiles, num_pages, table, k, v, q = setup(dev, seed=4)
    cont = kvq.alloc_cache(desc, dev)
    kvq.encode(desc, cont, k, v, 0)
    pool = scatter(cont, desc, tiles, table, num_pages)
    holes = table.clone()
    holes[0, 3] = -1          # tokens 192..255 of sequence 0
    holes[1, 0] = num_pages   # tokens 0..63 of sequence 1
    holes[2, :] = -1          # all of sequence 2
    paging = kvq.make_paging(holes, num_pages)
    # attention drops the absent tokens (the oracle over the present ones); a sequence
    # with none gives zeros
    out = kvq.attn_decode_paged(desc, pool, paging, q, 1000, out_dtype=torch.float32)
    out16 = kvq.attn_decode_paged(desc, pool, paging, q, 1000, out_dtype=torch.float16)
    torch.cuda.synchronize()
    got = unpack(cont.cpu().numpy(), 128, 128, 64, 3, 2, 1000, 0, 1000)
    kh, vh = oracle_dequant(got, oc.layer_signs(0, 5, 128), 128, 64)
    keep = [np.r_[0:192, 256:1000], np.r_[64:1000]]
    for b in range(2):
        ref = oc.attention(np64(q[b:b + 1]), kh[b:b + 1, keep[b]], vh[b:b + 1, keep[b]])
        rel = compare_attention(np64(out[b:b + 1]), ref, f"holes seq {b}")
        rel16 = compare_attention(np64(out16[b:b + 1]), ref, f"holes seq {b} fp16 out")
        note(f"[paged] sequence {b} with a dropped page: rel-L2 {rel:.2e} (fp16 {rel16:.2e})")
    assert not torch.any(out[2])
    assert not torch.any(out16[2])
    # dequantisation returns zero vectors for absent slots
    kd, vd = kvq.decode_paged(desc, pool, paging, 0, 1000, torch.float32)
    torch.cuda.synchronize()
    assert not torch.any(kd[0, 192:256]) and not torch.any(vd[1, 0:64])
    assert torch.any(kd[0, 0:192])
    # encode and append write nothing into absent pages
    before = pool.clone()
    kvq.encode_paged(desc, pool, paging, (k[:, 192:256] * 2).contiguous(),
                     (v[:, 192:256] * 2).contiguous(), 192)
    kvq.append_paged(desc, pool, paging, k[:, 10], v[:, 10],
                     torch.tensor([200, 20, 30], dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    changed = (pool != before).view(num_pages, -1).any(dim=1).nonzero().flatten().tolist()
    # only tile 3 of sequence 1 is present among the targets (tile 3 of sequence 0,
    # tile 0 of sequence 1 and all of sequence 2 map to no page)
    assert changed == [int(holes[1, 3])], changed


def test_paged_multi_query(dev):
    """Multi-query attention over a pool equals the contiguous call bit for bit; with
    pages removed, every query attends to the present tokens it may see (oracle)."""
    desc, tiles, num_pages, table, k, v, _ = setup(dev, seed=6)
    cont = torch.zeros(kvq.cache_bytes(desc), dtype=torch.uint8, device=dev)
    kvq.encode(desc, cont, k, v, 0)
    pool = scatter(cont, desc, tiles, table, num_pages)
    nq, g = 4, 4
    q = torch.randn(desc.batch, nq, desc.num_kv_heads * g, desc.head_dim, device=dev).half()
    for n in (1000, 130):
        ref = kvq.attn_multi(desc, cont, q, n, out_dtype=torch.float32)
        got = kvq.attn_multi(desc, pool, q, n, out_dtype=torch.float32,
                             paging=kvq.make_paging(table, num_pages))
        torch.cuda.synchronize()
        assert torch.equal(got, ref), n
    holes = table.clone()
    holes[0, 2] = -1          # tokens 128..191 of sequence 0
    holes[1, 15] = -1         # the tile holding sequence 1's last tokens (960..999)
    out = kvq.attn_multi(desc, pool, q, 1000, out_dtype=torch.float32,
                         paging=kvq.make_paging(holes, num_pages))
    torch.cuda.synchronize()
    got = unpack(cont.cpu().numpy(), 128, 128, 64, 3, 2, 1000, 0, 1000)
    kh, vh = oracle_dequant(got, oc.layer_signs(0, 5, 128), 128, 64)
    keep = [np.r_[0:128, 192:1000], np.r_[0:960], np.r_[0:1000]]
    worst = 0.0
    for b in range(3):
        for j in range(nq):
            lim = 1000 - nq + j + 1
            idx = keep[b][keep[b] < lim]
            ref = oc.attention(np64(q[b:b + 1, j]), kh[b:b + 1, idx], vh[b:b + 1, idx])
            worst = max(worst, compare_attention(np64(out[b:b + 1, j]), ref,
                                                 f"multi holes b={b} j={j}"))
    note(f"[paged] multi-query with dropped pages: worst rel-L2 {worst:.2e}")
