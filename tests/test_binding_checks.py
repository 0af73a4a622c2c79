"""The Python binding rejects arguments that would make a kernel read or write out of
bounds, before any library call: wrong shapes, dtypes, layouts, undersized buffers,
short page tables and tensors in host memory. CPU only (no kernel is launched: every
case fails its check first)."""

import pytest
import torch

kvq = pytest.importorskip("rotated_angle_quantization_amd")

D, HKV, B, CAP, G = 128, 2, 3, 256, 4


@pytest.fixture
def desc():
    return kvq.make_desc(D, HKV, B, CAP, 128, 64, 0, 0)


def cache_for(desc):
    return torch.zeros(kvq.cache_bytes(desc), dtype=torch.uint8)


def rows(ntok=5, dtype=torch.float16):
    return torch.zeros(B, ntok, HKV, D, dtype=dtype), torch.zeros(B, ntok, HKV, D, dtype=dtype)


def err(fn, *a, match, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_encode_checks(desc):
    cache = cache_for(desc)
    k, v = rows()
    err(kvq.encode, desc, cache, k[:2], v[:2], match="shape")            # batch
    err(kvq.encode, desc, cache, k[..., :64], v[..., :64], match="shape")  # head_dim
    err(kvq.encode, desc, cache, k, v.float(), match="dtype")
    err(kvq.encode, desc, cache, k.int(), v.int(), match="float16 or float32")
    kt = torch.zeros(B, 5, D, HKV, dtype=torch.float16).transpose(2, 3)
    err(kvq.encode, desc, cache, kt, kt, match="contiguous")
    err(kvq.encode, desc, cache[:-1], k, v, match="bytes")              # undersized cache
    err(kvq.encode, desc, cache.float(), k, v, match="uint8")
    err(kvq.encode, desc, cache, k, v, match="GPU memory")              # host tensors


def test_append_checks(desc):
    cache = cache_for(desc)
    k = torch.zeros(B, HKV, D, dtype=torch.float16)
    pos = torch.zeros(B, dtype=torch.int32)
    err(kvq.append, desc, cache, k, k, pos.long(), match="int32")       # int64 positions
    err(kvq.append, desc, cache, k, k, pos[:2], match="entries")
    err(kvq.append, desc, cache, k[:, :1], k[:, :1], pos, match="shape")
    err(kvq.append, desc, cache, k, k, pos, match="GPU memory")


def test_decode_checks(desc):
    cache = cache_for(desc)
    good = torch.zeros(B, 10, HKV, D, dtype=torch.float16)
    err(kvq.decode, desc, cache, 0, 10, out=(good[:, :5], good), match="shape")
    err(kvq.decode, desc, cache, 0, 10, out=(good, good.float()), match="dtype")
    err(kvq.decode, desc, cache, 0, 10, out=(good.transpose(1, 2).contiguous().transpose(1, 2),
                                             good), match="contiguous")
    err(kvq.decode, desc, cache[:100], 0, 10, match="bytes")
    err(kvq.decode, desc, cache, 0, 10, out=(good, good), match="GPU memory")


def test_attention_checks(desc):
    cache = cache_for(desc)
    q = torch.zeros(B, HKV * G, D, dtype=torch.float16)
    err(kvq.attn_decode, desc, cache, q[:1], CAP, match="shape")
    err(kvq.attn_decode, desc, cache, q[..., :64], CAP, match="shape")
    err(kvq.attn_decode, desc, cache, q.transpose(0, 1).contiguous().transpose(0, 1), CAP,
        match="contiguous")
    err(kvq.attn_decode, desc, cache, q, CAP, out=torch.zeros(B, HKV * G, 64), match="shape")
    err(kvq.attn_decode, desc, cache, q, CAP, out=torch.zeros(B, HKV * G, D, dtype=torch.int32),
        match="float16 or float32")
    err(kvq.attn_decode, desc, cache[:10], q, CAP, match="bytes")
    err(kvq.attn_decode, desc, cache, q, CAP, match="GPU memory")
    ws = torch.zeros(16, dtype=torch.uint8)
    err(kvq.attn_decode, desc, cache, q, CAP, workspace=ws, match="GPU memory")
    lens = torch.full((B,), CAP, dtype=torch.int32)
    err(kvq.attn_decode_varlen, desc, cache, q, lens.long(), CAP, match="int32")
    err(kvq.attn_decode_varlen, desc, cache, q, lens[:1], CAP, match="entries")
    err(kvq.attn_decode_varlen, desc, cache, q, lens, CAP, match="GPU memory")


def test_fused_and_multi_query_checks(desc):
    cache = cache_for(desc)
    k = torch.zeros(B, HKV, D, dtype=torch.float16)
    pos = torch.zeros(B, dtype=torch.int32)
    q = torch.zeros(B, HKV * G, D, dtype=torch.float16)
    err(kvq.attn_decode_append, desc, cache, k, k, pos.long(), q, CAP, match="int32")
    err(kvq.attn_decode_append, desc, cache, k, k, pos, q[:, :1, :64], CAP, match="shape")
    err(kvq.attn_decode_append, desc, cache, k, k, pos, q, CAP, match="GPU memory")
    qm = torch.zeros(B, 3, HKV * G, D, dtype=torch.float16)
    err(kvq.attn_multi, desc, cache, qm[:, :, :, :64], CAP, match="shape")
    err(kvq.attn_multi, desc, cache, qm, CAP, seq_lens=pos.long(), match="int32")
    err(kvq.attn_multi, desc, cache, qm, CAP, match="GPU memory")


def test_paged_checks(desc):
    table = torch.zeros(B, CAP // 64, dtype=torch.int32)
    paging = kvq.make_paging(table, 8)
    pool = torch.zeros(kvq.paged_pool_bytes(desc, 8), dtype=torch.uint8)
    k, v = rows()
    err(kvq.encode_paged, desc, pool[:-1], paging, k, v, match="bytes")
    short = kvq.make_paging(table[:1], 8)
    err(kvq.encode_paged, desc, pool, short, k, v, match="rows")
    err(kvq.encode_paged, desc, pool, kvq.Paging(table.data_ptr(), CAP // 64, 8), k, v,
        match="make_paging")
    one = torch.zeros(B, HKV, D, dtype=torch.float16)
    err(kvq.append_paged, desc, pool, paging, one, one, torch.zeros(B, dtype=torch.int64),
        match="int32")
    q = torch.zeros(B, HKV * G, D, dtype=torch.float16)
    err(kvq.attn_decode_paged, desc, pool, paging, q, CAP,
        seq_lens=torch.zeros(B, dtype=torch.int64), match="int32")
    err(kvq.attn_decode_paged, desc, pool, paging, q, CAP, match="GPU memory")
    err(kvq.decode_paged, desc, pool, paging, 0, 10, match="GPU memory")
