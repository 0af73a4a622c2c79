"""The allocation-free decode-attention entry point (kvq_attn_decode_static, called
through the C ABI) against kvq_attn_decode with a caller workspace: bit-identical
outputs on two calls in a row, the second with a smaller input (the shared scratch keeps
the first call's contents, and its split counters must be cleared by the call)."""

import pytest
import torch

from parity import note
from synthetic import get, layer_kv, query

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("rotated_angle_quantization_amd")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def encoded(dev, layer, batch, seq, nk, nv):
    cfg = get("mistral7b")
    k, v = layer_kv(cfg, layer, dev, seq=seq, batch=batch)
    desc = kvq.make_desc(cfg.d, cfg.hkv, batch, seq, nk, nv, layer, 0)
    cache = kvq.alloc_cache(desc, dev)
    kvq.encode(desc, cache, k, v, 0)
    return cfg, desc, cache, query(cfg, layer, dev, batch=batch)


def test_static_entry_point_equals_workspace_call_twice(dev):
    for batch, seq, nk, nv, dt in [(2, 3000, 128, 64, torch.float16),
                                   (1, 700, 256, 256, torch.float32)]:
        cfg, desc, cache, q = encoded(dev, 5, batch, seq, nk, nv)
        note(f"[static scratch] batch {batch} seq {seq} n=({nk},{nv}) "
             f"splits {kvq.attn_num_splits(desc, cfg.hq, seq)}")
        ref = kvq.attn_decode(desc, cache, q, seq, out_dtype=dt)
        out = torch.empty_like(ref)
        got = kvq.attn_decode_static(desc, cache, q, seq, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, ref), (batch, seq)
    # a shorter call on the same (now used) scratch with one split per sequence
    cfg, desc, cache, q = encoded(dev, 6, 1, 64, 128, 64)
    assert kvq.attn_num_splits(desc, cfg.hq, 64) == 1
    ref = kvq.attn_decode(desc, cache, q, 64)
    got = kvq.attn_decode_static(desc, cache, q, 64)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)

