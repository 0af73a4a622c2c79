"""Decode attention captured in a HIP graph (through torch's graph capture on the
library's stream): every replay must equal the eager call bit for bit, with eager work
and synchronisation between replays, for the one-launch (key table) and the two-launch
(query-rotation kernel first) forms and for the fused append step."""

import pytest
import torch

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("rotated_angle_quantization_amd")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.mark.parametrize("nk", [128, 200])  # key table / no table (prepare kernel + split)
def test_attention_graph_replays_equal_eager(dev, nk):
    torch.manual_seed(nk)
    d, hkv, g, bsz, cap = 128, 2, 8, 2, 3000
    desc = kvq.make_desc(d, hkv, bsz, cap, nk, 64, 1, 0)
    cache = kvq.alloc_cache(desc, dev)
    kvq.encode(desc, cache, torch.randn(bsz, cap, hkv, d, device=dev).half(),
               torch.randn(bsz, cap, hkv, d, device=dev).half(), 0)
    q = torch.randn(bsz, hkv * g, d, device=dev).half()
    ws = kvq.alloc_workspace(desc, hkv * g, cap, dev)
    ref = kvq.attn_decode(desc, cache, q, cap, out_dtype=torch.float32, workspace=ws)
    out = torch.empty_like(ref)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            kvq.attn_decode(desc, cache, q, cap, workspace=ws, out=out)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        # eager work in between replays
        eager = kvq.attn_decode(desc, cache, q, cap, out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(eager, ref)


def test_fused_step_graph_replays(dev):
    torch.manual_seed(3)
    d, hkv, g, bsz, cap = 128, 2, 4, 3, 1024
    desc = kvq.make_desc(d, hkv, bsz, cap, 128, 64, 1, 0)
    cache = kvq.alloc_cache(desc, dev)
    kvq.encode(desc, cache, torch.randn(bsz, cap, hkv, d, device=dev).half(),
               torch.randn(bsz, cap, hkv, d, device=dev).half(), 0)
    pos = torch.tensor([100, 500, 1000], dtype=torch.int32, device=dev)
    kn = torch.randn(bsz, hkv, d, device=dev).half()
    vn = torch.randn(bsz, hkv, d, device=dev).half()
    q = torch.randn(bsz, hkv * g, d, device=dev).half()
    ws = kvq.alloc_workspace(desc, hkv * g, cap, dev)
    base = cache.clone()
    ref = kvq.attn_decode_append(desc, cache, kn, vn, pos, q, cap, out_dtype=torch.float32,
                                 workspace=ws)
    ref_cache = cache.clone()
    out = torch.empty_like(ref)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            kvq.attn_decode_append(desc, cache, kn, vn, pos, q, cap, workspace=ws, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        cache.copy_(base)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        assert torch.equal(cache, ref_cache), rep
