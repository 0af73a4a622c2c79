"""One decode step in one launch (kvq_attn_decode_append): the token coded inside the
attention kernel must leave the cache bytes of kvq_append, and the output must be that
of kvq_attn_decode_varlen over the appended lengths, bit for bit; one step is also
checked against the oracle. Covers the three key-table modes, d 64 and 128, fp16 and
fp32 token inputs, slots at tile edges, slots past the attended range or the capacity,
paged pools with absent pages, and a loop of steps."""

import numpy as np
import pytest
import torch

from oracle import codec as oc
from parity import compare_attention, compare_codes, note, oracle_dequant, oracle_encode, unpack

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("rotated_angle_quantization_amd")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def filled_cache(dev, d, hkv, bsz, cap, nk, nv, seed):
    """A cache whose every slot holds coded data (so appends overwrite real codes)."""
    torch.manual_seed(seed)
    desc = kvq.make_desc(d, hkv, bsz, cap, nk, nv, 3, 0)
    cache = torch.zeros(kvq.cache_bytes(desc), dtype=torch.uint8, device=dev)
    k = torch.randn(bsz, cap, hkv, d, device=dev).half()
    v = torch.randn(bsz, cap, hkv, d, device=dev).half()
    kvq.encode(desc, cache, k, v, 0)
    return desc, cache


def step_both(desc, cache, kn, vn, pos, q, maxlen, ws):
    """(cache after, output) of the fused call and of append + varlen attention."""
    fused = cache.clone()
    out_f = kvq.attn_decode_append(desc, fused, kn, vn, pos, q, maxlen, out_dtype=torch.float32,
                                   workspace=ws)
    sep = cache.clone()
    kvq.append(desc, sep, kn, vn, pos)
    lens = (pos.long() + 1).clamp(max=maxlen).to(torch.int32)
    out_s = kvq.attn_decode_varlen(desc, sep, q, lens, maxlen, out_dtype=torch.float32,
                                   workspace=ws)
    torch.cuda.synchronize()
    return fused, out_f, sep, out_s


# (d, G, n_K, n_V): half table (n a power of two), full table, no table (n_K = 200 does
# not fit at G = 8), for d = 128 and d = 64; then codebooks of at most 32 bins (append,
# then attention over the 6-bit widened copy)
CASES = [(128, 4, 128, 64), (128, 4, 100, 40), (128, 8, 200, 256), (64, 8, 128, 64),
         (64, 1, 256, 128), (64, 4, 100, 40), (64, 8, 200, 100),
         (128, 4, 32, 64), (64, 2, 100, 5), (128, 8, 3, 17)]


@pytest.mark.parametrize("d,g,nk,nv", CASES)
@pytest.mark.parametrize("f32", [False, True])
def test_fused_step_equals_append_then_attend(dev, d, g, nk, nv, f32):
    hkv, bsz, cap = 2, 6, 1024
    desc, cache = filled_cache(dev, d, hkv, bsz, cap, nk, nv, seed=d + g + nk)
    # slot 0, the last slot of a tile, the first of the next, the last slot, a slot past
    # the attended range (max_seq_len 900 < capacity) and one past the capacity
    pos = torch.tensor([0, 63, 64, cap - 1, 950, cap], dtype=torch.int32, device=dev)
    dt = torch.float32 if f32 else torch.float16
    kn = torch.randn(bsz, hkv, d, device=dev).to(dt)
    vn = torch.randn(bsz, hkv, d, device=dev).to(dt)
    q = torch.randn(bsz, hkv * g, d, device=dev).half()
    ws = kvq.alloc_workspace(desc, hkv * g, 900, dev)
    fused, out_f, sep, out_s = step_both(desc, cache, kn, vn, pos, q, 900, ws)
    assert torch.equal(fused, sep)
    assert not torch.equal(fused, cache)
    assert torch.equal(out_f, out_s)


def test_fused_step_matches_oracle(dev):
    d, g, hkv, bsz, cap, nk, nv = 128, 4, 2, 3, 700, 128, 64
    desc, cache = filled_cache(dev, d, hkv, bsz, cap, nk, nv, seed=11)
    pos = torch.tensor([5, 699, 320], dtype=torch.int32, device=dev)
    kn = torch.randn(bsz, hkv, d, device=dev).half()
    vn = torch.randn(bsz, hkv, d, device=dev).half()
    q = torch.randn(bsz, hkv * g, d, device=dev).half()
    out = kvq.attn_decode_append(desc, cache, kn, vn, pos, q, cap, out_dtype=torch.float32)
    # the same step again with fp16 output (the appended bytes are rewritten unchanged)
    out16 = kvq.attn_decode_append(desc, cache, kn, vn, pos, q, cap, out_dtype=torch.float16)
    torch.cuda.synchronize()
    codes = unpack(cache.cpu().numpy(), d, nk, nv, bsz, hkv, cap, 0, cap)
    kh, vh = oracle_dequant(codes, oc.layer_signs(0, 3, d), nk, nv)
    # the appended tokens carry the oracle's codes of the new rows (the code rule of the
    # parity tests: bit-exact away from bin boundaries)
    sg = oc.layer_signs(0, 3, d)
    rows = np.arange(bsz)
    p_np = pos.cpu().numpy()
    got = {key: val[rows, p_np][:, None] for key, val in codes.items()}
    ek, ev = oracle_encode(np64(kn[:, None]), np64(vn[:, None]), sg, nk, nv)
    compare_codes(got, ek, ev)
    worst = 0.0
    for b, p in enumerate(pos.tolist()):
        ref = oc.attention(np64(q[b:b + 1]), kh[b:b + 1, :p + 1], vh[b:b + 1, :p + 1])
        worst = max(worst, compare_attention(np64(out[b:b + 1]), ref, f"fused b={b}"))
        worst = max(worst, compare_attention(np64(out16[b:b + 1]), ref, f"fused b={b} fp16"))
    note(f"[fused append] worst rel-L2 against the oracle (fp32 and fp16 out) {worst:.2e}")


def test_fused_decode_loop(dev):
    """Several steps in a row (one workspace) equal the same steps made with two calls."""
    d, g, hkv, bsz, cap, nk, nv = 128, 4, 4, 4, 512, 128, 64
    desc, cache = filled_cache(dev, d, hkv, bsz, cap, nk, nv, seed=5)
    lens = [10, 63, 200, 447]
    ws = kvq.alloc_workspace(desc, hkv * g, cap, dev)
    a, b = cache.clone(), cache.clone()
    for step in range(5):
        pos = torch.tensor(lens, dtype=torch.int32, device=dev)
        kn = torch.randn(bsz, hkv, d, device=dev).half()
        vn = torch.randn(bsz, hkv, d, device=dev).half()
        q = torch.randn(bsz, hkv * g, d, device=dev).half()
        out_a = kvq.attn_decode_append(desc, a, kn, vn, pos, q, cap, workspace=ws)
        kvq.append(desc, b, kn, vn, pos)
        out_b = kvq.attn_decode_varlen(desc, b, q, pos + 1, cap, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(a, b), step
        assert torch.equal(out_a, out_b), step
        lens = [n + 1 for n in lens]


def test_fused_step_paged(dev):
    d, g, hkv, bsz, cap, nk, nv = 128, 4, 2, 3, 640, 128, 64
    desc, cache = filled_cache(dev, d, hkv, bsz, cap, nk, nv, seed=9)
    tiles = cap // 64
    tb = kvq.tile_bytes(d, nk, nv)
    num_pages = bsz * tiles + 5
    torch.manual_seed(1)
    table = torch.randperm(num_pages)[: bsz * tiles].to(torch.int32).view(bsz, tiles).to(dev)
    c = cache.view(bsz, hkv, tiles, tb).permute(0, 2, 1, 3).reshape(bsz * tiles, hkv, tb)
    pool = torch.zeros(num_pages, hkv, tb, dtype=torch.uint8, device=dev)
    pool[table.flatten().long()] = c
    pool = pool.flatten()
    holes = table.clone()
    holes[2, 4] = -1  # the tile of sequence 2's new token has no page
    paging = kvq.make_paging(holes, num_pages)
    pos = torch.tensor([100, 639, 300], dtype=torch.int32, device=dev)
    kn = torch.randn(bsz, hkv, d, device=dev).half()
    vn = torch.randn(bsz, hkv, d, device=dev).half()
    q = torch.randn(bsz, hkv * g, d, device=dev).half()
    p_fused = pool.clone()
    out_f = kvq.attn_decode_append(desc, p_fused, kn, vn, pos, q, cap, paging=paging,
                                   out_dtype=torch.float32)
    p_sep = pool.clone()
    kvq.append_paged(desc, p_sep, paging, kn, vn, pos)
    out_s = kvq.attn_decode_paged(desc, p_sep, paging, q, cap, seq_lens=pos + 1,
                                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(p_fused, p_sep)
    assert torch.equal(out_f, out_s)
    # the absent page took no write; the two present ones did
    changed = (p_fused != pool).view(num_pages, -1).any(dim=1).nonzero().flatten().tolist()
    assert sorted(changed) == sorted([int(holes[0, 1]), int(holes[1, 9])])
