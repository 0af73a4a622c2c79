"""C-ABI checks that need no GPU: the library loads, exports every function the header
declares, and its host-only helpers and argument validation behave as documented.
Only error paths (which return before any HIP call) and ntok = 0 are exercised."""

import ctypes
import os
import re

import numpy as np
import pytest

from conftest import ROOT
from oracle import codec as oc
from oracle import layout as ol

kvq = pytest.importorskip("rotated_angle_quantization_amd")
lib = kvq.lib

OK, INVALID, UNSUPPORTED, CAPACITY, WORKSPACE = 0, 1, 2, 3, 4
FAKE = 0x10000  # aligned non-null address; never dereferenced on the paths tested


def header_functions():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    return sorted(set(re.findall(r"^\s*[\w\s\*]+?\b(kvq_\w+)\s*\(", text, re.M)))


def test_every_declared_function_is_exported():
    names = header_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(kvq.EXPORTS)


def test_version_and_status_strings():
    assert kvq.abi_version() == 10
    for s in range(6):
        assert lib.kvq_status_string(s)
    assert lib.kvq_status_string(99) == b"unknown status"


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("nk,nv", [(128, 64), (256, 256), (2, 3), (100, 33), (64, 128)])
def test_tile_and_cache_bytes_match_layout_definition(d, nk, nv):
    assert kvq.tile_bytes(d, nk, nv) == ol.tile_bytes(d, nk, nv)
    desc = kvq.make_desc(d, 3, 2, 100, nk, nv)
    assert kvq.cache_bytes(desc) == ol.cache_bytes(d, nk, nv, 2, 3, 100)


def test_invalid_descriptors_size_zero():
    assert kvq.tile_bytes(96, 128, 64) == 0
    assert kvq.tile_bytes(32, 128, 64) == 0
    assert kvq.tile_bytes(128, 1, 64) == 0
    assert kvq.tile_bytes(128, 128, 257) == 0
    for bad in (dict(head_dim=48), dict(num_kv_heads=0), dict(batch=0), dict(capacity=0),
                dict(capacity=2**31 - 63), dict(n_bins_k=300), dict(reserved=1)):
        desc = kvq.make_desc(128, 8, 1, 64, 128, 64)
        for k, v in bad.items():
            setattr(desc, k, v)
        assert kvq.cache_bytes(desc) == 0, bad


@pytest.mark.parametrize("seed,layer,d", [(0, 0, 64), (0, 5, 128), (12345, 31, 128),
                                          (2**63 + 7, 79, 256), (1, 2**31, 64)])
def test_library_signs_equal_oracle_signs(seed, layer, d):
    assert kvq.layer_signs(seed, layer, d) == oc.layer_signs(seed, layer, d).astype(int).tolist()


def _enc(desc, k=FAKE, v=FAKE, dtype=0, sb=0, st=0, sh=0, t0=0, ntok=1, cache=FAKE):
    return lib.kvq_encode(ctypes.byref(desc), cache, k, v, dtype, sb, st, sh, t0, ntok, None)


def test_encode_validation():
    desc = kvq.make_desc(128, 8, 1, 128, 128, 64)
    assert _enc(desc, ntok=0) == OK  # nothing to do, no device call
    assert _enc(desc, t0=100, ntok=29) == CAPACITY
    assert _enc(desc, k=None) == INVALID
    assert _enc(desc, cache=None) == INVALID
    assert _enc(desc, cache=FAKE + 8) == INVALID  # cache must be 16-byte aligned
    assert _enc(desc, dtype=7) == INVALID
    assert _enc(desc, k=FAKE + 2) == INVALID  # fp16 pairs need 4-byte alignment
    assert _enc(desc, dtype=1, k=FAKE + 4) == INVALID  # fp32 pairs need 8 bytes
    assert _enc(desc, st=3) == INVALID  # odd stride
    assert _enc(desc, sh=-2) == INVALID
    d256 = kvq.make_desc(256, 8, 1, 128, 128, 64)
    assert _enc(d256) == UNSUPPORTED
    assert lib.kvq_encode(None, FAKE, FAKE, FAKE, 0, 0, 0, 0, 0, 1, None) == INVALID


def test_decode_validation():
    desc = kvq.make_desc(64, 2, 1, 64, 128, 64)
    dec = lambda **kw: lib.kvq_decode(ctypes.byref(desc), kw.get("cache", FAKE),
                                      kw.get("k", FAKE), kw.get("v", FAKE), kw.get("dt", 0),
                                      kw.get("t0", 0), kw.get("ntok", 1), None)
    assert dec(ntok=0) == OK
    assert dec(t0=60, ntok=5) == CAPACITY
    assert dec(k=None) == INVALID
    assert dec(dt=2) == INVALID
    assert dec(v=FAKE + 2) == INVALID
    assert dec(k=FAKE + 8) == INVALID  # outputs must be 16-byte aligned
    assert dec(cache=FAKE + 8) == INVALID  # so must the cache


def _attn(desc, hq=32, seq=100, ws=FAKE, ws_bytes=1 << 30, q=FAKE, out=FAKE, qdt=0, odt=0,
          cache=FAKE):
    return lib.kvq_attn_decode(ctypes.byref(desc), cache, q, qdt, hq, seq, 0.0, out, odt, ws,
                               ws_bytes, None)


def test_attention_validation():
    desc = kvq.make_desc(128, 8, 2, 256, 128, 64)
    assert _attn(desc, hq=36) == INVALID  # not a multiple of Hkv
    assert _attn(desc, hq=24) == UNSUPPORTED  # G = 3
    assert _attn(desc, hq=128) == UNSUPPORTED  # G = 16
    assert _attn(desc, seq=0) == INVALID
    assert _attn(desc, seq=257) == CAPACITY
    assert _attn(desc, ws=None) == WORKSPACE
    assert _attn(desc, ws=FAKE + 64) == WORKSPACE  # needs 256-byte alignment
    need = kvq.attn_workspace_bytes(desc, 32, 100)
    assert need > 0
    assert _attn(desc, ws_bytes=need - 1) == WORKSPACE
    assert _attn(desc, q=None) == INVALID
    assert _attn(desc, out=FAKE + 2) == INVALID
    assert _attn(desc, qdt=3) == INVALID
    assert _attn(desc, cache=None) == INVALID
    assert _attn(desc, cache=FAKE + 4) == INVALID  # cache must be 16-byte aligned
    # 5-bit key angle codes: attended through a copy re-packed at 6 bits, placed in the
    # workspace after the partials (2 tiles per (sequence, kv head) for 100 tokens), then
    # 256 bytes for the fused step's sequence lengths
    small = kvq.make_desc(128, 8, 2, 256, 32, 64)
    wide = kvq.make_desc(128, 8, 2, 256, 64, 64)
    extra = kvq.attn_workspace_bytes(small, 32, 100) - kvq.attn_workspace_bytes(wide, 32, 100)
    assert extra == 2 * 8 * 2 * kvq.tile_bytes(128, 64, 64) + 256
    assert _attn(small, ws_bytes=kvq.attn_workspace_bytes(small, 32, 100) - 1) == WORKSPACE
    # a paged pool is not served at these widths (rejected before any device work)
    paged = lambda desc: lib.kvq_attn_decode_paged(
        ctypes.byref(desc), FAKE, ctypes.byref(kvq.Paging(FAKE, 4, 10)), FAKE, 0, 32, None,
        100, 0.0, FAKE, 0, FAKE, 1 << 30, None)
    assert paged(small) == UNSUPPORTED
    assert paged(kvq.make_desc(128, 8, 2, 256, 128, 17)) == UNSUPPORTED  # 5-bit value codes
    d64 = kvq.make_desc(64, 4, 1, 256, 256, 33)  # 8-bit / 6-bit: supported shape
    assert _attn(d64, hq=32, ws=None) == WORKSPACE


def test_split_plan_covers_sequence_without_empty_splits():
    for bsz, hkv, seq in [(1, 1, 1), (1, 1, 64), (1, 4, 4096), (4, 8, 32768), (1, 8, 131072),
                          (64, 8, 8192), (3, 2, 1000), (1, 1, 65)]:
        desc = kvq.make_desc(128, hkv, bsz, seq, 128, 64)
        s = kvq.attn_num_splits(desc, hkv, seq)
        ntiles = (seq + 63) // 64
        assert 1 <= s <= ntiles
        tps = -(-ntiles // s)
        assert (s - 1) * tps < ntiles <= s * tps  # last split is non-empty
        assert kvq.attn_workspace_bytes(desc, hkv * 4, seq) >= 4 * bsz * hkv * 4 * s * 130


def test_layer_signs_validation():
    buf = (ctypes.c_int8 * 8)()
    assert lib.kvq_layer_signs(0, 0, 6, buf) == INVALID
    assert lib.kvq_layer_signs(0, 0, 8, None) == INVALID
    assert lib.kvq_layer_signs(0, 0, 8, buf) == OK
    assert set(np.array(buf)) <= {-1, 1}


def _varlen(desc, hq=32, lens=FAKE, maxlen=100, ws=FAKE, ws_bytes=1 << 30, q=FAKE, out=FAKE,
            cache=FAKE):
    return lib.kvq_attn_decode_varlen(ctypes.byref(desc), cache, q, 0, hq, lens, maxlen, 0.0,
                                      out, 0, ws, ws_bytes, None)


def test_attention_varlen_validation():
    desc = kvq.make_desc(128, 8, 2, 256, 128, 64)
    assert _varlen(desc, lens=None) == INVALID
    assert _varlen(desc, lens=FAKE + 2) == INVALID  # uint32 lengths: 4-byte aligned
    assert _varlen(desc, maxlen=0) == INVALID
    assert _varlen(desc, maxlen=257) == CAPACITY
    assert _varlen(desc, lens=None, maxlen=257) == CAPACITY  # shape errors first
    assert _varlen(desc, hq=24) == UNSUPPORTED
    assert _varlen(desc, ws=None) == WORKSPACE
    assert _varlen(desc, cache=FAKE + 4) == INVALID
    assert _varlen(desc, q=None) == INVALID
    # the workspace needed is that of the fixed-length call at max_seq_len
    need = kvq.attn_workspace_bytes(desc, 32, 200)
    assert _varlen(desc, maxlen=200, ws_bytes=need - 1) == WORKSPACE


def _app(desc, cache=FAKE, k=FAKE, v=FAKE, dtype=0, sb=0, sh=0, pos=FAKE):
    return lib.kvq_append(ctypes.byref(desc), cache, k, v, dtype, sb, sh, pos, None)


def test_append_validation():
    desc = kvq.make_desc(128, 8, 2, 256, 128, 64)
    assert _app(desc, pos=None) == INVALID
    assert _app(desc, pos=FAKE + 2) == INVALID
    assert _app(desc, cache=None) == INVALID
    assert _app(desc, cache=FAKE + 8) == INVALID
    assert _app(desc, k=FAKE + 2) == INVALID
    assert _app(desc, dtype=1, v=FAKE + 4) == INVALID
    assert _app(desc, dtype=5) == INVALID
    assert _app(desc, sb=3) == INVALID
    assert _app(desc, sh=-2) == INVALID
    assert _app(kvq.make_desc(256, 8, 1, 128, 128, 64)) == UNSUPPORTED
    assert lib.kvq_append(None, FAKE, FAKE, FAKE, 0, 0, 0, FAKE, None) == INVALID


def _multi(desc, hq=32, nq=4, seq=100, ws=FAKE, ws_bytes=1 << 30, q=FAKE, out=FAKE, cache=FAKE):
    return lib.kvq_attn_multi(ctypes.byref(desc), cache, q, 0, hq, nq, seq, 0.0, out, 0, ws,
                              ws_bytes, None)


def test_attention_multi_validation():
    desc = kvq.make_desc(128, 8, 2, 256, 128, 64)
    assert _multi(desc, nq=0) == INVALID
    assert _multi(desc, nq=101, seq=100) == INVALID  # more queries than cached tokens
    assert _multi(desc, seq=257) == CAPACITY
    assert _multi(desc, hq=36) == INVALID
    assert _multi(desc, hq=24) == UNSUPPORTED  # G = 3
    assert _multi(desc, nq=9) == UNSUPPORTED  # 9 * 4 rows > 32
    assert _multi(desc, ws=None) == WORKSPACE
    need = kvq.attn_multi_workspace_bytes(desc, 32, 4, 100)
    assert need > 0
    assert _multi(desc, ws_bytes=need - 1) == WORKSPACE
    assert _multi(desc, cache=FAKE + 4) == INVALID
    assert _multi(desc, q=FAKE + 2) == INVALID
    # 5-bit key codes: the widened copy follows the partials in the workspace
    small = kvq.make_desc(128, 8, 2, 256, 32, 64)
    wide = kvq.make_desc(128, 8, 2, 256, 64, 64)
    assert (kvq.attn_multi_workspace_bytes(small, 32, 4, 100)
            - kvq.attn_multi_workspace_bytes(wide, 32, 4, 100)) == 2 * 8 * 2 * kvq.tile_bytes(128, 64, 64)
    assert lib.kvq_attn_multi_paged(ctypes.byref(small), FAKE, ctypes.byref(kvq.Paging(FAKE, 4, 10)),
                                    FAKE, 0, 32, 4, None, 100, 0.0, FAKE, 0, FAKE, 1 << 30,
                                    None) == UNSUPPORTED
    assert kvq.attn_multi_workspace_bytes(desc, 32, 9, 100) == 0


def test_paged_validation():
    desc = kvq.make_desc(128, 8, 2, 256, 128, 64)  # 4 tiles per sequence
    pg = kvq.Paging(FAKE, 4, 10)
    enc = lambda paging, **kw: lib.kvq_encode_paged(ctypes.byref(desc), kw.get("pool", FAKE),
                                                    paging, FAKE, FAKE, 0, 0, 0, 0, 0, 1, None)
    assert enc(None) == INVALID
    assert enc(ctypes.byref(kvq.Paging(None, 4, 10))) == INVALID
    assert enc(ctypes.byref(kvq.Paging(FAKE + 2, 4, 10))) == INVALID  # int32 table alignment
    assert enc(ctypes.byref(kvq.Paging(FAKE, 3, 10))) == INVALID  # fewer pages than tiles
    assert enc(ctypes.byref(kvq.Paging(FAKE, 4, 0))) == INVALID  # empty pool
    assert enc(ctypes.byref(pg), pool=FAKE + 8) == INVALID
    assert lib.kvq_attn_decode_paged(ctypes.byref(desc), FAKE, ctypes.byref(pg), FAKE, 0, 32,
                                     FAKE + 2, 100, 0.0, FAKE, 0, FAKE, 1 << 30, None) == INVALID
    assert lib.kvq_attn_decode_paged(ctypes.byref(desc), FAKE, None, FAKE, 0, 32, None, 100,
                                     0.0, FAKE, 0, FAKE, 1 << 30, None) == INVALID
    assert lib.kvq_decode_paged(ctypes.byref(desc), FAKE, ctypes.byref(pg), FAKE, FAKE, 0, 0, 0,
                                None) == OK  # nothing to do
    assert kvq.paged_pool_bytes(desc, 10) == 10 * 8 * kvq.tile_bytes(128, 128, 64)
    multi = lambda paging, **kw: lib.kvq_attn_multi_paged(
        ctypes.byref(desc), FAKE, paging, FAKE, 0, 32, kw.get("nq", 4), kw.get("lens"), 100, 0.0,
        FAKE, 0, FAKE, 1 << 30, None)
    assert multi(None) == INVALID
    assert multi(ctypes.byref(kvq.Paging(FAKE, 3, 10))) == INVALID
    assert multi(ctypes.byref(pg), nq=0) == INVALID
    assert multi(ctypes.byref(pg), lens=FAKE + 2) == INVALID


def test_attention_multi_varlen_validation():
    desc = kvq.make_desc(128, 8, 2, 256, 128, 64)
    mv = lambda **kw: lib.kvq_attn_multi_varlen(
        ctypes.byref(desc), FAKE, FAKE, 0, kw.get("hq", 32), kw.get("nq", 4), kw.get("lens", FAKE),
        kw.get("maxlen", 100), 0.0, FAKE, 0, FAKE, 1 << 30, None)
    assert mv(lens=None) == INVALID
    assert mv(lens=FAKE + 2) == INVALID
    assert mv(maxlen=257) == CAPACITY
    assert mv(lens=None, maxlen=257) == CAPACITY  # shape errors first
    assert mv(nq=101) == INVALID
    assert mv(hq=24) == UNSUPPORTED


def _fused(desc, cache=FAKE, paging=None, k=FAKE, v=FAKE, dtype=0, sb=0, sh=0, pos=FAKE, q=FAKE,
           hq=32, maxlen=100, out=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return lib.kvq_attn_decode_append(ctypes.byref(desc), cache, paging, k, v, dtype, sb, sh, pos,
                                      q, 0, hq, maxlen, 0.0, out, 0, ws, ws_bytes, None)


def test_fused_append_attention_validation():
    desc = kvq.make_desc(128, 8, 2, 256, 128, 64)
    assert _fused(desc, pos=None) == INVALID
    assert _fused(desc, pos=FAKE + 2) == INVALID
    assert _fused(desc, k=None) == INVALID
    assert _fused(desc, k=FAKE + 2) == INVALID
    assert _fused(desc, dtype=1, v=FAKE + 4) == INVALID
    assert _fused(desc, dtype=7) == INVALID
    assert _fused(desc, sb=5) == INVALID
    assert _fused(desc, sh=-2) == INVALID
    assert _fused(desc, maxlen=0) == INVALID
    assert _fused(desc, maxlen=257) == CAPACITY
    assert _fused(desc, pos=None, maxlen=257) == CAPACITY  # shape errors first
    assert _fused(desc, hq=24) == UNSUPPORTED
    assert _fused(desc, ws=None) == WORKSPACE
    assert _fused(desc, ws_bytes=kvq.attn_workspace_bytes(desc, 32, 100) - 1) == WORKSPACE
    assert _fused(desc, cache=FAKE + 4) == INVALID
    assert _fused(desc, q=None) == INVALID
    assert _fused(desc, paging=ctypes.byref(kvq.Paging(None, 4, 10))) == INVALID
    assert _fused(desc, paging=ctypes.byref(kvq.Paging(FAKE, 3, 10))) == INVALID
    # narrow codebooks: served on a contiguous cache (append, then the widened copy),
    # not on a paged pool
    pg4 = ctypes.byref(kvq.Paging(FAKE, 4, 10))
    assert _fused(kvq.make_desc(128, 8, 2, 256, 32, 64), paging=pg4) == UNSUPPORTED  # 5-bit K
    assert _fused(kvq.make_desc(128, 8, 2, 256, 128, 3), paging=pg4) == UNSUPPORTED  # 2-bit V
    narrow = kvq.make_desc(128, 8, 2, 256, 32, 64)
    assert _fused(narrow, ws_bytes=kvq.attn_workspace_bytes(narrow, 32, 100) - 1) == WORKSPACE
    assert _fused(narrow, q=None) == INVALID


def test_static_scratch_entry_point_rejects_before_any_device_work():
    """kvq_attn_decode_static: argument errors and shapes whose workspace exceeds the
    fixed scratch array are rejected on the host (no HIP call is reached)."""
    assert kvq.attn_static_scratch_bytes() == 8 << 20
    f = lib.kvq_attn_decode_static
    small = kvq.make_desc(128, 2, 1, 256, 128, 64)
    assert f(ctypes.byref(small), FAKE, None, 0, 8, 256, 0.0, FAKE, 0, None) == INVALID
    assert f(ctypes.byref(small), FAKE + 8, FAKE, 0, 8, 256, 0.0, FAKE, 0, None) == INVALID
    assert f(ctypes.byref(small), FAKE, FAKE, 0, 8, 300, 0.0, FAKE, 0, None) == CAPACITY
    assert f(ctypes.byref(small), FAKE, FAKE, 0, 48, 256, 0.0, FAKE, 0, None) == UNSUPPORTED
    # 256 sequences x 8 kv heads x 64 query heads: partials of 16 MiB > 8 MiB
    big = kvq.make_desc(128, 8, 256, 8192, 128, 64)
    need = kvq.attn_workspace_bytes(big, 64, 8192)
    assert need > kvq.attn_static_scratch_bytes()
    assert f(ctypes.byref(big), FAKE, FAKE, 0, 64, 8192, 0.0, FAKE, 0, None) == WORKSPACE


def test_sizes_are_zero_for_shapes_attention_does_not_serve():
    """Workspace and split helpers agree with kvq_attn_decode: 0 where it would return
    UNSUPPORTED (G = 16, d = 256) or INVALID; narrow codebooks are served."""
    ok = kvq.make_desc(128, 2, 1, 256, 128, 64)
    assert kvq.attn_workspace_bytes(ok, 8, 256) > 0
    for nk, nv in ((32, 64), (128, 17), (2, 2)):  # 5-bit keys, 5-bit values, 1-bit both
        narrow = kvq.make_desc(128, 2, 1, 256, nk, nv)
        assert kvq.attn_workspace_bytes(narrow, 8, 256) > kvq.attn_workspace_bytes(ok, 8, 256)
        assert kvq.attn_num_splits(narrow, 8, 256) > 0
    for desc, hq in ((kvq.make_desc(128, 2, 1, 256, 128, 64), 32),   # G = 16
                     (kvq.make_desc(256, 2, 1, 256, 128, 64), 8),    # d = 256
                     (kvq.make_desc(128, 2, 1, 256, 128, 64), 7)):   # Hq not a multiple
        assert kvq.attn_workspace_bytes(desc, hq, 256) == 0
        assert kvq.attn_num_splits(desc, hq, 256) == 0
    assert kvq.tile_bytes(32, 128, 64) == 0  # d = 32: key bit strings would split words


def test_workspace_helper_reports_the_shape_status():
    with pytest.raises(kvq.KvqError, match="UNSUPPORTED"):
        kvq.alloc_workspace(kvq.make_desc(128, 2, 1, 256, 128, 64), 32, 256, "cpu")  # G = 16
    with pytest.raises(kvq.KvqError, match="CAPACITY"):
        kvq.alloc_workspace(kvq.make_desc(128, 2, 1, 256, 128, 64), 8, 300, "cpu")


def test_probe_read_validation():
    lib = kvq.lib
    p = ctypes.c_void_p(4096)     # never dereferenced: each call fails its checks first
    assert lib.kvq_probe_read(None, 16, p, None) == 1
    assert lib.kvq_probe_read(p, 16, None, None) == 1
    assert lib.kvq_probe_read(ctypes.c_void_p(4104), 16, p, None) == 1   # not 16-aligned
    assert lib.kvq_probe_read(p, 24, p, None) == 1                       # not a multiple of 16
    assert lib.kvq_probe_read(p, 0, p, None) == 0                        # nothing to read
