"""Host-side checks of the triplet codec's library entry points (no GPU needed):
record and tile sizes against the layout definition, the library's Lloyd-Max tables
against the oracle's, and argument rejection before any device work."""

import ctypes

import numpy as np
import pytest

import rotated_angle_quantization_amd as kvq
from oracle import layout, triplet

CONFIGS = [(128, 4, 2, 3), (128, 3, 3, 3), (64, 2, 2, 2), (64, 6, 6, 7), (128, 1, 1, 1)]


@pytest.mark.parametrize("d,bd,bn,br", CONFIGS)
def test_sizes_match_layout_definition(d, bd, bn, br):
    desc = kvq.make_tri_desc(d, 3, 2, 130, bd, bn, br)
    assert kvq.tri_record_words(desc) == layout.tri_record_words(d, bd, bn, br)
    assert kvq.tri_tile_bytes(desc) == layout.tri_tile_bytes(d, bd, bn, br)
    assert kvq.tri_cache_bytes(desc) == 2 * 3 * 3 * layout.tri_tile_bytes(d, bd, bn, br)
    bits = triplet.record_bits(d, bd, bn, br)
    assert kvq.tri_record_words(desc) == -(-bits // 32)


@pytest.mark.parametrize("d,bd,bn,br", CONFIGS)
def test_library_codebook_equals_oracle_lloyd_max(d, bd, bn, br):
    """Both sides solve the same fixed-point problem (centroid condition on the closed-form
    marginals) independently; they must meet to well below any decision's resolution."""
    table = kvq.tri_codebook(kvq.make_tri_desc(d, 1, 1, 64, bd, bn, br))
    cb = triplet.Codebook(d, bd, bn, br)
    want = np.concatenate([cb.dir_levels, cb.norm_levels, cb.rest_levels,
                           cb.dir_bounds, cb.norm_bounds, cb.rest_bounds])
    assert table.shape == want.shape
    np.testing.assert_allclose(table, want, rtol=0, atol=1e-10)
    # ascending within each set, symmetric sets odd about zero
    n = [1 << bd, 1 << bn, 1 << br]
    off = 0
    for k in n:
        lev = table[off:off + k]
        assert np.all(np.diff(lev) > 0)
        off += k
    lev_dir = table[:n[0]]
    np.testing.assert_allclose(lev_dir, -lev_dir[::-1], atol=1e-15)


@pytest.mark.parametrize("d,kind_bits", [(128, (("oct", 6), ("norm", 6), ("coord", 8))),
                                         (64, (("oct", 3), ("norm", 2), ("coord", 5)))])
def test_library_levels_satisfy_centroid_conditions(d, kind_bits):
    """Independent of either side's iteration: every library level is the conditional mean
    of its cell under the oracle's marginal, cells bounded by the library's midpoints."""
    (_, bd), (_, bn), (_, br) = kind_bits
    table = kvq.tri_codebook(kvq.make_tri_desc(d, 1, 1, 64, bd, bn, br))
    off = 0
    for kind, bits in kind_bits:
        n = 1 << bits
        lev = table[off:off + n]
        off += n
        lo, hi, splits = triplet._support(kind)
        mid = 0.5 * (lev[:-1] + lev[1:])
        a = np.concatenate([[lo], mid])
        b = np.concatenate([mid, [hi]])
        mass, mom = triplet._cell_integrals(triplet._density(kind, d), a, b, splits)
        np.testing.assert_allclose(mom / mass, lev, rtol=0, atol=1e-13, err_msg=kind)


def test_invalid_descriptors_size_zero():
    bad = [kvq.make_tri_desc(96, 1, 1, 64, 2, 2, 2), kvq.make_tri_desc(128, 1, 1, 64, 0, 2, 2),
           kvq.make_tri_desc(128, 1, 1, 64, 7, 2, 2), kvq.make_tri_desc(128, 1, 1, 64, 2, 7, 2),
           kvq.make_tri_desc(128, 1, 1, 64, 2, 2, 9), kvq.make_tri_desc(128, 0, 1, 64, 2, 2, 2),
           kvq.make_tri_desc(128, 1, 0, 64, 2, 2, 2), kvq.make_tri_desc(128, 1, 1, 0, 2, 2, 2),
           kvq.make_tri_desc(128, 1, 1, 2**31 - 63, 2, 2, 2)]
    for desc in bad:
        assert kvq.tri_cache_bytes(desc) == 0, desc
        assert kvq.tri_record_words(desc) == 0, desc
        assert kvq.lib.kvq_tri_codebook_doubles(ctypes.byref(desc)) == 0, desc


def test_attention_workspace_zero_for_unserved_shapes():
    desc = kvq.make_tri_desc(128, 2, 1, 256, 4, 2, 3)
    assert kvq.tri_attn_workspace_bytes(desc, 8, 100) > 0
    assert kvq.tri_attn_workspace_bytes(desc, 6, 100) == 0      # G = 3
    assert kvq.tri_attn_workspace_bytes(desc, 32, 100) == 0     # G = 16
    assert kvq.tri_attn_workspace_bytes(desc, 3, 100) == 0      # not a multiple of Hkv
    assert kvq.tri_attn_workspace_bytes(desc, 8, 0) == 0
    assert kvq.tri_attn_workspace_bytes(desc, 8, 257) == 0      # beyond capacity


def test_entry_points_reject_before_device_work():
    lib = kvq.lib
    desc = kvq.make_tri_desc(128, 2, 1, 256, 4, 2, 3)
    bad = kvq.make_tri_desc(100, 2, 1, 256, 4, 2, 3)
    p = ctypes.c_void_p(256)     # never dereferenced: every call below fails its checks first
    E_INV, E_CAP, E_UNS, E_WS = 1, 3, 2, 4
    st = lib.kvq_tri_encode(ctypes.byref(bad), p, p, p, p, 0, 0, 0, 0, 0, 1, None)
    assert st == E_INV
    st = lib.kvq_tri_encode(ctypes.byref(desc), p, p, p, p, 0, 0, 0, 0, 250, 10, None)
    assert st == E_CAP
    st = lib.kvq_tri_encode(ctypes.byref(desc), p, p, p, p, 7, 0, 0, 0, 0, 1, None)
    assert st == E_INV
    st = lib.kvq_tri_encode(ctypes.byref(desc), None, p, p, p, 0, 0, 0, 0, 0, 1, None)
    assert st == E_INV
    assert lib.kvq_tri_encode(ctypes.byref(desc), None, None, None, None, 0, 0, 0, 0, 0, 0,
                              None) == 0      # empty range: nothing to do
    st = lib.kvq_tri_decode(ctypes.byref(desc), p, p, p, p, 0, 200, 100, None)
    assert st == E_CAP
    st = lib.kvq_tri_attn_decode(ctypes.byref(desc), p, p, p, 0, 6, 10, 0.0, p, 0, p, 1 << 20,
                                 None)
    assert st == E_UNS
    st = lib.kvq_tri_attn_decode(ctypes.byref(desc), p, p, p, 0, 8, 300, 0.0, p, 0, p, 1 << 20,
                                 None)
    assert st == E_CAP
    st = lib.kvq_tri_attn_decode(ctypes.byref(desc), p, p, p, 0, 8, 10, 0.0, p, 0, p, 16, None)
    assert st == E_WS
