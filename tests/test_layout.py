"""Pins for the oracle's packer/unpacker: hand-derived words, round trips and sizes."""

import numpy as np
import pytest

from conftest import read_golden
from oracle import layout as ol


def _token0_tile():
    d, p = 64, 32
    z = np.zeros((1, p), dtype=np.int64)
    k_angle = np.ones((1, p), dtype=np.int64)
    k_radius = np.arange(p)[None, :]
    v_angle = (np.arange(p)[None, :] % 2 == 0).astype(np.int64)
    v_radius = np.full((1, p), 15)
    del z
    return ol.pack_tile(d, 128, 64, k_angle, k_radius, np.array([1.0]), v_angle, v_radius,
                        np.array([0.5]), np.array([2.0]))


def test_hand_derived_words_d64():
    buf = _token0_tile()
    sizes = ol.plane_sizes(64, 128, 64)
    start, acc = {}, 0
    for name, sz in sizes.items():
        start[name] = acc
        acc += sz
    words = buf.view(np.uint32)
    for plane, idx, val in read_golden("layout_d64_words.txt"):
        got = int(words[start[plane] // 4 + int(idx)])
        assert got == int(val, 16), (plane, idx, hex(got))


@pytest.mark.parametrize("d,n_k,n_v", [(64, 128, 64), (128, 128, 64), (128, 256, 256),
                                       (128, 100, 40), (64, 2, 3), (256, 128, 64)])
def test_pack_unpack_round_trip(d, n_k, n_v):
    rng = np.random.default_rng(d + n_k + n_v)
    p = d // 2
    ntok = 50
    args = dict(
        k_angle=rng.integers(0, n_k, (ntok, p)), k_radius=rng.integers(0, 256, (ntok, p)),
        k_scale=rng.uniform(0, 100, ntok).astype(np.float16).astype(np.float64),
        v_angle=rng.integers(0, n_v, (ntok, p)), v_radius=rng.integers(0, 16, (ntok, p)),
        v_smin=rng.uniform(0, 1, ntok).astype(np.float16).astype(np.float64),
        v_smax=rng.uniform(1, 9, ntok).astype(np.float16).astype(np.float64))
    buf = ol.pack_tile(d, n_k, n_v, **args)
    assert buf.size == ol.tile_bytes(d, n_k, n_v)
    back = ol.unpack_tile(d, n_k, n_v, buf, ntok)
    for key, val in args.items():
        assert np.array_equal(back[key], val), key
    # unused slots are zero in a freshly packed tile
    assert not ol.unpack_tile(d, n_k, n_v, buf)["k_angle"][ntok:].any()


def test_tile_and_cache_sizes():
    for d, nk, nv, rec, _ in read_golden("bits_per_element.txt"):
        assert ol.tile_bytes(int(d), int(nk), int(nv)) == 64 * int(rec)
    # every plane starts on a 128-byte boundary for the supported shapes
    for d in (64, 128, 256):
        for nk in (64, 128, 256):
            for nv in (64, 128, 256):
                assert all(v % 128 == 0 for v in ol.plane_sizes(d, nk, nv).values())
    assert ol.cache_bytes(128, 128, 64, 4, 8, 32768) == 4 * 8 * 512 * 13184
    assert ol.cache_bytes(128, 128, 64, 1, 1, 65) == 2 * 13184
    with pytest.raises(ValueError):
        ol.plane_sizes(32, 128, 64)


def test_unpack_cache_ranges():
    rng = np.random.default_rng(3)
    d, nk, nv, bsz, hkv, cap = 64, 128, 64, 2, 2, 130
    p = d // 2
    tiles = 3
    tb = ol.tile_bytes(d, nk, nv)
    cache = np.zeros((bsz, hkv, tiles, tb), dtype=np.uint8)
    ref = {}
    for b in range(bsz):
        for h in range(hkv):
            for t in range(tiles):
                a = dict(k_angle=rng.integers(0, nk, (64, p)),
                         k_radius=rng.integers(0, 256, (64, p)),
                         k_scale=np.full(64, 1.5), v_angle=rng.integers(0, nv, (64, p)),
                         v_radius=rng.integers(0, 16, (64, p)),
                         v_smin=np.full(64, 0.25), v_smax=np.full(64, 3.0))
                cache[b, h, t] = ol.pack_tile(d, nk, nv, **a)
                ref[b, h, t] = a
    out = ol.unpack_cache(cache.reshape(-1), d, nk, nv, bsz, hkv, cap, 60, 70)
    for j in range(70):
        tok = 60 + j
        a = ref[1, 0, tok // 64]
        assert np.array_equal(out["k_angle"][1, j, 0], a["k_angle"][tok % 64])
        assert np.array_equal(out["v_radius"][1, j, 0], a["v_radius"][tok % 64])


def test_vectorised_unpack_matches_per_tile_unpack():
    rng = np.random.default_rng(11)
    for d, nk, nv in [(64, 128, 64), (128, 256, 256), (128, 100, 37)]:
        tb = ol.tile_bytes(d, nk, nv)
        tiles = rng.integers(0, 256, (3, tb), dtype=np.uint8)
        # keep the fp16 parameter planes finite
        fast = ol.unpack_tiles(tiles, d, nk, nv)
        for t in range(3):
            slow = ol.unpack_tile(d, nk, nv, tiles[t])
            for key in ("k_angle", "k_radius", "v_angle", "v_radius"):
                assert np.array_equal(fast[key][t], slow[key]), key
            for key in ("k_scale", "v_smin", "v_smax"):
                np.testing.assert_array_equal(fast[key][t], slow[key])
