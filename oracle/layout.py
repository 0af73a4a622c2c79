"""Oracle-side packer/unpacker for the compressed-cache byte layout.

TEST INFRASTRUCTURE (same rules as oracle.codec): written independently of the HIP
library from the layout definition below, in plain Python/NumPy bit operations.

The TurboAngle abstract (arXiv 2603.27467) stores codes but fixes no byte format; the
format here is this library's own, chosen so that a 64-lane wave reads it coalesced.

Layout of one layer's cache: [batch][kv_head][tile][tile bytes], tile = 64 token slots,
tiles_per_seq = ceil(capacity / 64). P = d / 2 pairs, bk / bv = angle code widths.
One tile holds six planes, in this order:

  KA  key angle codes     token-major words: word w of token t at 4*(w*64 + t);
                          token t's bit string (P*bk bits, LSB first) holds pair i's
                          code in bits [i*bk, (i+1)*bk)
  KR  key radius codes    token-major words: word w of token t at 4*(w*64 + t);
                          byte j of word w is the 8-bit code of pair 4w + j
  KS  key scale           64 fp16 values, token t at byte 2t
  VA  value angle codes   pair-major words: word w of pair i at 4*(w*P + i);
                          pair i's bit string (64*bv bits, LSB first) holds token t's
                          code in bits [t*bv, (t+1)*bv)
  VR  value radius codes  pair-major words: word w of pair i at 4*(w*P + i);
                          token t's 4-bit code in bits [4t, 4t+4) of pair i's string
  VP  value parameters    64 x (s_min fp16, s_max fp16), token t at byte 4t

Bit strings are little-endian: bit b is bit (b mod 32) of word b // 32.
"""

from __future__ import annotations

import numpy as np

from .codec import code_bits

TILE = 64


def plane_sizes(d: int, n_k: int, n_v: int) -> dict:
    p = d // 2
    bk, bv = code_bits(n_k), code_bits(n_v)
    if (p * bk) % 32 or (p * bv) % 32 or p % 4:
        raise ValueError("layout needs P*bits to fill whole 32-bit words (d >= 64)")
    return {
        "KA": TILE * p * bk // 8,
        "KR": TILE * p,
        "KS": 2 * TILE,
        "VA": p * 2 * bv * 4,
        "VR": p * 8 * 4,
        "VP": 4 * TILE,
    }


def tile_bytes(d: int, n_k: int, n_v: int) -> int:
    return sum(plane_sizes(d, n_k, n_v).values())


def cache_bytes(d: int, n_k: int, n_v: int, batch: int, hkv: int, capacity: int) -> int:
    tiles = (capacity + TILE - 1) // TILE
    return batch * hkv * tiles * tile_bytes(d, n_k, n_v)


def _offsets(d, n_k, n_v):
    off, acc = {}, 0
    for k, v in plane_sizes(d, n_k, n_v).items():
        off[k] = acc
        acc += v
    return off


def _bits_to_words(codes: np.ndarray, width: int) -> np.ndarray:
    """Pack a 1-D array of codes into little-endian 32-bit words, LSB first."""
    nbits = len(codes) * width
    words = np.zeros((nbits + 31) // 32, dtype=np.uint64)
    for idx, c in enumerate(codes.astype(np.uint64)):
        pos = idx * width
        w, sh = pos // 32, pos % 32
        words[w] |= (c << np.uint64(sh)) & np.uint64(0xFFFFFFFF)
        if sh + width > 32:
            words[w + 1] |= c >> np.uint64(32 - sh)
    return words.astype(np.uint32)


def _words_to_bits(words: np.ndarray, width: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.int64)
    w64 = words.astype(np.uint64)
    mask = (1 << width) - 1
    for idx in range(count):
        pos = idx * width
        w, sh = pos // 32, pos % 32
        v = int(w64[w]) >> sh
        if sh + width > 32:
            v |= int(w64[w + 1]) << (32 - sh)
        out[idx] = v & mask
    return out


def pack_tile(d, n_k, n_v, k_angle, k_radius, k_scale, v_angle, v_radius, v_smin, v_smax):
    """Pack up to 64 tokens of one (batch, kv head) into one tile's bytes.

    k_angle, k_radius, v_angle, v_radius: int [ntok, P]; k_scale, v_smin, v_smax: [ntok]
    float values that are exactly representable in fp16. Slots >= ntok are zero.
    """
    p = d // 2
    bk, bv = code_bits(n_k), code_bits(n_v)
    ntok = k_angle.shape[0]
    off = _offsets(d, n_k, n_v)
    buf = np.zeros(tile_bytes(d, n_k, n_v), dtype=np.uint8)
    u32 = buf.view(np.uint32)

    wk = p * bk // 32
    for t in range(ntok):
        words = _bits_to_words(k_angle[t], bk)
        for w in range(wk):
            u32[(off["KA"] // 4) + w * TILE + t] = words[w]
        words = _bits_to_words(k_radius[t], 8)
        for w in range(p // 4):
            u32[(off["KR"] // 4) + w * TILE + t] = words[w]
    ks = np.zeros(TILE, dtype=np.float16)
    ks[:ntok] = np.asarray(k_scale, dtype=np.float64)
    buf[off["KS"]:off["KS"] + 2 * TILE] = ks.view(np.uint8)

    va = np.zeros((p, TILE), dtype=np.int64)
    vr = np.zeros((p, TILE), dtype=np.int64)
    va[:, :ntok] = v_angle.T
    vr[:, :ntok] = v_radius.T
    for i in range(p):
        words = _bits_to_words(va[i], bv)
        for w in range(2 * bv):
            u32[(off["VA"] // 4) + w * p + i] = words[w]
        words = _bits_to_words(vr[i], 4)
        for w in range(8):
            u32[(off["VR"] // 4) + w * p + i] = words[w]
    vp = np.zeros((TILE, 2), dtype=np.float16)
    vp[:ntok, 0] = np.asarray(v_smin, dtype=np.float64)
    vp[:ntok, 1] = np.asarray(v_smax, dtype=np.float64)
    buf[off["VP"]:off["VP"] + 4 * TILE] = vp.reshape(-1).view(np.uint8)
    return buf


def unpack_tile(d, n_k, n_v, buf, ntok=TILE) -> dict:
    """Inverse of pack_tile for the first ntok token slots of one tile."""
    p = d // 2
    bk, bv = code_bits(n_k), code_bits(n_v)
    off = _offsets(d, n_k, n_v)
    buf = np.ascontiguousarray(np.asarray(buf, dtype=np.uint8))
    u32 = buf.view(np.uint32)
    wk = p * bk // 32

    k_angle = np.empty((ntok, p), dtype=np.int64)
    k_radius = np.empty((ntok, p), dtype=np.int64)
    for t in range(ntok):
        words = np.array([u32[(off["KA"] // 4) + w * TILE + t] for w in range(wk)])
        k_angle[t] = _words_to_bits(words, bk, p)
        words = np.array([u32[(off["KR"] // 4) + w * TILE + t] for w in range(p // 4)])
        k_radius[t] = _words_to_bits(words, 8, p)
    k_scale = buf[off["KS"]:off["KS"] + 2 * TILE].view(np.float16)[:ntok].astype(np.float64)

    v_angle = np.empty((ntok, p), dtype=np.int64)
    v_radius = np.empty((ntok, p), dtype=np.int64)
    for i in range(p):
        words = np.array([u32[(off["VA"] // 4) + w * p + i] for w in range(2 * bv)])
        v_angle[:, i] = _words_to_bits(words, bv, TILE)[:ntok]
        words = np.array([u32[(off["VR"] // 4) + w * p + i] for w in range(8)])
        v_radius[:, i] = _words_to_bits(words, 4, TILE)[:ntok]
    vp = buf[off["VP"]:off["VP"] + 4 * TILE].view(np.float16).reshape(TILE, 2)
    return {
        "k_angle": k_angle, "k_radius": k_radius, "k_scale": k_scale,
        "v_angle": v_angle, "v_radius": v_radius,
        "v_smin": vp[:ntok, 0].astype(np.float64), "v_smax": vp[:ntok, 1].astype(np.float64),
    }


def _field(words: np.ndarray, pos: int, width: int) -> np.ndarray:
    """Field [pos, pos + width) of little-endian word strings along the last axis."""
    w, sh = pos // 32, pos % 32
    v = words[..., w].astype(np.uint64) >> np.uint64(sh)
    if sh + width > 32:
        v |= words[..., w + 1].astype(np.uint64) << np.uint64(32 - sh)
    return (v & np.uint64((1 << width) - 1)).astype(np.int64)


def unpack_tiles(tiles: np.ndarray, d, n_k, n_v) -> dict:
    """Vectorised unpack of whole tiles: tiles is uint8 [..., tile_bytes]; returns codes
    shaped [..., 64, P] and parameters [..., 64] (same definitions as unpack_tile)."""
    p = d // 2
    bk, bv = code_bits(n_k), code_bits(n_v)
    off = _offsets(d, n_k, n_v)
    sizes = plane_sizes(d, n_k, n_v)
    tiles = np.ascontiguousarray(tiles)
    lead = tiles.shape[:-1]

    def plane(name):
        return tiles[..., off[name]:off[name] + sizes[name]]

    ka = plane("KA").view(np.uint32).reshape(lead + (p * bk // 32, TILE))
    ka = np.swapaxes(ka, -1, -2)  # [..., token, word]
    kr = np.swapaxes(plane("KR").view(np.uint32).reshape(lead + (p // 4, TILE)), -1, -2)
    va = np.swapaxes(plane("VA").view(np.uint32).reshape(lead + (2 * bv, p)), -1, -2)
    vr = np.swapaxes(plane("VR").view(np.uint32).reshape(lead + (8, p)), -1, -2)
    out = {
        "k_angle": np.stack([_field(ka, i * bk, bk) for i in range(p)], axis=-1),
        "k_radius": np.stack([_field(kr, i * 8, 8) for i in range(p)], axis=-1),
        "v_angle": np.stack([_field(va, t * bv, bv) for t in range(TILE)], axis=-2),
        "v_radius": np.stack([_field(vr, t * 4, 4) for t in range(TILE)], axis=-2),
        "k_scale": plane("KS").view(np.float16).astype(np.float64),
    }
    vp = plane("VP").view(np.float16).reshape(lead + (TILE, 2)).astype(np.float64)
    out["v_smin"] = vp[..., 0]
    out["v_smax"] = vp[..., 1]
    return out


def unpack_cache(cache: np.ndarray, d, n_k, n_v, batch, hkv, capacity, t0, ntok) -> dict:
    """Unpack tokens [t0, t0 + ntok) of every (batch, kv head) from a whole layer's
    cache bytes. Returns arrays shaped [batch, ntok, hkv, P] (codes) / [batch, ntok, hkv]."""
    tb = tile_bytes(d, n_k, n_v)
    tiles = (capacity + TILE - 1) // TILE
    cache = np.asarray(cache, dtype=np.uint8).reshape(batch, hkv, tiles, tb)
    lo, hi = t0 // TILE, (t0 + ntok + TILE - 1) // TILE
    u = unpack_tiles(cache[:, :, lo:hi], d, n_k, n_v)
    out = {}
    for k, v in u.items():
        # [B, H, tiles, 64, ...] -> [B, tokens, H, ...]
        v = v.reshape((batch, hkv, (hi - lo) * TILE) + v.shape[4:])
        v = v[:, :, t0 - lo * TILE:t0 - lo * TILE + ntok]
        out[k] = np.ascontiguousarray(np.swapaxes(v, 1, 2))
    return out


# ----------------------------------------------------------------------------------
# Triplet codec records (the layout defined at kvq_tri_desc in include/kvq.h): one
# token-head record is a little-endian bit string of 32-bit words: the fp16 bits of the
# vector norm in [0, 16), then for triplet j < T = d // 3 the s code, t code and norm
# code (b_dir, b_dir, b_norm bits) at 16 + j (2 b_dir + b_norm), then the leftover codes
# (b_rest bits each); padded to whole words. A tile of 64 slots is the key plane then the
# value plane, each [word][slot] (word w of slot t at 4 (w * 64 + t)).
# ----------------------------------------------------------------------------------


def tri_record_words(d: int, b_dir: int, b_norm: int, b_rest: int) -> int:
    t = d // 3
    return -(-(16 + t * (2 * b_dir + b_norm) + (d - 3 * t) * b_rest) // 32)


def tri_tile_bytes(d, b_dir, b_norm, b_rest) -> int:
    return 2 * tri_record_words(d, b_dir, b_norm, b_rest) * TILE * 4


def tri_record_bits(codes: dict, d: int, b_dir: int, b_norm: int, b_rest: int) -> int:
    """One record as a Python integer (bit i = bit i of the record)."""
    t = d // 3
    width = 2 * b_dir + b_norm
    val = int(codes["scale_bits"])
    for j in range(t):
        f = int(codes["s_code"][j]) | (int(codes["t_code"][j]) << b_dir) | \
            (int(codes["norm_code"][j]) << (2 * b_dir))
        val |= f << (16 + j * width)
    for r in range(d - 3 * t):
        val |= int(codes["rest_code"][r]) << (16 + t * width + r * b_rest)
    return val


def tri_unpack_tiles(tiles: np.ndarray, d, b_dir, b_norm, b_rest) -> dict:
    """tiles: uint8 [..., tile_bytes] -> codes of both planes, arrays [..., 64, ...]:
    k_/v_ s_code, t_code, norm_code [.., 64, T], rest_code [.., 64, d - 3T],
    scale (fp16 values, float64) [.., 64]."""
    words = tri_record_words(d, b_dir, b_norm, b_rest)
    tb = tri_tile_bytes(d, b_dir, b_norm, b_rest)
    lead = tiles.shape[:-1]
    w32 = np.ascontiguousarray(tiles).reshape(-1, tb).view("<u4").reshape(-1, 2, words, TILE)
    t = d // 3
    width = 2 * b_dir + b_norm
    out = {}
    for p, name in ((0, "k"), (1, "v")):
        rec = w32[:, p].astype(np.uint64)  # [n, words, 64]

        def field(off, wd):
            wi, sh = off // 32, off % 32
            lo = rec[:, wi, :]
            hi = rec[:, wi + 1, :] if wi + 1 < words else np.zeros_like(lo)
            return (((hi << np.uint64(32)) | lo) >> np.uint64(sh)) & np.uint64((1 << wd) - 1)

        f = np.stack([field(16 + j * width, width) for j in range(t)], axis=-1).astype(np.int64)
        rest = [field(16 + t * width + r * b_rest, b_rest) for r in range(d - 3 * t)]
        out[f"{name}_s_code"] = (f & ((1 << b_dir) - 1)).reshape(lead + (TILE, t))
        out[f"{name}_t_code"] = ((f >> b_dir) & ((1 << b_dir) - 1)).reshape(lead + (TILE, t))
        out[f"{name}_norm_code"] = (f >> (2 * b_dir)).reshape(lead + (TILE, t))
        out[f"{name}_rest_code"] = np.stack(rest, axis=-1).astype(np.int64).reshape(lead + (TILE, d - 3 * t))
        bits = (rec[:, 0, :] & np.uint64(0xFFFF)).astype(np.uint16)
        out[f"{name}_scale"] = bits.view(np.float16).astype(np.float64).reshape(lead + (TILE,))
    return out


def tri_unpack_cache(cache, d, b_dir, b_norm, b_rest, batch, hkv, capacity, t0, ntok) -> dict:
    """Codes of tokens [t0, t0 + ntok) of a triplet-coded cache, arrays
    [batch, ntok, hkv, ...] (the token-major order of the inputs)."""
    tb = tri_tile_bytes(d, b_dir, b_norm, b_rest)
    tiles = -(-capacity // TILE)
    c = np.asarray(cache, dtype=np.uint8)[: batch * hkv * tiles * tb].reshape(batch, hkv, tiles, tb)
    u = tri_unpack_tiles(c, d, b_dir, b_norm, b_rest)
    out = {}
    for key, val in u.items():
        val = val.reshape((batch, hkv, tiles * TILE) + val.shape[4:])[:, :, t0:t0 + ntok]
        out[key] = np.moveaxis(val, 1, 2)
    return out
