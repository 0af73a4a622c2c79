"""Oracle for the angle-quantised KV-cache codec: plain, slow, float64 NumPy.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline leg of
the benchmark may import this module. The HIP library never calls it, links it or
shares code with it; the two agree only because both follow the same definitions.

The method is the one in "TurboAngle: Near-Lossless KV Cache Compression via Uniform
Angle Quantization" (arXiv 2603.27467), Abstract:
  * each cached vector gets a random sign diagonal, then a fast Walsh-Hadamard transform;
  * in that domain, adjacent coordinates taken two at a time become (radius, angle);
  * each angle is rounded to one of n evenly spaced directions, with n set per layer
    and independently for keys and values (the paper's per-layer early boost);
  * radii are coded with different precision for the two tensors: 8 bits for keys,
    4 bits on a logarithmic scale for values;
  * nothing is calibrated on data: each step acts on one vector and is fixed by a seed.

Where the abstract leaves a step open, the reading taken is stated next to the code.
The Walsh-Hadamard transform here is a dense Sylvester matrix product (no butterflies),
so that each step can be checked by eye against its definition.
"""

from __future__ import annotations

import math

import numpy as np

# ----------------------------------------------------------------------------------
# Seeded sign diagonal.
#
# The TurboAngle abstract randomises the basis with a diagonal of random signs; the
# summary of "OCTOPUS: Joint Triplet Quantization for KV Cache via Octahedral
# Parametrization" (Research angle) notes that this codec family is fixed once a seed
# is chosen, with no data-dependent state.
# Reading: one +-1 diagonal per layer, shared by K, V and all heads, drawn from the
# SplitMix64 output function (Steele, Lea and Flood, "Fast splittable pseudorandom
# number generators", OOPSLA 2014), a counter-based generator with a published
# definition. sign[i] = -1 iff bit 63 of mix(mix(seed XOR layer) + i) is set.
# ----------------------------------------------------------------------------------

MASK64 = (1 << 64) - 1
SPLITMIX_GAMMA = 0x9E3779B97F4A7C15


def splitmix64_mix(z: int) -> int:
    """SplitMix64 step: add the golden gamma, then the two xor-shift-multiply rounds.

    Arithmetic is modulo 2**64 on Python integers.
    """
    z = (z + SPLITMIX_GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def layer_signs(seed: int, layer: int, d: int) -> np.ndarray:
    """The per-layer random sign diagonal sigma_l, as float64 +-1 of length d."""
    base = splitmix64_mix((seed ^ layer) & MASK64)
    out = np.empty(d, dtype=np.float64)
    for i in range(d):
        out[i] = -1.0 if (splitmix64_mix((base + i) & MASK64) >> 63) else 1.0
    return out


# ----------------------------------------------------------------------------------
# Walsh-Hadamard domain: the angles are taken after the fast Walsh-Hadamard transform
# (TurboAngle, Abstract).
# ----------------------------------------------------------------------------------


def hadamard(d: int) -> np.ndarray:
    """Dense Sylvester-Hadamard matrix: H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]."""
    if d < 1 or d & (d - 1):
        raise ValueError(f"head dimension must be a power of two, got {d}")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def inv_sqrt_d(d: int) -> float:
    """The normalisation factor 1/sqrt(d), rounded once to float64.

    Reading: the normalised transform is applied as one multiplication by this value.
    """
    return 1.0 / math.sqrt(d)


def rotate(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """y = H_d (sigma * x) / sqrt(d), natural (Sylvester) order, along the last axis."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the codec's contract")
    d = x.shape[-1]
    h = hadamard(d)
    return ((x * signs) @ h.T) * inv_sqrt_d(d)


def unrotate(y: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Inverse of rotate: x = sigma * (H_d y) / sqrt(d) (H is symmetric, H H = d I)."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    h = hadamard(d)
    return ((y @ h.T) * inv_sqrt_d(d)) * signs


# ----------------------------------------------------------------------------------
# Pairs -> polar. After the rotation, each pair of neighbouring coordinates is close
# to uniform in direction (TurboAngle, Abstract), which is why a uniform angle grid is
# used. Reading: pair i is (y[2i], y[2i+1]); angle = atan2(odd, even).
# ----------------------------------------------------------------------------------


def polar(y: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Return (r, theta) per consecutive pair; theta in (-pi, pi]."""
    a = y[..., 0::2]
    b = y[..., 1::2]
    return np.hypot(a, b), np.arctan2(b, a)


def code_bits(n: int) -> int:
    """Width of one angle code: ceil(log2 n) bits, for n in [2, 256]."""
    if not 2 <= n <= 256:
        raise ValueError(f"angle bin count must be in [2, 256], got {n}")
    return (n - 1).bit_length()


def angle_position(theta: np.ndarray, n: int) -> np.ndarray:
    """t = theta * n / (2 pi): the angle measured in bin widths (reading: n / (2 pi)
    is formed first, then one multiplication)."""
    return theta * (n / (2.0 * math.pi))


def angle_codes(r: np.ndarray, theta: np.ndarray, n: int) -> np.ndarray:
    """Uniform angle quantiser with n bins.

    Reading: bin centres sit at 2 pi k / n (k = 0 on the positive even axis) and each
    angle goes to the nearest centre, c = floor(t + 1/2) mod n. A zero pair gets
    code 0, since its angle is undefined.
    """
    t = angle_position(theta, n)
    c = np.mod(np.floor(t + 0.5), n).astype(np.int64)
    return np.where(r == 0.0, 0, c)


def angle_near_boundary(theta: np.ndarray, n: int, tol: float = 1e-6) -> np.ndarray:
    """True where theta lies within `tol` radians of a bin boundary ((k + 1/2) 2 pi / n)."""
    t = angle_position(theta, n)
    frac = t - np.floor(t)
    return (2.0 * math.pi / n) * np.abs(frac - 0.5) < tol


def angle_centres(n: int) -> np.ndarray:
    """Reconstruction angles 2 pi c / n for c = 0 .. n-1."""
    return 2.0 * math.pi * np.arange(n, dtype=np.float64) / n


# ----------------------------------------------------------------------------------
# Norm quantisation (TurboAngle, Abstract): key radii get 8 linear bits, value radii
# 4 bits on a log scale. Readings: per-vector parameters are stored as IEEE fp16 (round to
# nearest even, saturated at the largest finite fp16, 65504); the stored fp16 values
# are the ones used to encode, so encoder and decoder agree.
# ----------------------------------------------------------------------------------

FP16_MAX = 65504.0
FP16_MIN_NORMAL = 2.0 ** -14
K_RADIUS_LEVELS = 255  # 8 bits: codes 0..255
V_RADIUS_LEVELS = 15  # 4 bits: codes 0..15


def fp16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest fp16 value (ties to even), saturating at 65504."""
    x = np.minimum(np.asarray(x, dtype=np.float64), FP16_MAX)
    return x.astype(np.float16).astype(np.float64)


def k_radius_encode(r: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Key norms: 8-bit linear on [0, s], s = fp16(max r) per vector.

    Reading: 256 levels c * s / 255 (both 0 and s included), nearest level by
    floor(255 r / s + 1/2), clamped to [0, 255]; s = 0 gives all-zero codes.
    Returns (s, rho) with s of shape [...], rho of shape [..., P].
    """
    s = fp16_round(np.max(r, axis=-1))
    safe = np.where(s > 0.0, s, 1.0)[..., None]
    rho = np.clip(np.floor(K_RADIUS_LEVELS * r / safe + 0.5), 0, K_RADIUS_LEVELS)
    rho = np.where((s > 0.0)[..., None], rho, 0.0)
    return s, rho.astype(np.int64)


def k_radius_decode(s: np.ndarray, rho: np.ndarray) -> np.ndarray:
    return rho * (np.asarray(s, dtype=np.float64)[..., None] / K_RADIUS_LEVELS)


def v_radius_encode(r: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Value norms: 4 bits uniform in log space between the per-vector min and max.

    Readings: s_max = fp16(max r); s_min = fp16(max(min r, 2^-14)) (the floor is the
    smallest normal fp16 and keeps the logarithm finite for zero pairs); 16 levels
    s_min * exp(k L / 15) with L = ln(s_max / s_min); nearest level in log space,
    floor(15 ln(r / s_min) / L + 1/2) clamped to [0, 15]; r below s_min -> code 0;
    s_max <= s_min (a flat or tiny vector) -> all codes 0, reconstructed as s_max.
    Returns (s_min, s_max, rho).
    """
    s_max = fp16_round(np.max(r, axis=-1))
    s_min = fp16_round(np.maximum(np.min(r, axis=-1), FP16_MIN_NORMAL))
    degenerate = s_max <= s_min
    lam = np.log(np.where(degenerate, 2.0, s_max) / np.where(degenerate, 1.0, s_min))
    ratio = np.where(r < s_min[..., None], 1.0, r / s_min[..., None])
    rho = np.floor(V_RADIUS_LEVELS * np.log(ratio) / lam[..., None] + 0.5)
    rho = np.clip(rho, 0, V_RADIUS_LEVELS)
    rho = np.where(r < s_min[..., None], 0.0, rho)
    rho = np.where(degenerate[..., None], 0.0, rho)
    return s_min, s_max, rho.astype(np.int64)


def v_radius_decode(s_min: np.ndarray, s_max: np.ndarray, rho: np.ndarray) -> np.ndarray:
    s_min = np.asarray(s_min, dtype=np.float64)
    s_max = np.asarray(s_max, dtype=np.float64)
    degenerate = s_max <= s_min
    lam = np.log(np.where(degenerate, 2.0, s_max) / np.where(degenerate, 1.0, s_min))
    r_hat = s_min[..., None] * np.exp(rho * lam[..., None] / V_RADIUS_LEVELS)
    return np.where(degenerate[..., None], s_max[..., None], r_hat)


# ----------------------------------------------------------------------------------
# Whole-vector encode / decode.
# ----------------------------------------------------------------------------------


def encode_k(x: np.ndarray, signs: np.ndarray, n: int) -> dict:
    """Encode key vectors x[..., d]. Returns angle codes, radius codes, fp16 scale,
    plus the float64 intermediates the parity rules need (theta, boundary flags)."""
    y = rotate(x, signs)
    r, theta = polar(y)
    c = angle_codes(r, theta, n)
    s, rho = k_radius_encode(r)
    return {"angle": c, "radius": rho, "scale": s, "theta": theta, "r": r,
            "near_boundary": angle_near_boundary(theta, n) & (r != 0.0)}


def encode_v(x: np.ndarray, signs: np.ndarray, n: int) -> dict:
    """Encode value vectors x[..., d]. Returns angle codes, log-radius codes and the
    fp16 (s_min, s_max) pair, plus float64 intermediates."""
    y = rotate(x, signs)
    r, theta = polar(y)
    c = angle_codes(r, theta, n)
    s_min, s_max, rho = v_radius_encode(r)
    return {"angle": c, "radius": rho, "s_min": s_min, "s_max": s_max, "theta": theta,
            "r": r, "near_boundary": angle_near_boundary(theta, n) & (r != 0.0)}


def pairs_from_polar(r_hat: np.ndarray, c: np.ndarray, n: int) -> np.ndarray:
    """Rotated-domain reconstruction: y_hat[2i] = r cos, y_hat[2i+1] = r sin."""
    ang = angle_centres(n)[c]
    out = np.empty(r_hat.shape[:-1] + (2 * r_hat.shape[-1],), dtype=np.float64)
    out[..., 0::2] = r_hat * np.cos(ang)
    out[..., 1::2] = r_hat * np.sin(ang)
    return out


def dequant_k_rotated(angle, radius, scale, n) -> np.ndarray:
    return pairs_from_polar(k_radius_decode(scale, radius), angle, n)


def dequant_v_rotated(angle, radius, s_min, s_max, n) -> np.ndarray:
    return pairs_from_polar(v_radius_decode(s_min, s_max, radius), angle, n)


def dequant_k(angle, radius, scale, n, signs) -> np.ndarray:
    """x_hat = sigma * H y_hat / sqrt(d) for keys."""
    return unrotate(dequant_k_rotated(angle, radius, scale, n), signs)


def dequant_v(angle, radius, s_min, s_max, n, signs) -> np.ndarray:
    """x_hat = sigma * H y_hat / sqrt(d) for values."""
    return unrotate(dequant_v_rotated(angle, radius, s_min, s_max, n), signs)


# ----------------------------------------------------------------------------------
# Attention over the compressed cache: the plain definition on dequantised vectors.
# Readings: softmax scale 1/sqrt(d) unless given; grouped-query attention maps query
# head h to kv head floor(h / G), G = Hq / Hkv; all seq_len cached tokens attend.
# ----------------------------------------------------------------------------------


def attention(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray,
              scale: float | None = None) -> np.ndarray:
    """Single-token decode attention.

    q: [B, Hq, d]; k_hat, v_hat: [B, L, Hkv, d] (already dequantised); returns [B, Hq, d].
    s_j = scale <q, k_j>; p = softmax(s) (max subtracted); o = sum_j p_j v_j.
    """
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q.shape
    hkv = k_hat.shape[2]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    g = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.empty((bsz, hq, d), dtype=np.float64)
    for b in range(bsz):
        for h in range(hq):
            kv = h // g
            s = scale * (k_hat[b, :, kv, :] @ q[b, h])
            p = np.exp(s - np.max(s))
            p /= np.sum(p)
            out[b, h] = p @ v_hat[b, :, kv, :]
    return out


def bits_per_element(d: int, n_k: int, n_v: int) -> float:
    """Stored bits per cached element (K and V together) for one token-head record:
    angle codes, 8-bit K radii, 4-bit V radii, one fp16 K scale, two fp16 V params."""
    p = d // 2
    bits = p * code_bits(n_k) + p * 8 + 16 + p * code_bits(n_v) + p * 4 + 32
    return bits / (2 * d)
