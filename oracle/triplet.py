"""Oracle for the triplet (octahedral) KV-cache codec: plain, slow, float64 NumPy/SciPy.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline leg of
the benchmark may import this module. The HIP library never calls it, links it or
shares code with it; the two agree only because both follow the same definitions.

The method is the one summarised for "OCTOPUS: Joint Triplet Quantization for KV Cache
via Octahedral Parametrization" (TL;DR, What is new):
  * after the structured random rotation, the rotated coordinates are quantised three
    at a time instead of one at a time;
  * each triplet's direction is carried to the square [-1, 1]^2 by the octahedral
    parametrisation;
  * the two square coordinates and the triplet's norm are each Lloyd-Max quantised
    against the marginal distributions the implementation itself produces (not
    asymptotic ones);
  * the split of bits between direction and norm is not uniform and depends only on
    the head dimension;
  * nothing is fitted to data (data-oblivious, fixed by a seed: Research angle).

Readings of the steps the page leaves open (each is used below where it applies):
  R1 rotation: the angle codec's seeded sign diagonal and normalised Sylvester
     Walsh-Hadamard transform (codec.rotate), so both codecs share one rotated domain.
  R2 scale: N = ||y|| (= ||x||) is stored as fp16 (round to nearest even, saturating at
     65504); the triplets are taken from u = y / N, so every quantiser works on
     scale-free values. N = 0 gives u = 0.
  R3 grouping: triplet j is (u[3j], u[3j+1], u[3j+2]) for j < T = floor(d / 3); the
     d - 3T leftover coordinates (2 for d = 128, 1 for d = 64) are quantised one by one
     with their own Lloyd-Max quantiser.
  R4 octahedral map: the standard octahedral parametrisation: p = w / |w|_1; on the
     upper half (p3 >= 0) the square point is (p1, p2); the lower half is folded over
     the diamond's edges to ((1 - |p2|) sgn p1, (1 - |p1|) sgn p2) with sgn(0) = +1.
     The page calls the map equal-area and also says its Jacobian is only near-uniform;
     the standard map has the second property (its density is derived below), which is
     the plainest reading. A zero triplet maps to (0, 0).
  R5 marginals ("implementation-matched"): with the rotation, a generic vector's unit
     vector u behaves as uniform on the sphere S^(d-1); then a triplet's direction is
     uniform on S^2 independently of its norm, and the exact finite-d marginals are:
       octahedral coordinate s (and t): density f_oct below (closed form);
       triplet norm rho: rho^2 ~ Beta(3/2, (d - 3)/2);
       one coordinate: density proportional to (1 - u^2)^((d - 3)/2) on [-1, 1].
  R6 Lloyd-Max: 2^b levels; the decision boundaries are the midpoints of neighbouring
     levels and each level is the conditional mean of its cell. Iteration starts from
     the levels at the (i + 1/2) / 2^b quantiles and stops when no level moves by more
     than 1e-14. Cell integrals use 40-point Gauss-Legendre rules on each cell (cells
     are split at 0 for the octahedral density, whose derivative has a kink there).
     Quantisation picks the nearest level, the lower one at an exact midpoint.
  R7 bit allocation: b_dir bits for each square coordinate, b_norm for the norm,
     b_rest per leftover coordinate. For a per-triplet budget B = 2 b_dir + b_norm the
     split minimising the expected squared error of a unit-vector triplet under the
     fitted quantisers is taken (allocation()); it depends on d only through the norm
     marginal. b_rest = round(B / 3) (the same rate per coordinate).
  R8 reconstruction: triplet j -> N_hat * rho_hat * w_hat with w_hat the inverse
     octahedral map of (s_hat, t_hat) normalised to unit length; a leftover coordinate
     -> N_hat * u_hat; then the inverse rotation. N_hat is the stored fp16 value.
  R9 keys and values use the same codec and parameters.
"""

from __future__ import annotations

import math

import numpy as np
from scipy import special

from . import codec

FP16_MAX = 65504.0
GL_POINTS = 40
LLOYD_TOL = 1e-14
LLOYD_MAX_ITER = 200000


# ----------------------------------------------------------------------------------
# Octahedral parametrisation (R4)
# ----------------------------------------------------------------------------------


def _sgn(x: np.ndarray) -> np.ndarray:
    return np.where(x < 0.0, -1.0, 1.0)


def octa_encode(w: np.ndarray) -> np.ndarray:
    """Directions [..., 3] (any nonzero length) -> square points [..., 2]; zero -> (0, 0)."""
    w = np.asarray(w, dtype=np.float64)
    l1 = np.sum(np.abs(w), axis=-1, keepdims=True)
    p = w / np.where(l1 > 0.0, l1, 1.0)
    p1, p2, p3 = p[..., 0], p[..., 1], p[..., 2]
    s = np.where(p3 >= 0.0, p1, (1.0 - np.abs(p2)) * _sgn(p1))
    t = np.where(p3 >= 0.0, p2, (1.0 - np.abs(p1)) * _sgn(p2))
    return np.stack([s, t], axis=-1)


def octa_decode(st: np.ndarray) -> np.ndarray:
    """Square points [..., 2] -> unit directions [..., 3] (inverse of octa_encode)."""
    st = np.asarray(st, dtype=np.float64)
    s, t = st[..., 0], st[..., 1]
    z = 1.0 - np.abs(s) - np.abs(t)
    x = np.where(z >= 0.0, s, (1.0 - np.abs(t)) * _sgn(s))
    y = np.where(z >= 0.0, t, (1.0 - np.abs(s)) * _sgn(t))
    v = np.stack([x, y, z], axis=-1)
    return v / np.linalg.norm(v, axis=-1, keepdims=True)


def octa_density(s: np.ndarray, t: np.ndarray) -> np.ndarray:
    """Joint density of (s, t) on [-1, 1]^2 for a direction uniform on the sphere.

    On the diamond |s| + |t| <= 1 a square point is the point (s, t, 1 - |s| - |t|) of
    the octahedron; central projection of an octahedron face onto the unit sphere
    scales area by 1 / |p|^3 once the face is projected onto the (s, t) plane, so the
    density there is 1 / (4 pi |p|^3). The folded corners carry the lower half with the
    same density at the mirrored diamond point.
    """
    s = np.asarray(s, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    inside = np.abs(s) + np.abs(t) <= 1.0
    a = np.where(inside, s, (1.0 - np.abs(t)) * _sgn(s))
    b = np.where(inside, t, (1.0 - np.abs(s)) * _sgn(t))
    c = 1.0 - np.abs(a) - np.abs(b)
    return (a * a + b * b + c * c) ** -1.5 / (4.0 * math.pi)


def octa_marginal(s: np.ndarray) -> np.ndarray:
    """Marginal density of one octahedral coordinate, f(s) = integral of octa_density
    over t, in closed form. For s in [0, 1] the integral over the diamond part
    (0 <= t <= 1 - s) and over the folded part (1 - s <= t <= 1) are integrals of
    (2 x^2 + beta x + c)^(-3/2) with c = s^2 + (1 - s)^2 (antiderivative
    2 (4 x + beta) / ((8 c - beta^2) sqrt(2 x^2 + beta x + c))), giving
        f(s) = [2 (1 - s) / (2 s^2 + (1 - s)^2) + 2 s / (s^2 + 2 (1 - s)^2)]
               / (2 pi sqrt(c)),
    and f(-s) = f(s)."""
    s = np.abs(np.asarray(s, dtype=np.float64))
    c = s * s + (1.0 - s) ** 2
    return (2.0 * (1.0 - s) / (2.0 * s * s + (1.0 - s) ** 2)
            + 2.0 * s / (s * s + 2.0 * (1.0 - s) ** 2)) / (2.0 * math.pi * np.sqrt(c))


# ----------------------------------------------------------------------------------
# Marginals of the norm and of a single coordinate (R5)
# ----------------------------------------------------------------------------------


def norm_density(r: np.ndarray, d: int) -> np.ndarray:
    """Density of the norm of three coordinates of a uniform unit vector in R^d:
    rho^2 ~ Beta(3/2, (d - 3) / 2), so f(r) = 2 r^2 (1 - r^2)^((d - 5) / 2) / B."""
    r = np.asarray(r, dtype=np.float64)
    a, b = 1.5, (d - 3) / 2.0
    return 2.0 * r * r * np.clip(1.0 - r * r, 0.0, None) ** (b - 1.0) / special.beta(a, b)


def coord_density(u: np.ndarray, d: int) -> np.ndarray:
    """Density of one coordinate of a uniform unit vector in R^d: (1 - u^2)^((d-3)/2) / B."""
    u = np.asarray(u, dtype=np.float64)
    return np.clip(1.0 - u * u, 0.0, None) ** ((d - 3) / 2.0) / special.beta(0.5, (d - 1) / 2.0)


def _support(kind: str) -> tuple[float, float, list[float]]:
    """Support of a marginal and the interior points where its cells are split."""
    if kind == "oct":
        return -1.0, 1.0, [0.0]
    if kind == "norm":
        return 0.0, 1.0, []
    return -1.0, 1.0, [0.0]


def _density(kind: str, d: int):
    if kind == "oct":
        return octa_marginal
    if kind == "norm":
        return lambda r: norm_density(r, d)
    return lambda u: coord_density(u, d)


# ----------------------------------------------------------------------------------
# Lloyd-Max (R6)
# ----------------------------------------------------------------------------------

_GL_X, _GL_W = np.polynomial.legendre.leggauss(GL_POINTS)


def _cell_integrals(f, lo: np.ndarray, hi: np.ndarray, splits: list[float]):
    """Mass and first moment of density f over each cell [lo_i, hi_i] (Gauss-Legendre,
    cells split at the given interior points)."""
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    edges = [lo]
    for p in splits:
        edges.append(np.clip(np.full_like(lo, p), lo, hi))
    edges.append(hi)
    mass = np.zeros_like(lo)
    mom = np.zeros_like(lo)
    for a, b in zip(edges[:-1], edges[1:]):
        half = 0.5 * (b - a)
        mid = 0.5 * (b + a)
        x = mid[:, None] + half[:, None] * _GL_X[None, :]
        fx = f(x)
        mass += half * (fx @ _GL_W)
        mom += half * ((fx * x) @ _GL_W)
    return mass, mom


def lloyd_max_density(f, lo: float, hi: float, splits: list[float], bits: int):
    """Lloyd-Max quantiser with 2^bits levels for density f on [lo, hi] (R6): levels
    start at the (i + 1/2) / 2^bits quantiles (bisection on the Gauss-Legendre CDF) and
    move to their cells' conditional means until none moves by more than 1e-14.
    Returns (levels, boundaries, iterations)."""

    def cdf(x: float) -> float:
        m, _ = _cell_integrals(f, np.array([lo]), np.array([x]), splits)
        return float(m[0])

    total = cdf(hi)

    def quantile(q: float) -> float:
        a, b = lo, hi
        for _ in range(200):
            mid = 0.5 * (a + b)
            if mid <= a or mid >= b:
                break
            if cdf(mid) < q * total:
                a = mid
            else:
                b = mid
        return 0.5 * (a + b)

    n = 1 << bits
    levels = np.array([quantile((i + 0.5) / n) for i in range(n)])
    for it in range(1, LLOYD_MAX_ITER + 1):
        bounds = 0.5 * (levels[:-1] + levels[1:])
        a = np.concatenate([[lo], bounds])
        b = np.concatenate([bounds, [hi]])
        mass, mom = _cell_integrals(f, a, b, splits)
        new = np.where(mass > 0.0, mom / np.where(mass > 0.0, mass, 1.0), levels)
        moved = float(np.max(np.abs(new - levels)))
        levels = new
        if moved <= LLOYD_TOL:
            break
    return levels, 0.5 * (levels[:-1] + levels[1:]), it


_LLOYD_CACHE: dict = {}


def lloyd_max(kind: str, d: int, bits: int) -> tuple[np.ndarray, np.ndarray, int]:
    """Lloyd-Max quantiser with 2^bits levels for the marginal `kind` ('oct', 'norm' or
    'coord') at head dimension d. Returns (levels, boundaries, iterations)."""
    key = (kind, d if kind != "oct" else 0, bits)
    if key not in _LLOYD_CACHE:
        lo, hi, splits = _support(kind)
        _LLOYD_CACHE[key] = lloyd_max_density(_density(kind, d), lo, hi, splits, bits)
    lev, bnd, it = _LLOYD_CACHE[key]
    return lev.copy(), bnd.copy(), it


def quantise(x: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """Index of the nearest level (the lower one at an exact midpoint): brute force."""
    x = np.asarray(x, dtype=np.float64)
    return np.argmin(np.abs(x[..., None] - levels), axis=-1).astype(np.int64)


class Codebook:
    """The three quantisers of one configuration (head dim d, b_dir, b_norm, b_rest)."""

    def __init__(self, d: int, b_dir: int, b_norm: int, b_rest: int):
        if d not in (64, 128) or not (1 <= b_dir <= 6 and 1 <= b_norm <= 6 and 1 <= b_rest <= 8):
            raise ValueError("unsupported triplet configuration")
        self.d, self.b_dir, self.b_norm, self.b_rest = d, b_dir, b_norm, b_rest
        self.dir_levels, self.dir_bounds, _ = lloyd_max("oct", d, b_dir)
        self.norm_levels, self.norm_bounds, _ = lloyd_max("norm", d, b_norm)
        self.rest_levels, self.rest_bounds, _ = lloyd_max("coord", d, b_rest)

    @property
    def triplets(self) -> int:
        return self.d // 3

    @property
    def rest(self) -> int:
        return self.d - 3 * self.triplets


def record_bits(d: int, b_dir: int, b_norm: int, b_rest: int) -> int:
    """Bits of one token-head record: fp16 scale, T triplets of 2 b_dir + b_norm bits,
    d - 3T leftover codes of b_rest bits."""
    t = d // 3
    return 16 + t * (2 * b_dir + b_norm) + (d - 3 * t) * b_rest


def bits_per_element(d: int, b_dir: int, b_norm: int, b_rest: int) -> float:
    """Stored bits per element, the record padded to whole 32-bit words."""
    return 32 * math.ceil(record_bits(d, b_dir, b_norm, b_rest) / 32) / d


# ----------------------------------------------------------------------------------
# Encode / dequantise (R1-R3, R8)
# ----------------------------------------------------------------------------------


def fp16_round(x: np.ndarray) -> np.ndarray:
    x = np.minimum(np.asarray(x, dtype=np.float64), FP16_MAX)
    return x.astype(np.float16).astype(np.float64)


def encode(x: np.ndarray, signs: np.ndarray, cb: Codebook) -> dict:
    """Vectors x [..., d] -> codes. Returns s_code, t_code, norm_code [..., T],
    rest_code [..., d - 3T], scale (fp16 values) [...], plus the float64 quantities the
    decisions were taken on (st [..., T, 2], rho [..., T], rest [..., d - 3T])."""
    y = codec.rotate(x, signs)
    n = np.linalg.norm(y, axis=-1)
    u = y / np.where(n > 0.0, n, 1.0)[..., None]
    t = cb.triplets
    tri = u[..., : 3 * t].reshape(u.shape[:-1] + (t, 3))
    rho = np.linalg.norm(tri, axis=-1)
    st = octa_encode(tri)
    rest = u[..., 3 * t:]
    return {
        "s_code": quantise(st[..., 0], cb.dir_levels),
        "t_code": quantise(st[..., 1], cb.dir_levels),
        "norm_code": quantise(rho, cb.norm_levels),
        "rest_code": quantise(rest, cb.rest_levels),
        "scale": fp16_round(n),
        "st": st, "rho": rho, "rest": rest,
    }


def near_boundary(values: np.ndarray, bounds: np.ndarray, tol: float = 1e-9) -> np.ndarray:
    """True where a value lies within tol of a decision boundary."""
    values = np.asarray(values, dtype=np.float64)
    return np.min(np.abs(values[..., None] - bounds), axis=-1) < tol


def dequant(codes: dict, signs: np.ndarray, cb: Codebook) -> np.ndarray:
    """Codes -> vectors x_hat [..., d]."""
    st = np.stack([cb.dir_levels[codes["s_code"]], cb.dir_levels[codes["t_code"]]], axis=-1)
    w = octa_decode(st)
    rho = cb.norm_levels[codes["norm_code"]]
    tri = (rho[..., None] * w).reshape(rho.shape[:-1] + (3 * cb.triplets,))
    rest = cb.rest_levels[codes["rest_code"]]
    u_hat = np.concatenate([tri, rest], axis=-1)
    y_hat = np.asarray(codes["scale"], dtype=np.float64)[..., None] * u_hat
    return codec.unrotate(y_hat, signs)


def attention(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, scale=None) -> np.ndarray:
    """Decode attention on dequantised vectors: the plain definition (codec.attention)."""
    return codec.attention(q, k_hat, v_hat, scale=scale)


# ----------------------------------------------------------------------------------
# Bit allocation (R7)
# ----------------------------------------------------------------------------------


def _dir_inner(b_dir: int, levels: np.ndarray, grid: int = 16) -> float:
    """E[w . w_hat] for a uniform direction w and its quantised reconstruction, by
    Gauss-Legendre over each cell of the square (cells split at 0 and at the diamond's
    edges would be exact; the rule here is accurate to ~1e-6, enough to rank splits)."""
    bounds = np.concatenate([[-1.0], 0.5 * (levels[:-1] + levels[1:]), [1.0]])
    gx, gw = np.polynomial.legendre.leggauss(grid)
    total = 0.0
    for i in range(len(levels)):
        for j in range(len(levels)):
            a0, a1, b0, b1 = bounds[i], bounds[i + 1], bounds[j], bounds[j + 1]
            s = 0.5 * (a0 + a1) + 0.5 * (a1 - a0) * gx
            t = 0.5 * (b0 + b1) + 0.5 * (b1 - b0) * gx
            ss, tt = np.meshgrid(s, t, indexing="ij")
            dens = octa_density(ss, tt)
            w = octa_decode(np.stack([ss, tt], axis=-1))
            w_hat = octa_decode(np.array([levels[i], levels[j]]))
            val = dens * (w @ w_hat)
            total += 0.25 * (a1 - a0) * (b1 - b0) * float(gw @ val @ gw)
    return total


def triplet_distortion(d: int, b_dir: int, b_norm: int) -> float:
    """E |rho w - rho_hat w_hat|^2 for one triplet of a uniform unit vector in R^d (norm
    and direction independent): E rho^2 + E rho_hat^2 - 2 E[rho rho_hat] E[w . w_hat]."""
    lev, bnd, _ = lloyd_max("norm", d, b_norm)
    a = np.concatenate([[0.0], bnd])
    b = np.concatenate([bnd, [1.0]])
    mass, mom = _cell_integrals(lambda r: norm_density(r, d), a, b, [])
    e_rho2 = 3.0 / d
    e_rhohat2 = float(np.sum(mass * lev * lev))
    e_rho_rhohat = float(np.sum(mom * lev))
    dir_levels, _, _ = lloyd_max("oct", d, b_dir)
    return e_rho2 + e_rhohat2 - 2.0 * e_rho_rhohat * _dir_inner(b_dir, dir_levels)


def allocation(d: int, budget: int) -> tuple[int, int, int]:
    """(b_dir, b_norm, b_rest) for a per-triplet budget of `budget` bits (R7)."""
    best = None
    for b_norm in range(1, 7):
        rest = budget - b_norm
        if rest % 2 or not 1 <= rest // 2 <= 6:
            continue
        dist = triplet_distortion(d, rest // 2, b_norm)
        if best is None or dist < best[0]:
            best = (dist, rest // 2, b_norm)
    if best is None:
        raise ValueError(f"no split of {budget} bits per triplet")
    return best[1], best[2], max(1, min(8, round(budget / 3)))
