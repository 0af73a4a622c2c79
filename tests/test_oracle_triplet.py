"""Pins for the triplet (octahedral) codec oracle: each check ties it to something other
than itself - hand-worked map values, the map's inverse, closed-form marginals against
the joint density and against Monte Carlo samples of uniform directions, the Lloyd-Max
solver against Max's published Gaussian quantisers and the exact uniform quantiser, the
centroid condition checked by an independent adaptive integrator, the analytic
distortion against measured reconstruction error, and hand-worked record sizes."""

import math

import numpy as np
import pytest
from scipy import integrate, stats

from conftest import read_golden
from oracle import codec as oc
from oracle import triplet as tr


# ---------------------------------------------------------------- octahedral map


@pytest.mark.parametrize("w,st", [
    ((0, 0, 1), (0, 0)), ((1, 0, 0), (1, 0)), ((0, -1, 0), (0, -1)),
    ((0, 0, -1), (1, 1)),                      # sgn(0) = +1 on the fold
    ((1, 1, 1), (1 / 3, 1 / 3)),
    ((1, 2, -1), (0.5, 0.75)),                 # p = (1, 2, -1)/4: ((1 - 1/2), (1 - 1/4))
    ((-3, 1, -1), (-0.8, 0.4)),                # p = (-3, 1, -1)/5: (-(1 - 1/5), (1 - 3/5))
    ((0, 0, 0), (0, 0)),
])
def test_octahedral_map_hand_values(w, st):
    np.testing.assert_allclose(tr.octa_encode(np.array(w, float)), st, atol=1e-15)


def test_octahedral_map_inverts_and_covers_the_square():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((200000, 3))
    w /= np.linalg.norm(w, axis=1, keepdims=True)
    st = tr.octa_encode(w)
    assert np.all(np.abs(st) <= 1.0)
    np.testing.assert_allclose(tr.octa_decode(st), w, atol=2e-15)
    # every point of the square is the image of a direction
    sq = rng.uniform(-1, 1, (200000, 2))
    np.testing.assert_allclose(tr.octa_encode(tr.octa_decode(sq)), sq, atol=2e-15)


# ---------------------------------------------------------------- marginals


def test_octahedral_marginal_is_the_joint_density_integrated():
    for s in np.linspace(-0.99, 0.99, 23):
        num = integrate.quad(lambda t: float(tr.octa_density(np.array(s), np.array(t))), -1, 1,
                             points=[-(1 - abs(s)), 0.0, 1 - abs(s)], epsabs=1e-13)[0]
        assert abs(num - float(tr.octa_marginal(np.array(s)))) < 1e-12, s
    total = integrate.dblquad(lambda t, s: float(tr.octa_density(np.array(s), np.array(t))),
                              -1, 1, -1, 1, epsabs=1e-10)[0]
    assert abs(total - 1.0) < 1e-7  # no breakpoints at the kinks: a looser rule
    assert abs(integrate.quad(tr.octa_marginal, -1, 0)[0] + integrate.quad(tr.octa_marginal, 0, 1)[0] - 1) < 1e-12


def _ks(samples, density, lo, hi):
    """Kolmogorov-Smirnov distance between samples and the density's CDF."""
    x = np.sort(samples)
    grid = np.linspace(lo, hi, 4001)
    f = density(grid)
    cdf = np.concatenate([[0.0], np.cumsum(0.5 * (f[1:] + f[:-1]) * np.diff(grid))])
    return float(np.max(np.abs(np.interp(x, grid, cdf) - np.arange(1, len(x) + 1) / len(x))))


def test_marginals_match_uniform_directions_monte_carlo():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((2_000_000, 3))
    st = tr.octa_encode(w)
    assert _ks(st[:, 0], tr.octa_marginal, -1, 1) < 2e-3
    assert _ks(st[:, 1], tr.octa_marginal, -1, 1) < 2e-3
    for d in (64, 128):
        u = rng.standard_normal((100_000, d))
        u /= np.linalg.norm(u, axis=1, keepdims=True)
        rho = np.linalg.norm(u[:, :3], axis=1)
        assert _ks(rho, lambda r: tr.norm_density(r, d), 0, 1) < 6e-3
        assert _ks(u[:, 5], lambda x: tr.coord_density(x, d), -1, 1) < 6e-3
    # the norm marginal is the Beta law's, by an independent routine
    r = np.linspace(0.01, 0.6, 50)
    np.testing.assert_allclose(tr.norm_density(r, 128),
                               2 * r * stats.beta.pdf(r * r, 1.5, (128 - 3) / 2), rtol=1e-10)


# ---------------------------------------------------------------- Lloyd-Max


def test_lloyd_max_reproduces_max_1960_gaussian_quantisers():
    g = lambda x: np.exp(-x * x / 2) / math.sqrt(2 * math.pi)  # noqa: E731
    for row in read_golden("lloyd_max_gaussian.txt"):
        n = int(row[0])
        want = np.array([float(v) for v in row[1:]])
        lev, bnd, _ = tr.lloyd_max_density(g, -12.0, 12.0, [0.0], n.bit_length() - 1)
        pos = lev[n // 2:]
        np.testing.assert_allclose(pos, want, atol=6e-4, rtol=0)
        np.testing.assert_allclose(lev, -lev[::-1], atol=1e-12)
    lev, _, _ = tr.lloyd_max_density(lambda x: np.sqrt(2 / math.pi) * np.exp(-x * x / 2) + 0 * x,
                                     0.0, 12.0, [], 1)
    np.testing.assert_allclose(lev, [0.4528, 1.510], atol=6e-4)  # half-Gaussian = Max's N = 4


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_max_of_a_uniform_density_is_the_uniform_quantiser(bits):
    lev, bnd, _ = tr.lloyd_max_density(lambda x: 0.5 + 0 * x, -1.0, 1.0, [], bits)
    n = 1 << bits
    np.testing.assert_allclose(lev, -1 + (2 * np.arange(n) + 1) / n, atol=1e-13)
    np.testing.assert_allclose(bnd, -1 + 2 * np.arange(1, n) / n, atol=1e-13)


@pytest.mark.parametrize("kind,d,bits", [("oct", 128, 4), ("oct", 128, 2), ("norm", 128, 2),
                                         ("norm", 64, 3), ("coord", 128, 3), ("coord", 64, 2)])
def test_fitted_quantisers_meet_the_lloyd_max_conditions(kind, d, bits):
    """Each level is its cell's conditional mean (checked with SciPy's adaptive
    integrator, not the Gauss-Legendre rule of the fit); boundaries are midpoints."""
    lev, bnd, _ = tr.lloyd_max(kind, d, bits)
    f = {"oct": tr.octa_marginal, "norm": lambda r: tr.norm_density(r, d),
         "coord": lambda u: tr.coord_density(u, d)}[kind]
    lo = 0.0 if kind == "norm" else -1.0
    edges = np.concatenate([[lo], bnd, [1.0]])
    for i in range(len(lev)):
        a, b = edges[i], edges[i + 1]
        pts = [0.0] if a < 0.0 < b else None
        m = integrate.quad(f, a, b, points=pts, epsabs=1e-14, epsrel=1e-12, limit=200)[0]
        mu = integrate.quad(lambda x: x * f(x), a, b, points=pts, epsabs=1e-14,
                            epsrel=1e-12, limit=200)[0]
        assert abs(mu / m - lev[i]) < 1e-10, (i, mu / m, lev[i])
    np.testing.assert_allclose(bnd, 0.5 * (lev[1:] + lev[:-1]), atol=0)
    assert np.all(np.diff(lev) > 0)


def test_quantise_is_the_nearest_level_with_ties_low():
    lev = np.array([-1.0, 0.0, 2.0])
    np.testing.assert_array_equal(tr.quantise(np.array([-0.5, 1.0, 1.1, -5, 9]), lev),
                                  [0, 1, 2, 0, 2])


# ---------------------------------------------------------------- codec


def test_record_bits_worked_by_hand():
    for d, bd, bn, br, bits, words, bpe in read_golden("triplet_bits.txt"):
        d, bd, bn, br = int(d), int(bd), int(bn), int(br)
        assert tr.record_bits(d, bd, bn, br) == int(bits)
        assert math.ceil(int(bits) / 32) == int(words)
        assert tr.bits_per_element(d, bd, bn, br) == float(bpe)


def test_allocation_is_non_uniform_and_follows_the_distortion():
    # the norm gets fewer bits than each direction coordinate at these budgets
    assert tr.allocation(128, 10) == (4, 2, 3)
    assert tr.allocation(128, 7) == (3, 1, 2)
    # the rule picks the smallest distortion among the splits of the budget
    d = 128
    picks = {(bd, 10 - 2 * bd): tr.triplet_distortion(d, bd, 10 - 2 * bd) for bd in (2, 3, 4)}
    assert min(picks, key=picks.get) == (4, 2)


@pytest.mark.parametrize("d,alloc", [(128, (4, 2, 3)), (64, (3, 3, 3))])
def test_reconstruction_error_matches_the_analytic_distortion(d, alloc):
    """Encode + dequantise Gaussian vectors: the mean squared error of the unit-vector
    triplets equals the analytic expectation of the fitted quantisers (a dropped term, a
    wrong sign or a swapped coordinate anywhere in the chain would break this)."""
    cb = tr.Codebook(d, *alloc)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20000, d))
    sg = oc.layer_signs(0, 2, d)
    codes = tr.encode(x, sg, cb)
    st = np.stack([cb.dir_levels[codes["s_code"]], cb.dir_levels[codes["t_code"]]], axis=-1)
    w_hat = tr.octa_decode(st)
    rho_hat = cb.norm_levels[codes["norm_code"]]
    y = oc.rotate(x, sg)
    u = y / np.linalg.norm(y, axis=-1, keepdims=True)
    tri = u[:, : 3 * cb.triplets].reshape(-1, cb.triplets, 3)
    err = np.mean(np.sum((tri - rho_hat[..., None] * w_hat) ** 2, axis=-1))
    want = tr.triplet_distortion(d, alloc[0], alloc[1])
    assert abs(err / want - 1) < 0.03, (err, want)
    # the full reconstruction: relative error close to sqrt of the per-coordinate share
    x_hat = tr.dequant(codes, sg, cb)
    rel = np.linalg.norm(x_hat - x, axis=-1) / np.linalg.norm(x, axis=-1)
    assert 0.5 * math.sqrt(want * d / 3) < np.mean(rel) < 1.5 * math.sqrt(want * d / 3)


def test_constructed_vectors_give_hand_derived_codes():
    """x = sign * (column k of H) * c rotates to c sqrt(d) e_k: the triplet holding k is
    the axis direction (norm 1), every other triplet is zero."""
    d = 128
    cb = tr.Codebook(d, 4, 2, 3)
    sg = oc.layer_signs(0, 0, d)
    h = oc.hadamard(d)
    for k, axis in ((0, 0), (4, 1), (8, 2), (127, None)):
        x = sg * h[:, k] * 0.75
        c = tr.encode(x[None], sg, cb)
        j = k // 3
        n = 1 << 4
        if axis is None:  # a leftover coordinate: u = +1
            assert c["rest_code"][0, k - 3 * cb.triplets] == (1 << 3) - 1
            continue
        want_st = {0: (n - 1, tr.quantise(0.0, cb.dir_levels)),
                   1: (tr.quantise(0.0, cb.dir_levels), n - 1),
                   2: (tr.quantise(0.0, cb.dir_levels), tr.quantise(0.0, cb.dir_levels))}[axis]
        assert (c["s_code"][0, j], c["t_code"][0, j]) == want_st
        assert c["norm_code"][0, j] == (1 << 2) - 1
        others = np.delete(np.arange(cb.triplets), j)
        assert np.all(c["norm_code"][0, others] == 0)
        assert c["scale"][0] == np.float16(0.75 * math.sqrt(d))


def test_zero_vector_and_attention_definition():
    cb = tr.Codebook(64, 2, 2, 2)
    sg = oc.layer_signs(0, 1, 64)
    c = tr.encode(np.zeros((1, 64)), sg, cb)
    assert c["scale"][0] == 0.0
    assert np.all(tr.dequant(c, sg, cb) == 0.0)
    # attention over dequantised vectors is the codec's plain definition
    rng = np.random.default_rng(4)
    k, v, q = rng.standard_normal((1, 50, 1, 64)), rng.standard_normal((1, 50, 1, 64)), rng.standard_normal((1, 2, 64))
    kh = tr.dequant(tr.encode(k, sg, cb), sg, cb)
    vh = tr.dequant(tr.encode(v, sg, cb), sg, cb)
    np.testing.assert_allclose(tr.attention(q, kh, vh), oc.attention(q, kh, vh), atol=0)
