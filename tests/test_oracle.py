"""Pins for the oracle: each check ties it to something other than itself (published
check values, hand-derived fixtures, closed forms, brute force, a library routine)."""

import math

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import codec as oc
from synthetic import get, layer_kv


# ---------------------------------------------------------------- sign diagonal


def test_splitmix64_published_values():
    rows = read_golden("splitmix64_seed0.txt")
    state = 0
    for idx, hexval in rows:
        # the generator's k-th output is mix((k - 1) * gamma)
        assert oc.splitmix64_mix(state) == int(hexval, 16), idx
        state = (state + oc.SPLITMIX_GAMMA) & oc.MASK64


def test_signs_equal_worked_vectors():
    """Sign vectors worked out in bash 64-bit arithmetic from the published SplitMix64
    definition (tests/golden/layer_signs_worked.sh), including (seed, layer) pairs where
    seed ^ layer differs from seed + layer."""
    rows = read_golden("layer_signs.txt")
    assert len(rows) == 3
    for seed, layer, d, *signs in rows:
        got = oc.layer_signs(int(seed), int(layer), int(d))
        assert got.tolist() == [float(x) for x in signs], (seed, layer)


def test_signs_are_pm1_balanced_and_seeded():
    s = oc.layer_signs(0, 0, 4096)
    assert set(np.unique(s)) == {-1.0, 1.0}
    assert abs(s.mean()) < 0.05
    assert np.array_equal(s, oc.layer_signs(0, 0, 4096))
    assert not np.array_equal(s[:128], oc.layer_signs(0, 1, 128))
    assert not np.array_equal(s[:128], oc.layer_signs(1, 0, 128))
    # a prefix of a longer diagonal is the shorter one (index-addressed generator)
    assert np.array_equal(oc.layer_signs(5, 3, 64), oc.layer_signs(5, 3, 128)[:64])


# ---------------------------------------------------------------- Walsh-Hadamard


def test_hadamard_matches_hand_written_h8():
    rows = read_golden("hadamard_8.txt")
    h8 = np.array([[float(v) for v in r] for r in rows])
    assert np.array_equal(oc.hadamard(8), h8)


@pytest.mark.parametrize("d", [1, 2, 4, 16, 64, 128, 256])
def test_hadamard_closed_form_and_orthogonality(d):
    h = oc.hadamard(d)
    i = np.arange(d)
    pop = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    assert np.array_equal(h, (-1.0) ** pop)
    assert np.array_equal(h @ h.T, d * np.eye(d))


def test_rotation_by_explicit_sum_small_d():
    rng = np.random.default_rng(1)
    for d in (2, 4, 8, 16):
        x = rng.standard_normal(d)
        sg = oc.layer_signs(7, 2, d)
        y = oc.rotate(x, sg)
        for k in range(d):
            ref = sum((-1) ** bin(i & k).count("1") * sg[i] * x[i] for i in range(d))
            assert y[k] == pytest.approx(ref / math.sqrt(d), abs=1e-14)


def test_rotation_preserves_norm_and_inverts():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 128))
    sg = oc.layer_signs(0, 3, 128)
    y = oc.rotate(x, sg)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1),
                               rtol=1e-14)
    np.testing.assert_allclose(oc.unrotate(y, sg), x, atol=1e-13)


def test_rotation_of_signed_hadamard_column_is_one_hot():
    d = 64
    sg = oc.layer_signs(0, 0, d)
    h = oc.hadamard(d)
    for k in (0, 5, 63):
        y = oc.rotate(sg * h[:, k], sg)
        expect = np.zeros(d)
        expect[k] = math.sqrt(d)
        np.testing.assert_allclose(y, expect, atol=1e-13)


# ---------------------------------------------------------------- polar + angles


def test_polar_reconstructs_pairs_and_known_angles():
    rng = np.random.default_rng(3)
    y = rng.standard_normal((10, 64))
    r, th = oc.polar(y)
    np.testing.assert_allclose(r * np.cos(th), y[:, 0::2], atol=1e-15 * 8)
    np.testing.assert_allclose(r * np.sin(th), y[:, 1::2], atol=1e-15 * 8)
    r, th = oc.polar(np.array([1.0, 0.0, 0.0, 2.0, -3.0, 0.0, 0.0, -1.0]))
    np.testing.assert_allclose(r, [1, 2, 3, 1])
    np.testing.assert_allclose(th, [0, math.pi / 2, math.pi, -math.pi / 2])


@pytest.mark.parametrize("n", [2, 3, 8, 64, 100, 128, 256])
def test_angle_code_equals_brute_force_nearest_centre(n):
    rng = np.random.default_rng(n)
    th = rng.uniform(-math.pi, math.pi, 20000)
    r = np.ones_like(th)
    keep = ~oc.angle_near_boundary(th, n, tol=1e-9)
    c = oc.angle_codes(r, th, n)
    cent = 2 * math.pi * np.arange(n) / n
    dist = np.abs(np.exp(1j * th)[:, None] - np.exp(1j * cent)[None, :])
    brute = np.argmin(dist, axis=1)
    assert np.array_equal(c[keep], brute[keep])
    # chord bound per unit radius: |u(theta) - u(theta_hat)| <= 2 sin(pi / 2n)
    chord = np.abs(np.exp(1j * th) - np.exp(1j * cent[c]))
    assert np.all(chord <= 2 * math.sin(math.pi / (2 * n)) + 1e-12)


def test_angle_codes_special_cases():
    n = 128
    assert oc.angle_codes(np.array([0.0]), np.array([1.0]), n)[0] == 0  # zero pair
    assert oc.angle_codes(np.array([1.0]), np.array([math.pi]), n)[0] == n // 2
    assert oc.angle_codes(np.array([1.0]), np.array([-math.pi]), n)[0] == n // 2
    assert oc.angle_codes(np.array([1.0]), np.array([-1e-3]), n)[0] == 0
    assert oc.angle_codes(np.array([1.0]), np.array([-2 * math.pi / n]), n)[0] == n - 1
    b = (3 + 0.5) * 2 * math.pi / n
    assert oc.angle_near_boundary(np.array([b + 5e-7, b - 5e-7]), n).all()
    assert not oc.angle_near_boundary(np.array([b + 2e-6, b - 2e-6]), n).any()


def _vector_from_pairs(r, ang, signs):
    """x whose rotated pairs are exactly r * (cos ang, sin ang) (up to fp64 rounding)."""
    y = np.empty(r.shape[:-1] + (2 * r.shape[-1],))
    y[..., 0::2] = r * np.cos(ang)
    y[..., 1::2] = r * np.sin(ang)
    return oc.unrotate(y, signs)


@pytest.mark.parametrize("n", [64, 128, 256])
def test_on_centre_inputs_give_exact_angle_codes(n):
    rng = np.random.default_rng(10 + n)
    d = 128
    sg = oc.layer_signs(0, 1, d)
    codes = rng.integers(0, n, (40, d // 2))
    r = rng.uniform(0.1, 4.0, (40, d // 2))
    x = _vector_from_pairs(r, 2 * math.pi * codes / n, sg)
    enc = oc.encode_k(x, sg, n)
    assert np.array_equal(enc["angle"], codes)
    enc = oc.encode_v(x, sg, n)
    assert np.array_equal(enc["angle"], codes)


# ---------------------------------------------------------------- fp16 parameters


def test_fp16_rounding_hand_values():
    for a, b in read_golden("fp16_rounding.txt"):
        assert oc.fp16_round(np.array([float.fromhex(a)]))[0] == float.fromhex(b), a


# ---------------------------------------------------------------- key radii


def test_k_radius_is_nearest_of_256_levels():
    rng = np.random.default_rng(4)
    r = np.abs(rng.standard_normal((300, 64))) * rng.uniform(0.01, 100, (300, 1))
    s, rho = oc.k_radius_encode(r)
    levels = np.arange(256)[None, None, :] * (s[:, None, None] / 255)
    brute = np.argmin(np.abs(r[..., None] - levels), axis=-1)
    assert np.array_equal(rho, brute)
    assert np.all(s == s.astype(np.float16).astype(np.float64))


def test_k_radius_constructed_levels_exact():
    d, n = 128, 128
    sg = oc.layer_signs(0, 0, d)
    s = 3.25  # an fp16 value
    rho = np.arange(64) * 4 + 3
    rho[10] = 255
    rho[11] = 0
    ang = 2 * math.pi * np.arange(64) % n / n
    x = _vector_from_pairs(rho * s / 255, ang, sg)
    enc = oc.encode_k(x, sg, n)
    assert enc["scale"] == s
    assert np.array_equal(enc["radius"], rho)


def test_k_radius_degenerate_cases():
    s, rho = oc.k_radius_encode(np.zeros((1, 8)))
    assert s[0] == 0 and not rho.any()
    s, rho = oc.k_radius_encode(np.array([[1e6, 5e5, 0.0]]))
    assert s[0] == 65504.0 and rho[0, 0] == 255 and rho[0, 1] == 255 and rho[0, 2] == 0


# ---------------------------------------------------------------- value radii


def test_v_radius_is_nearest_log_level():
    rng = np.random.default_rng(5)
    r = np.exp(rng.uniform(-3, 3, (300, 64)))
    s_min, s_max, rho = oc.v_radius_encode(r)
    lam = np.log(s_max / s_min)
    levels = s_min[:, None] * np.exp(np.arange(16)[None, :] * lam[:, None] / 15)
    inside = (r >= s_min[:, None]) & (r <= s_max[:, None])
    brute = np.argmin(np.abs(np.log(r[..., None]) - np.log(levels[:, None, :])), axis=-1)
    assert np.array_equal(rho[inside], brute[inside])
    assert np.all(rho[r < s_min[:, None]] == 0)
    assert np.all(rho[r > s_max[:, None]] == 15)
    # the endpoints of each vector use the end codes
    assert np.all(rho[np.arange(300), np.argmin(r, 1)] == 0)
    assert np.all(rho[np.arange(300), np.argmax(r, 1)] == 15)


def test_v_radius_degenerate_and_zero_pairs():
    s_min, s_max, rho = oc.v_radius_encode(np.full((1, 8), 2.0))
    assert s_min[0] == s_max[0] == 2.0 and not rho.any()
    rhat = oc.v_radius_decode(s_min, s_max, rho)
    assert np.all(rhat == 2.0)
    s_min, s_max, rho = oc.v_radius_encode(np.array([[0.0, 1.0, 4.0]]))
    assert s_min[0] == 2.0 ** -14 and s_max[0] == 4.0
    assert list(rho[0]) == [0, round(15 * math.log(2 ** 14) / math.log(2 ** 16)), 15]


# ---------------------------------------------------------------- whole codec error bound


def _error_bound(enc_r, n, rhat):
    return np.sqrt(np.sum((2 * enc_r * math.sin(math.pi / (2 * n)) + np.abs(enc_r - rhat)) ** 2,
                          axis=-1))


@pytest.mark.parametrize("d,n_k,n_v", [(64, 128, 64), (128, 128, 64), (128, 256, 256)])
def test_reconstruction_error_within_closed_form_bound(d, n_k, n_v):
    cfg = get("mistral7b")
    k, v = layer_kv(cfg, 0, seq=64, batch=1)
    x_k = k[0, :, :, :d].reshape(-1, d).double().numpy()
    x_v = v[0, :, :, :d].reshape(-1, d).double().numpy()
    sg = oc.layer_signs(0, 0, d)

    ek = oc.encode_k(x_k, sg, n_k)
    xk_hat = oc.dequant_k(ek["angle"], ek["radius"], ek["scale"], n_k, sg)
    s = ek["scale"][:, None]
    delta_k = s / 510 + np.maximum(0.0, ek["r"] - s)
    bound_k = np.sqrt(np.sum((2 * ek["r"] * math.sin(math.pi / (2 * n_k)) + delta_k) ** 2, -1))
    err_k = np.linalg.norm(x_k - xk_hat, axis=-1)
    assert np.all(err_k <= bound_k * (1 + 1e-9))

    ev = oc.encode_v(x_v, sg, n_v)
    xv_hat = oc.dequant_v(ev["angle"], ev["radius"], ev["s_min"], ev["s_max"], n_v, sg)
    lam = np.log(ev["s_max"] / ev["s_min"])[:, None]
    smin, smax = ev["s_min"][:, None], ev["s_max"][:, None]
    r = ev["r"]
    delta_v = np.where(r < smin, smin - r,
                       np.where(r > smax, r - smax, r * (np.exp(lam / 30) - 1)))
    bound_v = np.sqrt(np.sum((2 * r * math.sin(math.pi / (2 * n_v)) + delta_v) ** 2, -1))
    err_v = np.linalg.norm(x_v - xv_hat, axis=-1)
    assert np.all(err_v <= bound_v * (1 + 1e-9))
    # the bound is not vacuous: errors are a sizeable part of it, and small vs |x|
    assert np.median(err_k / bound_k) > 0.2
    assert np.median(err_k / np.linalg.norm(x_k, axis=-1)) < 0.05


def test_rotated_angles_near_uniform():
    """The abstract's premise: after the rotation, pair angles are close to uniform.
    Checked on the isotropic value recipe (16-bin chi-square, 15 d.o.f.). Keys with a
    few fixed outlier channels put each pair near a fixed direction per head, so their
    histogram is clustered by construction; that is not gated."""
    cfg = get("tinyllama")
    _, v = layer_kv(cfg, 0, seq=512, batch=1)
    x = v[0].reshape(-1, 64).double().numpy()
    _, th = oc.polar(oc.rotate(x, oc.layer_signs(0, 0, 64)))
    hist, _ = np.histogram(th, bins=16, range=(-math.pi, math.pi))
    expect = th.size / 16
    chi2 = np.sum((hist - expect) ** 2 / expect)
    assert chi2 < 60


# ---------------------------------------------------------------- attention


def _gqa_sdpa(q, k, v, scale):
    """torch's scaled_dot_product_attention in float64 on the CPU, GQA by repetition."""
    bsz, hq, d = q.shape
    g = hq // k.shape[2]
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    qt = torch.from_numpy(q)[:, :, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[:, :, 0, :].numpy()


def test_attention_matches_library_sdpa():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 8, 64))
    k = rng.standard_normal((2, 37, 2, 64)) * 2
    v = rng.standard_normal((2, 37, 2, 64))
    ours = oc.attention(q, k, v)
    ref = _gqa_sdpa(q, k, v, 1 / 8)
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-13)


def test_attention_single_token_returns_value():
    rng = np.random.default_rng(7)
    v = rng.standard_normal((1, 1, 1, 32))
    out = oc.attention(rng.standard_normal((1, 4, 32)), rng.standard_normal((1, 1, 1, 32)), v)
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], v[0, 0, 0])


def test_rotated_domain_attention_identity():
    """Scores from rotated q and rotated-domain keys, values summed in the rotated
    domain and one inverse transform at the end, equal the plain definition."""
    rng = np.random.default_rng(8)
    d, n_k, n_v = 128, 128, 64
    sg = oc.layer_signs(0, 5, d)
    x_k = rng.standard_normal((300, d))
    x_v = rng.standard_normal((300, d))
    q = rng.standard_normal(d)
    ek, ev = oc.encode_k(x_k, sg, n_k), oc.encode_v(x_v, sg, n_v)
    yk = oc.dequant_k_rotated(ek["angle"], ek["radius"], ek["scale"], n_k)
    yv = oc.dequant_v_rotated(ev["angle"], ev["radius"], ev["s_min"], ev["s_max"], n_v)
    s = (yk @ oc.rotate(q, sg)) / math.sqrt(d)
    p = np.exp(s - s.max())
    o_rot = oc.unrotate((p @ yv) / p.sum(), sg)
    o_ref = oc.attention(q[None, None], oc.unrotate(yk, sg)[None, :, None],
                         oc.unrotate(yv, sg)[None, :, None])[0, 0]
    np.testing.assert_allclose(o_rot, o_ref, rtol=1e-12, atol=1e-12)


def test_split_softmax_merge_equals_unsplit():
    """Log-sum-exp combination of partial (max, sum, weighted sum) over any partition
    of the sequence gives the unsplit softmax average."""
    rng = np.random.default_rng(9)
    s = rng.standard_normal(1000) * 3
    v = rng.standard_normal((1000, 16))
    p = np.exp(s - s.max())
    ref = (p @ v) / p.sum()
    cuts = np.sort(rng.choice(np.arange(1, 1000), 7, replace=False))
    parts = np.split(np.arange(1000), cuts)
    m = [s[idx].max() for idx in parts]
    l_ = [np.exp(s[idx] - mi).sum() for idx, mi in zip(parts, m)]
    acc = [np.exp(s[idx] - mi) @ v[idx] for idx, mi in zip(parts, m)]
    big = max(m)
    tot_l = sum(li * math.exp(mi - big) for li, mi in zip(l_, m))
    tot = sum(ai * math.exp(mi - big) for ai, mi in zip(acc, m))
    np.testing.assert_allclose(tot / tot_l, ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- bits per element


def test_bits_per_element_hand_values():
    for d, nk, nv, rec, bpe in read_golden("bits_per_element.txt"):
        d, nk, nv = int(d), int(nk), int(nv)
        assert oc.bits_per_element(d, nk, nv) == float(bpe)
        assert oc.bits_per_element(d, nk, nv) * 2 * d / 8 == int(rec)


def test_non_finite_input_rejected():
    with pytest.raises(ValueError):
        oc.rotate(np.array([1.0, np.nan]), np.ones(2))


def test_radius_decoders_hit_the_interval_ends():
    """Closed forms: key code 255 reconstructs the stored scale, code 0 zero; value
    codes 0 and 15 reconstruct s_min and s_max, and successive value levels have a
    constant ratio (s_max / s_min)^(1/15)."""
    s = np.array([2.5])
    assert oc.k_radius_decode(s, np.array([[0, 255, 51]]))[0].tolist() == [0.0, 2.5, 0.5]
    s_min, s_max = np.array([0.125]), np.array([8.0])
    lv = oc.v_radius_decode(s_min, s_max, np.arange(16)[None, :])[0]
    assert lv[0] == pytest.approx(0.125, rel=1e-15)
    assert lv[15] == pytest.approx(8.0, rel=1e-14)
    np.testing.assert_allclose(lv[1:] / lv[:-1], 64.0 ** (1 / 15), rtol=1e-13)


def test_exact_tie_has_two_correct_codes():
    """A pair exactly on a bin edge (only angles at multiples of pi/4 can be): with
    n = 100 an edge sits at 45 degrees (12.5 bins). The rule floor(t + 1/2) sends the
    exact tie to bin 13; float64 evaluation of t lands just below 12.5 and gives 12.
    Both bins meet at the edge, so the parity rule accepts either."""
    import sys, os
    sys.path.insert(0, os.path.dirname(__file__))
    from parity import compare_codes
    n = 100
    r, th = oc.polar(np.array([[0.75, 0.75]]))
    t = oc.angle_position(th, n)
    assert abs(t[0, 0] - 12.5) < 1e-12
    assert oc.angle_codes(r, th, n)[0, 0] in (12, 13)
    enc = {"angle": oc.angle_codes(r, th, n), "theta": th, "r": r, "n": n,
           "near_boundary": oc.angle_near_boundary(th, n), "radius": np.zeros((1, 1), int),
           "scale": np.zeros(1), "s_min": np.zeros(1), "s_max": np.zeros(1)}
    for code in (12, 13):
        got = {"k_angle": np.array([[code]]), "v_angle": np.array([[code]]),
               "k_radius": np.zeros((1, 1), int), "v_radius": np.zeros((1, 1), int),
               "k_scale": np.zeros(1), "v_smin": np.zeros(1), "v_smax": np.zeros(1)}
        assert compare_codes(got, enc, enc)["pairs"] == 2
    got["k_angle"] = np.array([[14]])
    with pytest.raises(AssertionError):
        compare_codes(got, enc, enc)
