"""CPU checks of the encoder's fp32 fast paths (the device functions angle_f32 /
angle_code, key_level and value_level): NumPy float32 emulations over dense grids,
with the hardware reciprocal, square root and log2 modelled as correctly rounded and
then off by one ulp either way. Wherever the device code trusts its fp32 estimate (the
estimate lies farther than its margin from a decision boundary), the decision must
equal the binary64 definition, and the angle estimate must stay within the error bound
its margin is derived from. The polynomial is the one in kvq_codec_dev.h, as printed by
the fit script beside it."""

import importlib.util
import os

import numpy as np
import pytest

from conftest import ROOT

f32 = np.float32
CSRC = os.path.join(ROOT, "rotated_angle_quantization_amd", "csrc")


def _fit_module():
    spec = importlib.util.spec_from_file_location("fit_atan01", os.path.join(CSRC, "fit_atan01.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def device_coefficients():
    """The coefficients written in kvq_codec_dev.h's atan01 (highest degree first)."""
    import re
    text = open(os.path.join(CSRC, "kvq_codec_dev.h")).read()
    body = text[text.index("float atan01(float z)"):]
    body = body[:body.index("return p * z;")]
    vals = [float(x) for x in re.findall(r"(-?\d+\.\d+(?:e-?\d+)?)f", body)]
    assert len(vals) == 7
    return np.array(vals[::-1], dtype=np.float32)  # c[0] .. c[6]


def ulp_variants(x):
    """x (float32) and its neighbours one ulp down and up."""
    x = np.asarray(x, np.float32)
    return [x, np.nextafter(x, f32(-np.inf)), np.nextafter(x, f32(np.inf))]


def fma32(a, b, c):
    return (np.float64(1) * a.astype(np.float64) * b.astype(np.float64)
            + c.astype(np.float64)).astype(np.float32)


def test_fit_script_reproduces_device_coefficients():
    fit = _fit_module()
    np.testing.assert_array_equal(fit.fit(), device_coefficients())
    assert fit.max_error(device_coefficients()) < 3.4e-7


def angle_f32(a64, b64, c, rcp_variant):
    af, bf = a64.astype(np.float32), b64.astype(np.float32)
    ax, ay = np.abs(af), np.abs(bf)
    mx, mn = np.maximum(ax, ay), np.minimum(ax, ay)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = ulp_variants((f32(1) / mx).astype(np.float32))[rcp_variant]
        z = (mn * r).astype(np.float32)
    s = (z * z).astype(np.float32)
    p = np.full_like(z, c[6])
    for k in range(5, -1, -1):
        p = fma32(p, s, np.full_like(z, c[k]))
    p = (p * z).astype(np.float32)
    t = np.where(ay > ax, (f32(1.5707963267948966) - p).astype(np.float32), p)
    t = np.where(af < 0, (f32(3.141592653589793) - t).astype(np.float32), t)
    return np.copysign(t, bf).astype(np.float32)


def dense_angles():
    """Angles over the circle, dense near the octant lines, axes and every bin edge of
    the codebooks tested below."""
    th = list(np.linspace(-np.pi, np.pi, 200001))
    for n in (33, 64, 100, 128, 256):
        edges = (np.arange(-n // 2 - 1, n // 2 + 2) + 0.5) * 2 * np.pi / n
        for dl in (0, 1e-7, 3e-7, 1e-6, 3e-6, 7e-6, 9e-6, 1.2e-5, 3e-5):
            th.extend(edges + dl)
            th.extend(edges - dl)
    for k in range(-4, 5):
        for dl in (0, 1e-9, 1e-7, 1e-5):
            th.extend([k * np.pi / 4 + dl, k * np.pi / 4 - dl])
    th = np.array(th)
    return th[(th > -np.pi) & (th <= np.pi)]


@pytest.mark.parametrize("scale", [2.0 ** -59, 1e-3, 1.0, 3.7e4, 2.0 ** 59])
def test_angle_estimate_within_its_bound(scale):
    c = device_coefficients()
    th = dense_angles()
    a, b = scale * np.cos(th), scale * np.sin(th)
    exact = np.arctan2(b, a)
    for v in range(3):
        est = angle_f32(a, b, c, v).astype(np.float64)
        err = np.abs(np.angle(np.exp(1j * (est - exact))))
        assert err.max() < 8e-7, (scale, v, err.max())


@pytest.mark.parametrize("n", [33, 64, 100, 128, 256])
def test_angle_code_fast_path_equals_binary64(n):
    c = device_coefficients()
    th = dense_angles()
    a, b = np.cos(th) * 1.7, np.sin(th) * 1.7
    t = np.arctan2(b, a) * n / (2 * np.pi)
    exact = np.mod(np.floor(t + 0.5), n).astype(np.int64)
    bpr = f32(n / (2 * np.pi))
    trust = (f32(0.5) - (f32(8e-6) * bpr).astype(np.float32)).astype(np.float32)
    for v in range(3):
        est = angle_f32(a, b, c, v)
        x = (est * bpr).astype(np.float32)  # position in bins
        cf = np.rint(x)
        res = (x - cf).astype(np.float32)
        trusted = np.abs(res) <= trust
        code = np.mod(cf.astype(np.int64), n)
        assert trusted.mean() > 0.95
        bad = trusted & (code != exact)
        assert not bad.any(), (n, v, th[bad][:5])


def fp16_values(lo, hi, count):
    x = np.geomspace(lo, hi, count)
    return np.unique(x.astype(np.float16).astype(np.float64))


def test_key_level_fast_path_equals_binary64():
    for s in fp16_values(1e-3, 65504, 40):
        m = np.arange(1, 256)
        thr = (m - 0.5) * s / 255  # radii on the level boundaries
        r = np.concatenate([thr * (1 + d) for d in (0, 1e-7, -1e-7, 1e-5, -1e-5, 3e-4, -3e-4)]
                           + [np.linspace(0, s, 5001)])
        r = r[(r >= 0) & (r <= s)]
        r2 = r * r
        exact = np.clip(np.floor(255 * np.sqrt(r2) / s + 0.5), 0, 255)
        for vr in range(3):
            sc255 = (f32(255) * ulp_variants(f32(1) / f32(s))[vr]).astype(np.float32)
            for vs in range(3):
                sq = ulp_variants(np.sqrt(r2.astype(np.float32)).astype(np.float32))[vs]
                for fused in (True, False):
                    if fused:
                        t = fma32(sq, np.full_like(sq, sc255), np.full_like(sq, f32(0.5)))
                    else:
                        t = ((sq * sc255).astype(np.float32) + f32(0.5)).astype(np.float32)
                    t = np.minimum(t, f32(256))
                    trusted = np.abs(t - np.rint(t)) >= f32(5e-4)
                    level = np.clip(np.floor(t), 0, 255)
                    bad = trusted & (level != exact)
                    assert not bad.any(), (s, r[bad][:3])


def test_value_level_fast_path_equals_binary64():
    rng = np.random.default_rng(5)
    for _ in range(60):
        smin = fp16_values(2.0 ** -14, 1e3, 1)[0] * 10 ** rng.uniform(0, 2)
        smin = float(np.float16(smin))
        smax = float(np.float16(smin * 10 ** rng.uniform(0.01, 3)))
        if not smax > smin or smax > 65504:
            continue
        L = np.log(smax / smin)
        m = np.arange(1, 16)
        thr = smin * np.exp((m - 0.5) * L / 15)
        r = np.concatenate([thr * (1 + d) for d in (0, 1e-7, -1e-7, 1e-6, -1e-6, 1e-5, -1e-5)]
                           + [np.geomspace(smin, smax, 4001)])
        r2 = r * r
        exact = np.clip(np.floor(15 * np.log(np.sqrt(r2) / smin) / L + 0.5), 0, 15)
        l2f = np.log2((f32(smax) * (f32(1) / f32(smin))).astype(np.float32)).astype(np.float32)
        for vl in range(3):
            scale = (f32(7.5) * ulp_variants(f32(1) / ulp_variants(l2f)[vl])[0]).astype(np.float32)
            inv = ulp_variants(f32(1) / f32(smin * smin))[vl]
            arg = (r2.astype(np.float32) * inv).astype(np.float32)
            for vg in range(3):
                lr = ulp_variants(np.log2(arg).astype(np.float32))[vg]
                t = np.minimum(fma32(lr, np.full_like(lr, scale), np.full_like(lr, f32(0.5))),
                               f32(16))
                fl = np.floor(t)
                # the device bounds |lr| by 2 l2 + 1 for the whole vector
                trust = (f32(0.5) - (scale * (f32(4e-6) + f32(1e-6) * (f32(2) * l2f + f32(1)))
                                     + f32(2e-5))).astype(np.float32)
                assert (np.abs(lr) <= 2 * l2f + 1).all()
                trusted = np.abs((t - fl - f32(0.5)).astype(np.float32)) <= trust
                level = np.clip(fl, 0, 15)
                bad = trusted & (level != exact)
                assert not bad.any(), (smin, smax, r[bad][:3])


@pytest.mark.parametrize("d", [64, 128])
def test_fp16_pairs_inside_estimate_range(d):
    """For fp16 inputs the encoder skips the estimate's range test: every nonzero
    rotated component is a signed sum of fp16 values (multiples of 2^-24) scaled by
    1/sqrt(d), and at most 65504 sqrt(d) in size. Checked on the extremes: one smallest
    subnormal, a vector of +-65504, and random mixtures of tiny and huge values."""
    from oracle import codec
    rng = np.random.default_rng(11)
    sg = codec.layer_signs(0, 0, d)
    xs = [np.zeros(d), np.full(d, 65504.0), np.where(sg > 0, 65504.0, -65504.0)]
    xs[0][rng.integers(d)] = 2.0 ** -24
    for _ in range(200):
        x = np.where(rng.random(d) < 0.5, 2.0 ** -24 * rng.integers(1, 4, d),
                     65504.0 * rng.choice([-1.0, 1.0], d))
        x[rng.random(d) < 0.7] = 0.0
        xs.append(x.astype(np.float16).astype(np.float64))
    for x in xs:
        y = codec.rotate(x[None], sg)[0]
        nz = np.abs(y[y != 0.0])
        assert nz.size == 0 or (nz.min() >= 2.0 ** -60 and nz.max() <= 2.0 ** 60)
        assert np.abs(y).max() <= 65504.0 * np.sqrt(d)
        nzp = np.maximum(np.abs(y[0::2]), np.abs(y[1::2]))
        nzp = nzp[nzp > 0]
        assert nzp.size == 0 or nzp.min() >= 2.0 ** -24 / np.sqrt(d)
