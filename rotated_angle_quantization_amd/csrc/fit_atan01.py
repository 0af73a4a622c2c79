"""Fits the coefficients of atan01() in kvq_codec_dev.h and reports its error.

atan(z) on [0, 1] is approximated by an odd polynomial z * sum_{k<7} c_k z^(2k). The c_k
minimise the largest absolute error over a dense grid of z in [0, 1]: Lawson's
iteration (weighted least squares, each weight multiplied by its point's error after
every solve, which converges to the minimax solution on the grid), in float64; the
result is rounded to float32. The error is then measured with the kernel's evaluation
order (Horner in s = z^2 with fused multiply-adds, each rounded once to float32; the
final product p * z rounded to float32) against float64 atan.

    python rotated_angle_quantization_amd/csrc/fit_atan01.py

prints the float32 coefficients (highest degree first, as the kernel's Horner loop uses
them) and the maximum absolute error in radians.
"""

from __future__ import annotations

import numpy as np

TERMS = 7


def fit(n_grid: int = 40001, iterations: int = 200) -> np.ndarray:
    z = np.linspace(0.0, 1.0, n_grid)
    s = z * z
    a = np.stack([z * s ** k for k in range(TERMS)], axis=1)  # columns z^(2k+1)
    y = np.arctan(z)
    w = np.ones_like(z)
    for _ in range(iterations):
        sw = np.sqrt(w)
        c, *_ = np.linalg.lstsq(a * sw[:, None], y * sw, rcond=None)
        w = w * np.abs(a @ c - y)
        w /= w.sum()
    return c.astype(np.float32)  # c[k] multiplies z^(2k+1)


def fma32(a, b, c):
    """fmaf: the float32 product is exact in float64 (24 + 24 bits), so one rounding."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def atan01_f32(z: np.ndarray, c: np.ndarray) -> np.ndarray:
    z = z.astype(np.float32)
    s = (z * z).astype(np.float32)
    p = np.full_like(z, c[TERMS - 1])
    for k in range(TERMS - 2, -1, -1):
        p = fma32(p, s, np.full_like(z, c[k]))
    return (p * z).astype(np.float32)


def max_error(c: np.ndarray, n: int = 2_000_001) -> float:
    z = np.linspace(0.0, 1.0, n).astype(np.float32)
    return float(np.max(np.abs(atan01_f32(z, c).astype(np.float64) - np.arctan(z.astype(np.float64)))))


if __name__ == "__main__":
    c = fit()
    for k in range(TERMS - 1, -1, -1):
        print(f"c[{k}] = {float(c[k])!r}f")
    print(f"max |atan01 - atan| on [0, 1] in float32 evaluation: {max_error(c):.3e} rad")
