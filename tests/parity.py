"""Comparison rules between the HIP library and the oracle (used by the GPU tests and
the smoke check).

  codes      bit-exact; an angle-code mismatch is excused only when the oracle's
             float64 angle lies within 1e-6 rad of a bin boundary, and excused
             mismatches must stay below 1e-5 of the pairs compared. An angle exactly on
             a boundary (a tie: the oracle's float64 angle within 1e-12 rad of it, which
             only pairs at multiples of pi/4 can reach exactly) has two correct codes,
             the two bins that meet there; either is accepted and not counted. Radius
             codes and fp16 parameters must always match.
  dequant    ||x_hat_gpu - x_hat_oracle||_2 <= 1e-3 ||x||_2 per (token, kv head), both
             decoding the same code bytes.
  attention  ||o_gpu - o_oracle||_2 / ||o_oracle||_2 <= 2e-3 per (batch, query head),
             o_oracle computed by the plain definition on the oracle's dequantisation of
             the same cache bytes.
"""

from __future__ import annotations

import sys

import numpy as np

from oracle import codec as oc
from oracle import layout as ol

ANGLE_EXEMPT_RAD = 1e-6
ANGLE_TIE_RAD = 1e-12
EXEMPT_FRACTION = 1e-5
DEQUANT_TOL = 1e-3
ATTN_TOL = 2e-3


def note(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def oracle_encode(x_k: np.ndarray, x_v: np.ndarray, signs: np.ndarray, n_k: int, n_v: int):
    ek, ev = oc.encode_k(x_k, signs, n_k), oc.encode_v(x_v, signs, n_v)
    ek["n"], ev["n"] = n_k, n_v
    return ek, ev


def compare_codes(got: dict, ek: dict, ev: dict) -> dict:
    """got: unpacked GPU codes (arrays [..., P] / [...]); ek, ev: oracle encodings of the
    same vectors (same leading shape). Asserts the code rule; returns counts."""
    stats = {}
    pairs = 0
    excused_total = 0
    for name, enc, angle_key in (("k", ek, "k_angle"), ("v", ev, "v_angle")):
        n = enc["n"]
        mism = got[angle_key] != enc["angle"]
        # exact ties: either bin meeting at the boundary is correct
        tie = oc.angle_near_boundary(enc["theta"], n, tol=ANGLE_TIE_RAD) & (enc["r"] != 0.0)
        t = oc.angle_position(enc["theta"], n)
        lower = np.mod(np.floor(t), n).astype(np.int64)
        upper = np.mod(lower + 1, n)
        tie_ok = tie & ((got[angle_key] == lower) | (got[angle_key] == upper))
        mism &= ~tie_ok
        bad = mism & ~enc["near_boundary"]
        if bad.any():
            idx = np.argwhere(bad)[:5]
            raise AssertionError(f"{name} angle codes differ away from bin boundaries at "
                                 f"{idx.tolist()} (gpu {got[angle_key][bad][:5]}, oracle "
                                 f"{enc['angle'][bad][:5]}); {int(bad.sum())} total")
        excused_total += int(mism.sum())
        pairs += mism.size
        stats[f"{name}_angle_excused"] = int(mism.sum())
    assert excused_total <= EXEMPT_FRACTION * pairs, (excused_total, pairs)
    np.testing.assert_array_equal(got["k_radius"], ek["radius"], err_msg="key radius codes")
    np.testing.assert_array_equal(got["v_radius"], ev["radius"], err_msg="value radius codes")
    np.testing.assert_array_equal(got["k_scale"], ek["scale"], err_msg="key fp16 scale")
    np.testing.assert_array_equal(got["v_smin"], ev["s_min"], err_msg="value fp16 s_min")
    np.testing.assert_array_equal(got["v_smax"], ev["s_max"], err_msg="value fp16 s_max")
    stats["pairs"] = pairs
    return stats


def oracle_dequant(got: dict, signs: np.ndarray, n_k: int, n_v: int):
    k_hat = oc.dequant_k(got["k_angle"], got["k_radius"], got["k_scale"], n_k, signs)
    v_hat = oc.dequant_v(got["v_angle"], got["v_radius"], got["v_smin"], got["v_smax"], n_v,
                         signs)
    return k_hat, v_hat


FP16_HALF_SUBNORMAL = 2.0 ** -25


def compare_dequant(gpu_hat: np.ndarray, ref_hat: np.ndarray, x: np.ndarray, what: str,
                    fp16_out: bool = False):
    """Per-vector bound 1e-3 ||x||. An fp16 output cannot resolve values below the fp16
    subnormal spacing 2^-24, so fp16 outputs also get half that spacing per element
    (sqrt(d) 2^-25 in norm): the storage format's own quantum, not codec error."""
    err = np.linalg.norm(gpu_hat.astype(np.float64) - ref_hat, axis=-1)
    norm = np.linalg.norm(x.astype(np.float64), axis=-1)
    bound = DEQUANT_TOL * norm
    if fp16_out:
        bound = bound + np.sqrt(x.shape[-1]) * FP16_HALF_SUBNORMAL
    ok = err <= bound + 1e-30
    if not ok.all():
        i = np.argwhere(~ok)[:5]
        raise AssertionError(f"{what}: dequant error above 1e-3 |x| at {i.tolist()}: "
                             f"err {err[~ok][:5]}, |x| {norm[~ok][:5]}")
    return float(np.max(err / np.maximum(norm, 1e-30)))


def compare_attention(gpu_out: np.ndarray, ref_out: np.ndarray, what: str) -> float:
    num = np.linalg.norm(gpu_out.astype(np.float64) - ref_out, axis=-1)
    den = np.linalg.norm(ref_out, axis=-1)
    rel = num / np.maximum(den, 1e-30)
    if not (rel <= ATTN_TOL).all():
        i = np.argwhere(rel > ATTN_TOL)[:5]
        raise AssertionError(f"{what}: attention rel-L2 above 2e-3 at {i.tolist()}: "
                             f"{rel[rel > ATTN_TOL][:5]}")
    return float(rel.max())


def unpack(cache_np: np.ndarray, cfg_d, n_k, n_v, batch, hkv, capacity, t0, ntok) -> dict:
    return ol.unpack_cache(cache_np, cfg_d, n_k, n_v, batch, hkv, capacity, t0, ntok)
