"""The synthetic fidelity harness (bits per element against reconstruction, softmax and
attention error): its figures come from the library and must agree with the same
figures computed from the oracle's own encode, dequantisation and attention on the same
inputs; errors must shrink as the codebooks grow."""

import math

import numpy as np
import pytest
import torch

from oracle import codec as oc
from parity import note
from synthetic import get, layer_kv, query

kvq = pytest.importorskip("rotated_angle_quantization_amd")
from rotated_angle_quantization_amd import fidelity  # noqa: E402


def test_bits_per_element_matches_the_layout_definition():
    for d in (64, 128):
        for nk, nv in ((128, 64), (256, 256), (32, 32), (100, 40)):
            assert math.isclose(fidelity.bits_per_element(d, nk, nv),
                                oc.bits_per_element(d, nk, nv))


def oracle_fidelity(k, v, q, n_k, n_v, layer):
    """The harness's figures from the oracle: fp64 encode, dequantisation, attention."""
    x_k, x_v, qn = (t.detach().to("cpu", torch.float64).numpy() for t in (k, v, q))
    sg = oc.layer_signs(0, layer, x_k.shape[-1])
    ek, ev = oc.encode_k(x_k, sg, n_k), oc.encode_v(x_v, sg, n_v)
    kh = oc.dequant_k(ek["angle"], ek["radius"], ek["scale"], n_k, sg)
    vh = oc.dequant_v(ev["angle"], ev["radius"], ev["s_min"], ev["s_max"], n_v, sg)
    out = oc.attention(qn, kh, vh)
    ref = oc.attention(qn, x_k, x_v)
    return {
        "key_nmse": float(((kh - x_k) ** 2).sum() / (x_k ** 2).sum()),
        "value_nmse": float(((vh - x_v) ** 2).sum() / (x_v ** 2).sum()),
        "attn_rel_l2_mean": float((np.linalg.norm(out - ref, axis=-1)
                                   / np.linalg.norm(ref, axis=-1)).mean()),
    }


@pytest.mark.gpu
def test_fidelity_matches_oracle_and_shrinks_with_codebook_size():
    dev = torch.device("cuda:0")
    cfg = get("tinyllama")
    k, v = layer_kv(cfg, 1, dev, seq=1024)
    q = query(cfg, 1, dev)
    rows = fidelity.sweep(k, v, q, [64, 128, 256], layer=1, extra=[(128, 64)])
    for r in rows:
        note(f"[fidelity] n=({r['n_k']},{r['n_v']}) {r['bits_per_element']:.3f} b/elem "
             f"key {r['key_nmse']:.2e} value {r['value_nmse']:.2e} "
             f"KL {r['softmax_kl_mean']:.2e} attn {r['attn_rel_l2_mean']:.2e}")
    by = {(r["n_k"], r["n_v"]): r for r in rows}
    # key error falls with n_K (n_V fixed), value error with n_V (n_K fixed)
    kn = [by[(n, 256)]["key_nmse"] for n in (64, 128, 256)]
    vn = [by[(256, n)]["value_nmse"] for n in (64, 128, 256)]
    assert all(a > b for a, b in zip(kn, kn[1:])), kn
    assert all(a > b for a, b in zip(vn, vn[1:])), vn
    kl = [by[(n, 256)]["softmax_kl_mean"] for n in (64, 128, 256)]
    assert all(a > b for a, b in zip(kl, kl[1:])), kl
    # the value side leaves the softmax weights alone: same keys, same weights
    assert by[(256, 64)]["softmax_kl_mean"] == pytest.approx(by[(256, 256)]["softmax_kl_mean"])
    # parity with the oracle's own pipeline on the same inputs
    for nk, nv in ((128, 64), (64, 256)):
        ref = oracle_fidelity(k, v, q, nk, nv, 1)
        got = by[(nk, nv)]
        for key in ref:
            assert got[key] == pytest.approx(ref[key], rel=2e-2, abs=1e-7), (nk, nv, key)
