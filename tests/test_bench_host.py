"""Host-side checks of bench.py that need no GPU: the one-GPU contract, the oracle CPU
baseline it reports, and the kernel name it matches against the profiler's records."""

import json
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402
from synthetic import get  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_is_the_oracle_on_a_bounded_sample():
    out = bench.cpu_baseline(get("tinyllama"), 0.01)
    assert out["kind"] == "oracle" and out["unit"] == "GB/s"
    assert out["cores"] == len(os.sched_getaffinity(0))
    assert out["value"] > 0 and out["decode_token_heads_per_s"] > 0
    assert out["encode_token_heads_per_s"] > 0 and out["cpu_model"]
    assert "layers [0, 21]" in out["sample"] and "first 64 tokens" in out["sample"]
    json.dumps(out)


@pytest.mark.parametrize("d,g,nk,nv,name", [
    (128, 4, 128, 64, "attn_decode_kernel<128, 4, 7, 6, 6>"),     # half table + MFMA values
    (128, 4, 256, 256, "attn_decode_kernel<128, 4, 8, 8, 7>"),    # 8-bit keys: MFMA both
    (128, 4, 100, 40, "attn_decode_kernel<128, 4, 7, 6, 5>"),     # full table + MFMA values
    (128, 4, 128, 256, "attn_decode_kernel<128, 4, 7, 8, 6>"),    # half table + MFMA values
    (128, 4, 100, 256, "attn_decode_kernel<128, 4, 7, 8, 1>"),    # full table, vector values
    (128, 4, 200, 40, "attn_decode_kernel<128, 4, 8, 6, 7>"),     # no table fits: MFMA
    (128, 2, 100, 40, "attn_decode_kernel<128, 2, 7, 6, 5>"),     # full table + MFMA values
    (128, 2, 256, 256, "attn_decode_kernel<128, 2, 8, 8, 6>"),    # half table + MFMA values
    (128, 8, 200, 256, "attn_decode_kernel<128, 8, 8, 8, 7>"),
    (64, 8, 128, 64, "attn_decode_kernel<64, 8, 7, 6, 7>"),
    (64, 4, 128, 64, "attn_decode_kernel<64, 4, 7, 6, 6>"),
    (128, 2, 128, 64, "attn_decode_kernel<128, 2, 7, 6, 5>"),     # two heads: full table
])
def test_kernel_name_follows_the_variant_rule(d, g, nk, nv, name):
    assert bench.attn_kernel_name(d, g, nk, nv) == name


@pytest.mark.parametrize("d,nk,nv,per_token_head", [
    # record of one token-head: key angle codes, key radius bytes and fp16 scale; value
    # angle codes, radius nibbles and two fp16 parameters
    (128, 128, 64, 64 * 7 // 8 + 64 + 2 + 64 * 6 // 8 + 64 // 2 + 4),   # 206
    (128, 256, 256, 64 + 64 + 2 + 64 + 32 + 4),                         # 230
    (64, 128, 64, 32 * 7 // 8 + 32 + 2 + 32 * 6 // 8 + 16 + 4),         # 106
])
def test_algorithmic_bytes_are_the_record_sizes(d, nk, nv, per_token_head):
    pytest.importorskip("rotated_angle_quantization_amd")
    assert bench.record_bytes(d, nk, nv, 4096) == 4096 * per_token_head
