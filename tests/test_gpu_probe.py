"""The read-only streaming probe reads every 16-byte word it is given: a buffer whose
words fold (XOR) to the probe's constant in exactly one thread makes that thread write
the constant to the sink, and an ordinary buffer leaves the sink untouched."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("rotated_angle_quantization_amd")

MAGIC = 0x9E3779B9


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.mark.parametrize("n16", [1, 1000, 1 << 20, (1 << 22) + 77])
def test_probe_reads_every_word(dev, n16):
    # word k is read by lane k % 64 of the wave that owns its 512-word chunk; with only
    # word k nonzero, only that lane folds to the constant and writes it, to sink slot
    # k % 64. Checked for the first and last words and words in between (the last chunk
    # is partial unless n16 is a multiple of 512).
    rng = np.random.default_rng(n16)
    for k in sorted({0, n16 - 1, n16 // 2, n16 // 3, int(rng.integers(n16))}):
        words = np.zeros(n16 * 4, dtype=np.uint32)
        words[k * 4 + 2] = MAGIC
        buf = torch.from_numpy(words.view(np.int32)).to(dev)
        sink = torch.zeros(64, dtype=torch.int32, device=dev)
        kvq.probe_read(buf, sink)
        torch.cuda.synchronize()
        got = sink.cpu().numpy().view(np.uint32)
        want = np.zeros(64, dtype=np.uint32)
        want[k % 64] = MAGIC
        np.testing.assert_array_equal(got, want, err_msg=f"n16 {n16} word {k}")


def test_probe_ordinary_buffer_leaves_sink(dev):
    buf = torch.arange(1 << 20, dtype=torch.int32, device=dev)
    sink = torch.zeros(64, dtype=torch.int32, device=dev)
    kvq.probe_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.count_nonzero()) == 0
