"""The HBM probes read (and copy) every byte they are given exactly once.

qmv_probe_read folds what it loads into one XOR per workgroup; the expected
values are the XORs of the words each workgroup's contiguous chunk covers
(chunks of whole 1024-vector steps, at most 1024 workgroups).  A probe that
skipped or repeated loads would give other values -- the byte counters are
calibrated on the assumption that it does neither.
"""
import numpy as np
import pytest
import torch

from block_quantized_weight_qmv_amd import qmv
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu

THREADS = 256


def _expected(words, blocks):
    """words: uint32 [nvec, 4]; XOR per workgroup of the words it reads."""
    nvec = words.shape[0]
    per_vec = np.bitwise_xor.reduce(words, axis=1)
    step = THREADS * 4  # workgroup b reads vectors [b chunk, (b + 1) chunk)
    chunk = -(-nvec // blocks)
    chunk = -(-chunk // step) * step
    out = np.zeros(blocks, dtype=np.uint32)
    starts = np.arange(0, nvec, chunk)
    out[:len(starts)] = np.bitwise_xor.reduceat(per_vec, starts)
    return (out & 0xFFFF).astype(np.float32)


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 7254016, 256 << 20, (256 << 20) + 16 * 1000],
                         ids=["16B", "ragged", "o-proj", "256MiB", "256MiB-ragged"])
def test_probe_read_folds_every_word(nbytes):
    say(f"probe read {nbytes} bytes")
    g = np.random.default_rng(nbytes % 1000)
    words = g.integers(0, 2 ** 32, size=(nbytes // 16, 4), dtype=np.uint32)
    src = torch.from_numpy(words.view(np.uint8).reshape(-1)).to(DEV)
    blocks = qmv.qmv_probe_read_outputs(nbytes)
    out = torch.full((blocks,), -1.0, dtype=torch.float32, device=DEV)
    qmv.qmv_probe_read(src, nbytes, out)
    torch.cuda.synchronize()
    assert blocks == max(1, min(1024, -(-(nbytes // 16) // (THREADS * 4))))
    want = _expected(words, blocks)
    np.testing.assert_array_equal(out.cpu().numpy(), want)


@pytest.mark.parametrize("nbytes", [16, 1 << 20, (3 << 20) + 48])
def test_probe_copy_copies(nbytes):
    say(f"probe copy {nbytes} bytes")
    g = np.random.default_rng(7)
    src = torch.from_numpy(g.integers(0, 256, size=nbytes, dtype=np.uint8)).to(DEV)
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device=DEV)
    qmv.qmv_probe_copy(src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert int(dst[nbytes:].abs().sum()) == 0
