"""The binding refuses device buffers the kernels could not use safely (CPU only).

The C ABI receives raw pointers and cannot see a buffer's size, placement or
element type, so the Python binding checks torch tensors before any call:
GPU placement, contiguity, element type against the dtype code, and size
against batch x cols (x), batch x rows (y) or rows x cols (dequant output).
These tests use CPU tensors and stand-in tensor objects, so no GPU is needed
and no kernel is ever launched."""
import numpy as np
import pytest
import torch

from block_quantized_weight_qmv_amd import qmv

FAKE = 1 << 40  # an aligned address that is never dereferenced


class DevTensor:
    """Stand-in for a device tensor: only what the binding's checks look at."""

    def __init__(self, dtype, numel, contiguous=True):
        self.dtype, self._n, self._c = dtype, numel, contiguous
        self.is_cuda = True

    def is_contiguous(self):
        return self._c

    def numel(self):
        return self._n

    def element_size(self):
        return torch.empty(0, dtype=self.dtype).element_size()

    def data_ptr(self):
        return FAKE


def _w(rows=8, cols=512):
    return qmv.qmv_create_weights("q4_k", rows, cols, FAKE, qmv.qmv_packed_size("q4_k", rows, cols))


def _status(fn, *a):
    with pytest.raises(qmv.QmvError) as e:
        fn(*a)
    return e.value.status


def test_gemv_refuses_host_and_bad_tensors():
    w = _w()
    y = DevTensor(torch.float32, 8)
    x = DevTensor(torch.float32, 512)
    assert _status(qmv.qmv_gemv, "q4_k", w, torch.zeros(512), "f32", y, 8, 512, 1) == -6   # CPU tensor
    assert _status(qmv.qmv_gemv, "q4_k", w, np.zeros(512, np.float32), "f32", y, 8, 512, 1) == -6
    assert _status(qmv.qmv_gemv, "q4_k", w, DevTensor(torch.float32, 512, False), "f32", y, 8, 512, 1) == -6
    assert _status(qmv.qmv_gemv, "q4_k", w, DevTensor(torch.float16, 512), "f32", y, 8, 512, 1) == -2
    assert _status(qmv.qmv_gemv, "q4_k", w, DevTensor(torch.float32, 511), "f32", y, 8, 512, 1) == -5
    assert _status(qmv.qmv_gemv, "q4_k", w, DevTensor(torch.float32, 1023), "f32", DevTensor(torch.float32, 16),
                   8, 512, 2) == -5                                                          # x of batch 2
    assert _status(qmv.qmv_gemv, "q4_k", w, x, "f32", DevTensor(torch.float32, 7), 8, 512, 1) == -5
    assert _status(qmv.qmv_gemv, "q4_k", w, x, "f32", DevTensor(torch.float16, 16), 8, 512, 1) == -2
    assert _status(qmv.qmv_gemv, "q4_k", w, DevTensor(torch.float32, 256), "bf16", y, 8, 512, 1) == -2
    # bf16 activations as bfloat16 or as their 16-bit patterns; sizes counted in elements
    for dt in (torch.bfloat16, torch.int16):
        assert _status(qmv.qmv_gemv, "q4_k", w, DevTensor(dt, 511), "bf16", y, 8, 512, 1) == -5


def test_gemv_multi_checks_every_item():
    w = _w()
    ok = (w, DevTensor(torch.float16, 512), DevTensor(torch.float32, 8))
    bad_y = (w, DevTensor(torch.float16, 512), DevTensor(torch.float32, 4))
    with pytest.raises(qmv.QmvError, match="item 1 y"):
        qmv.qmv_gemv_multi("q4_k", "f16", 1, [ok, bad_y])
    with pytest.raises(qmv.QmvError, match="item 0 x"):
        qmv.qmv_gemv_multi("q4_k", "f16", 1, [(w, torch.zeros(512, dtype=torch.float16), ok[2])])


def test_dequant_and_create_checks():
    w = _w()
    assert _status(qmv.qmv_dequant, w, DevTensor(torch.float32, 8 * 512 - 1), "f32") == -5
    assert _status(qmv.qmv_dequant, w, DevTensor(torch.float16, 8 * 512), "f32") == -2
    assert _status(qmv.qmv_dequant, w, torch.zeros(8 * 512), "f32") == -6
    n = qmv.qmv_packed_size("q4_k", 8, 512)
    assert _status(qmv.qmv_create_weights, "q4_k", 8, 512, torch.zeros(n, dtype=torch.uint8)) == -6
    assert _status(qmv.qmv_create_weights, "q4_k", 8, 512, DevTensor(torch.uint8, n - 16), n) == -5


def test_swiglu_and_caller_workspace_checks():
    w = _w()
    x, h = DevTensor(torch.float32, 512), DevTensor(torch.float32, 8)
    with pytest.raises(qmv.QmvError, match="not on a GPU"):
        qmv.qmv_gemv_swiglu("q4_k", w, w, torch.zeros(512), "f32", h, 8, 512, 1)
    with pytest.raises(qmv.QmvError, match="needs 8"):
        qmv.qmv_gemv_swiglu("q4_k", w, w, x, "f32", DevTensor(torch.float32, 7), 8, 512, 1)
    with pytest.raises(qmv.QmvError, match="dtype"):
        qmv.qmv_gemv_swiglu("q4_k", w, w, DevTensor(torch.float16, 512), "f32", h, 8, 512, 1)
    ok = (w, x, h)
    with pytest.raises(qmv.QmvError, match="workspace: holds 100"):
        qmv.qmv_gemv_multi_ws("q4_k", "f32", 1, [ok], DevTensor(torch.uint8, 100), 256)
    with pytest.raises(qmv.QmvError, match="not on a GPU"):
        qmv.qmv_gemv_multi_ws("q4_k", "f32", 1, [ok], torch.zeros(256, dtype=torch.uint8), 256)
