"""qmv_dequant on the GPU against the oracle: bit-exact (+0 and -0 compare equal)."""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_weight_qmv_amd import qmv
from gpu_util import DEV, Weights, say

pytestmark = pytest.mark.gpu

FMTS = ("q8_0", "q4_k", "q6_k", "int4_g128", "q5_k")
SHAPES = [(1, 1), (3, 2), (37, 14), (130, 17), (5, 74)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,nblk", SHAPES)
def test_dequant_f32_bit_exact(fmt, rows, nblk):
    cols = nblk * oracle.QK[fmt]
    say(f"dequant f32 {fmt} {rows}x{cols}")
    w = Weights(fmt, rows, cols, seed=900 + rows + nblk)
    out = torch.full((rows, cols), float("nan"), dtype=torch.float32, device=DEV)
    qmv.qmv_dequant(w.desc, out, "f32")
    got = out.cpu().numpy()
    want = oracle.dequant32(fmt, w.oracle_bytes(), rows, cols)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("out_dtype", ["f16", "bf16"])
def test_dequant_half_outputs_round_to_nearest_even(fmt, out_dtype):
    rows, cols = 19, 3 * oracle.QK[fmt]
    say(f"dequant {out_dtype} {fmt} {rows}x{cols}")
    w = Weights(fmt, rows, cols, seed=77)
    tdt = torch.float16 if out_dtype == "f16" else torch.bfloat16
    out = torch.empty((rows, cols), dtype=tdt, device=DEV)
    qmv.qmv_dequant(w.desc, out, out_dtype)
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    w32 = oracle.dequant32(fmt, w.oracle_bytes(), rows, cols)
    if out_dtype == "f16":
        want = w32.astype(np.float16).view(np.uint16)
    else:
        want = oracle.f32_to_bf16_bits_rne(w32)
    zero = (want & 0x7FFF) == 0
    assert np.array_equal(np.where(zero, 0, got), np.where(zero, 0, want))


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_edge_scales(fmt):
    """Zero, subnormal, largest and negative fp16 scales; extreme codes."""
    rows, cols = 8, 2 * oracle.QK[fmt]
    from synth import gen_weights
    f = gen_weights(fmt, rows, cols, 5)
    sk = "s_bits" if fmt == "int4_g128" else "d_bits"
    f[sk][...] = np.resize(np.array([0x0000, 0x0001, 0x03FF, 0x7BFF, 0xBC00, 0x8001], np.uint16), f[sk].shape)
    if fmt in ("q4_k", "q5_k"):
        f["dmin_bits"][...] = np.resize(np.array([0x7BFF, 0x0000, 0x0001, 0x3C00], np.uint16), f["dmin_bits"].shape)
    key, lo, hi = {"q8_0": ("q", -128, 127), "q4_k": ("u", 0, 15), "q6_k": ("q", 0, 63),
                   "int4_g128": ("q", -8, 7), "q5_k": ("u", 0, 31)}[fmt]
    f[key][::2] = lo
    f[key][1::2] = hi
    w = Weights(fmt, rows, cols, fields=f)
    out = torch.empty((rows, cols), dtype=torch.float32, device=DEV)
    qmv.qmv_dequant(w.desc, out, "f32")
    assert np.array_equal(out.cpu().numpy(), oracle.dequant32(fmt, w.oracle_bytes(), rows, cols))
