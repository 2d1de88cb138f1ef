"""Floating-point encodings used by the block formats, written from IEEE 754.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* binary16 (fp16): 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
  Block scales of every format are fp16, little-endian.
* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits; the upper
  half of a binary32.  Activations of the batched path are bf16.

Infinities and NaNs are outside the block-format contract (no scale may be
one), so the decoders reject them instead of inventing a value.
"""
from __future__ import annotations

import numpy as np


def fp16_bits_to_f64(bits) -> np.ndarray:
    """Exact float64 value of each binary16 bit pattern.

    normal:    (-1)^s * (1024 + f) * 2^(e - 25)      for 1 <= e <= 30
    subnormal: (-1)^s * f * 2^-24                    for e == 0
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    s = b >> 15
    e = (b >> 10) & 0x1F
    f = b & 0x3FF
    if np.any(e == 0x1F):
        raise ValueError("fp16 Inf/NaN is not a valid block scale")
    mag = np.where(e == 0, np.ldexp(f.astype(np.float64), -24),
                   np.ldexp((1024 + f).astype(np.float64), e - 25))
    return np.where(s == 1, -mag, mag)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact float64 value of each bfloat16 bit pattern.

    normal:    (-1)^s * (128 + f) * 2^(e - 134)      for 1 <= e <= 254
    subnormal: (-1)^s * f * 2^-133                   for e == 0
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    s = b >> 15
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    if np.any(e == 0xFF):
        raise ValueError("bf16 Inf/NaN activations are not supported")
    mag = np.where(e == 0, np.ldexp(f.astype(np.float64), -133),
                   np.ldexp((128 + f).astype(np.float64), e - 134))
    return np.where(s == 1, -mag, mag)


def f32_to_bf16_bits_rne(x) -> np.ndarray:
    """Round finite float32 values to bfloat16, nearest with ties to even.

    The low 16 bits of the binary32 pattern are the discarded fraction.  Adding
    0x7FFF plus the lowest kept bit and truncating rounds up exactly when the
    discarded part exceeds half an ulp, or equals it and the kept bit is odd.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    if np.any((u & 0x7F800000) == 0x7F800000):
        raise ValueError("non-finite value")
    keep_lsb = (u >> 16) & 1
    return ((u + 0x7FFF + keep_lsb) >> 16).astype(np.uint16)
