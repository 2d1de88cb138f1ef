"""The GEMV the fused kernels must reproduce, by its plain definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

hipEngine 0.3.0, "Core principles": every fused composite has an unfused chain
that is the correctness baseline.  Here the unfused chain is: dequantize every
weight exactly (``dequant64``), convert the activations exactly to float64,
and take the float64 product  y64[b, r] = sum_k W[r, k] * x[b, k].

x is [batch, cols] and y is [batch, rows], the layout of the C ABI.

Tolerance definitions (the GPU accumulates in float32, so its sums are not
unique; only these bounds are):

* normwise relative error per batch row b:
      max_r |y[b, r] - y64[b, r]| / max_r |y64[b, r]|
  gated at 2e-3 for the GEMVs.
* elementwise a-priori bound, valid for any float32 summation order when the
  weights and activations enter exactly:
      |y - y64| <= gamma_{K+1} * sum_k |W[r, k] x[b, k]|,
      gamma_n = n u / (1 - n u),  u = 2^-24
  (Higham, "Accuracy and Stability of Numerical Algorithms", section 3.1).
"""
from __future__ import annotations

import numpy as np

from .formats import dequant64, row_slice
from .fp import bf16_bits_to_f64, fp16_bits_to_f64


def x_to_f64(x, x_dtype: str) -> np.ndarray:
    """Exact float64 value of activations given as f32 / f16 arrays or bf16 bits."""
    x = np.asarray(x)
    if x_dtype == "f32":
        if x.dtype != np.float32:
            raise TypeError("f32 activations must be float32")
        return x.astype(np.float64)
    if x_dtype == "f16":
        if x.dtype != np.float16:
            raise TypeError("f16 activations must be float16")
        return fp16_bits_to_f64(x.view(np.uint16))
    if x_dtype == "bf16":
        if x.dtype != np.uint16:
            raise TypeError("bf16 activations are passed as uint16 bit patterns")
        return bf16_bits_to_f64(x)
    raise ValueError(f"unknown activation dtype {x_dtype!r}")


def gemv64(fmt: str, data, rows: int, cols: int, x, x_dtype: str,
           row_chunk: int = 4096) -> np.ndarray:
    """y64 = x64 @ W64^T, float64 [batch, rows]; W decoded in row chunks."""
    x64 = x_to_f64(x, x_dtype).reshape(-1, cols)
    y = np.empty((x64.shape[0], rows), np.float64)
    for r0 in range(0, rows, row_chunk):
        r1 = min(rows, r0 + row_chunk)
        w = dequant64(fmt, row_slice(fmt, data, rows, cols, r0, r1), r1 - r0, cols)
        y[:, r0:r1] = x64 @ w.T
    return y


def gemv64_rows(fmt: str, data, rows: int, cols: int, x, x_dtype: str,
                row_ids) -> np.ndarray:
    """y64 restricted to the given rows: float64 [batch, len(row_ids)]."""
    x64 = x_to_f64(x, x_dtype).reshape(-1, cols)
    ids = np.asarray(row_ids, np.int64)
    w = np.stack([dequant64(fmt, row_slice(fmt, data, rows, cols, int(r), int(r) + 1), 1, cols)[0]
                  for r in ids])
    return x64 @ w.T


def normwise_rel_err(y, y64) -> np.ndarray:
    """Per batch row b: max_r |y[b, r] - y64[b, r]| / max_r |y64[b, r]| (float64).

    The reduction runs over the output rows r (the last axis), one value per
    activation row b.  Two cases the ratio leaves open are fixed here:

    * an all-zero reference row (max_r |y64| = 0, e.g. every weight of the
      matrix zero): every exact product is then zero and any float32 sum of
      them is exactly zero, so the only acceptable result is exact zero --
      the error is 0 if y is zero there and +inf otherwise;
    * a NaN or infinity in y gives +inf, so no NaN can slip through a
      ``<=`` comparison.
    """
    y = np.asarray(y, np.float64).reshape(np.shape(y64))
    y64 = np.asarray(y64, np.float64)
    diff = np.abs(y - y64)
    diff = np.where(np.isfinite(diff), diff, np.inf)
    num = np.max(diff, axis=-1)
    den = np.max(np.abs(y64), axis=-1)
    zero_ref = den == 0
    safe = np.where(zero_ref, 1.0, den)
    return np.where(zero_ref, np.where(num == 0, 0.0, np.inf), num / safe)


def gamma(n: int) -> float:
    """gamma_n = n u / (1 - n u) with u = 2^-24, the float32 unit roundoff."""
    u = 2.0 ** -24
    return n * u / (1 - n * u)


def elementwise_bound(fmt: str, data, rows: int, cols: int, x, x_dtype: str,
                      row_chunk: int = 4096) -> np.ndarray:
    """gamma_{K+1} * sum_k |W[r, k] x[b, k]|, float64 [batch, rows].

    A diagnostic, not a gate: it bounds a float32 dot product of exact
    operands in any summation order.  Kernels that apply scales after partial
    sums (the factored sub-block form) round differently and may exceed it."""
    x64 = np.abs(x_to_f64(x, x_dtype).reshape(-1, cols))
    out = np.empty((x64.shape[0], rows), np.float64)
    for r0 in range(0, rows, row_chunk):
        r1 = min(rows, r0 + row_chunk)
        w = np.abs(dequant64(fmt, row_slice(fmt, data, rows, cols, r0, r1), r1 - r0, cols))
        out[:, r0:r1] = x64 @ w.T
    return gamma(cols + 1) * out


def gemv64_and_bound(fmt: str, data, rows: int, cols: int, x, x_dtype: str,
                     row_chunk: int = 4096):
    """(gemv64, elementwise_bound) of the same operands, each row chunk decoded once."""
    x64 = x_to_f64(x, x_dtype).reshape(-1, cols)
    ax = np.abs(x64)
    y = np.empty((x64.shape[0], rows), np.float64)
    b = np.empty_like(y)
    for r0 in range(0, rows, row_chunk):
        r1 = min(rows, r0 + row_chunk)
        w = dequant64(fmt, row_slice(fmt, data, rows, cols, r0, r1), r1 - r0, cols)
        y[:, r0:r1] = x64 @ w.T
        b[:, r0:r1] = ax @ np.abs(w).T
    return y, gamma(cols + 1) * b


def elementwise_bound_rows(fmt: str, data, rows: int, cols: int, x, x_dtype: str,
                           row_ids) -> np.ndarray:
    """elementwise_bound restricted to the given rows: float64 [batch, len(row_ids)]."""
    x64 = np.abs(x_to_f64(x, x_dtype).reshape(-1, cols))
    ids = np.asarray(row_ids, np.int64)
    w = np.stack([dequant64(fmt, row_slice(fmt, data, rows, cols, int(r), int(r) + 1), 1, cols)[0]
                  for r in ids])
    return gamma(cols + 1) * (x64 @ np.abs(w).T)


def silu64(g) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g)) in float64, elementwise.

    hipfire's Qwen2 decoder ("Key Technical Specifications") names a SwiGLU
    FFN; silu is the gate nonlinearity of SwiGLU.  For g below about -709,
    exp(-g) overflows to +inf and the quotient is -0, the limit of silu."""
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu64(fmt: str, gate_data, up_data, rows: int, cols: int, x, x_dtype: str,
             row_ids=None) -> np.ndarray:
    """h64 = silu(W_gate x) * (W_up x), float64 [batch, rows] (or the listed rows).

    The SwiGLU FFN input of hipfire's Qwen2 decoder, computed by the unfused
    chain that hipEngine 0.3.0 ("Core principles") keeps beside every fused
    composite: the two GEMVs of the oracle, then the elementwise product of
    silu of the gate with the up projection, all in float64."""
    if row_ids is None:
        g = gemv64(fmt, gate_data, rows, cols, x, x_dtype)
        u = gemv64(fmt, up_data, rows, cols, x, x_dtype)
    else:
        g = gemv64_rows(fmt, gate_data, rows, cols, x, x_dtype, row_ids)
        u = gemv64_rows(fmt, up_data, rows, cols, x, x_dtype, row_ids)
    return silu64(g) * u
