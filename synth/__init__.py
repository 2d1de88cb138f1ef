"""Seeded synthetic inputs for the block-quantized GEMV workloads.

This module only draws random numbers: integer codes, fp16 scale bit patterns
and activation vectors.  It contains none of the quantization method's
arithmetic (no packing, no decoding, no products), so the CPU oracle and the
HIP library can both be fed from it without sharing any part of the method.

Every tensor comes from ``numpy.random.Generator(PCG64(seed))`` with
``seed = 1000 * config + tensor_index``.  Distributions follow the workload
descriptions of the decode GEMV configurations:

* Q8_0: fp16 scale d ~ U(0.002, 0.02), int8 codes ~ U{-127..127}.
* Q4_K: fp16 d and dmin ~ U(0.001, 0.01), 6-bit sub-block scale and min
  ~ U{0..63}, 4-bit codes ~ U{0..15}.
* Q5_K: as Q4_K, with 5-bit codes ~ U{0..31}.
* Q6_K: fp16 d ~ U(0.001, 0.01), int8 sub-scales ~ U{-128..127}, 6-bit codes
  ~ U{0..63}.
* INT4 symmetric group-128: codes ~ U{-8..7}, fp16 group scale
  ~ U(0.005, 0.05).
* Activations ~ N(0, 1) in fp32, fp16 (numpy's rounding of the fp32 draw) or
  bf16 (the upper 16 bits of the fp32 draw).

The 7B-shaped matrix sizes (hidden 3584, FFN 18944, 4 KV heads of 128, vocab
152064) describe one decoder layer of a Qwen2.5-7B-class model, the model the
"annotated-llm-runtime" article (datastack.it summary, section "I numeri" and
the closing paragraph of "Tre bug che insegnano") runs with INT4 group-128
weights, and the Q4_K_M GGUF files hipEngine 0.3.0 serves ("GGUF Support").
"""
from __future__ import annotations

import numpy as np

QK = {"q8_0": 32, "q4_k": 256, "q6_k": 256, "int4_g128": 128, "q5_k": 256}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def fp16_uniform_bits(g: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    """Bit patterns of float16 values drawn U(lo, hi) (numpy's fp16 rounding)."""
    return g.uniform(lo, hi, size=shape).astype(np.float16).view(np.uint16)


def gen_q8_0(rows: int, cols: int, seed: int, d_range=(0.002, 0.02)) -> dict:
    g = rng(seed)
    nb = cols // 32
    d_bits = fp16_uniform_bits(g, (rows, nb), *d_range)
    q = g.integers(-127, 128, size=(rows, cols), dtype=np.int8)
    return {"d_bits": d_bits, "q": q}


def gen_q4_k(rows: int, cols: int, seed: int, d_range=(0.001, 0.01),
             dmin_range=(0.001, 0.01)) -> dict:
    g = rng(seed)
    nb = cols // 256
    d_bits = fp16_uniform_bits(g, (rows, nb), *d_range)
    dmin_bits = fp16_uniform_bits(g, (rows, nb), *dmin_range)
    sc = g.integers(0, 64, size=(rows, nb, 8), dtype=np.uint8)
    m = g.integers(0, 64, size=(rows, nb, 8), dtype=np.uint8)
    u = g.integers(0, 16, size=(rows, cols), dtype=np.uint8)
    return {"d_bits": d_bits, "dmin_bits": dmin_bits, "sc": sc, "m": m, "u": u}


def gen_q5_k(rows: int, cols: int, seed: int, d_range=(0.001, 0.01),
             dmin_range=(0.001, 0.01)) -> dict:
    g = rng(seed)
    nb = cols // 256
    d_bits = fp16_uniform_bits(g, (rows, nb), *d_range)
    dmin_bits = fp16_uniform_bits(g, (rows, nb), *dmin_range)
    sc = g.integers(0, 64, size=(rows, nb, 8), dtype=np.uint8)
    m = g.integers(0, 64, size=(rows, nb, 8), dtype=np.uint8)
    u = g.integers(0, 32, size=(rows, cols), dtype=np.uint8)
    return {"d_bits": d_bits, "dmin_bits": dmin_bits, "sc": sc, "m": m, "u": u}


def gen_q6_k(rows: int, cols: int, seed: int, d_range=(0.001, 0.01)) -> dict:
    g = rng(seed)
    nb = cols // 256
    d_bits = fp16_uniform_bits(g, (rows, nb), *d_range)
    sc = g.integers(-128, 128, size=(rows, nb, 16), dtype=np.int8)
    q = g.integers(0, 64, size=(rows, cols), dtype=np.uint8)
    return {"d_bits": d_bits, "sc": sc, "q": q}


def gen_int4_g128(rows: int, cols: int, seed: int, s_range=(0.005, 0.05)) -> dict:
    g = rng(seed)
    ng = cols // 128
    s_bits = fp16_uniform_bits(g, (rows, ng), *s_range)
    q = g.integers(-8, 8, size=(rows, cols), dtype=np.int8)
    return {"s_bits": s_bits, "q": q}


GENERATORS = {"q8_0": gen_q8_0, "q4_k": gen_q4_k, "q6_k": gen_q6_k,
              "int4_g128": gen_int4_g128, "q5_k": gen_q5_k}


def gen_weights(fmt: str, rows: int, cols: int, seed: int, **kw) -> dict:
    return GENERATORS[fmt](rows, cols, seed, **kw)


def gen_x(batch: int, cols: int, dtype: str, seed: int) -> np.ndarray:
    """Activations [batch, cols] ~ N(0, 1).

    dtype "f32" -> float32, "f16" -> float16, "bf16" -> uint16 bf16 bit patterns.
    """
    g = rng(seed)
    x = g.standard_normal(size=(batch, cols)).astype(np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    raise ValueError(f"unknown activation dtype {dtype!r}")


# ---------------------------------------------------------------------------
# Workload catalogue.  Each entry lists (name, rows, cols) matrices; the seed of
# matrix i is 1000 * config + i and the seed of its activation is
# 1000 * config + 100 + i.
# ---------------------------------------------------------------------------
HIDDEN, FFN, KV, VOCAB = 3584, 18944, 512, 152064

CONFIGS = {
    1: {"name": "q8_0_gemv_1536", "fmt": "q8_0", "x_dtype": "f32", "batch": [1],
        "mats": [("w", 1536, 1536)]},
    2: {"name": "int4_g128_ffn_7b", "fmt": "int4_g128", "x_dtype": "f16", "batch": [1],
        "mats": [("gate", FFN, HIDDEN), ("up", FFN, HIDDEN), ("down", HIDDEN, FFN)]},
    3: {"name": "q4_k_layer_7b", "fmt": "q4_k", "x_dtype": "f32", "batch": [1],
        "mats": [("q", HIDDEN, HIDDEN), ("k", KV, HIDDEN), ("v", KV, HIDDEN),
                 ("o", HIDDEN, HIDDEN), ("gate", FFN, HIDDEN), ("up", FFN, HIDDEN),
                 ("down", HIDDEN, FFN)]},
    4: {"name": "q6_k_lm_head_7b", "fmt": "q6_k", "x_dtype": "f32", "batch": [1],
        "mats": [("lm_head", VOCAB, HIDDEN)]},
    5: {"name": "q4_k_batched_ffn_7b", "fmt": "q4_k", "x_dtype": "bf16",
        "batch": [1, 4, 16, 64, 512], "mats": [("gate", FFN, HIDDEN)]},
    # Q5_K holds the expert-down projections of a Q4_K_M file (hipEngine 0.3.0,
    # "GGUF Support", payload table); the 7B down shape stands in for them.
    6: {"name": "q5_k_ffn_down_7b", "fmt": "q5_k", "x_dtype": "f32", "batch": [1],
        "mats": [("down", HIDDEN, FFN)]},
}


def weight_seed(config: int, index: int) -> int:
    return 1000 * config + index


def x_seed(config: int, index: int) -> int:
    return 1000 * config + 100 + index
