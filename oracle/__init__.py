"""CPU oracle for block-quantized weight dequantization and GEMV.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or run anything under this directory.  The only permitted users are the test
suite (``tests/``), the ``smoke()`` check in ``__graft_entry__.py`` and the
``cpu_baseline`` leg of ``bench.py``.

What it computes, and from which passage:

* VTE (kyuubyn.github.io/VTE), feature list: the engine dequantizes Q4_K, Q6_K
  and Q8_0 byte for byte in llama.cpp's reference block layout and checks each
  layer against NumPy.  The oracle is that NumPy decoder: a bit-level reader of
  each block layout, producing the exact value of every weight in float64.
* "Costruire un runtime di inference LLM da zero" (datastack.it), closing
  paragraph of "Tre bug che insegnano": weights are symmetric INT4 with one
  scale per group of 128.  The group-128 plane layout is this library's own
  reading (planar codes then planar fp16 scales, offset-binary nibbles).
* LLM170 README, testing bullets, and hipEngine 0.3.0, "Core principles": a CPU
  reference is the correctness gate for every GPU kernel; fused kernels are
  checked against an unfused chain.  The oracle's GEMV is the unfused chain:
  dequantize to float64, then a float64 matrix-vector product.
* hipfire, Qwen2 decoder "Key Technical Specifications": the FFN is SwiGLU.
  The oracle's SwiGLU input h = silu(W_gate x) * (W_up x) is that unfused
  chain again: two float64 GEMVs, then silu(g) = g / (1 + exp(-g)) times u.

Everything is plain numpy in float64.  The decoders are deliberately
unblocked and unfused so they can be checked against the layout tables by eye.

Pins (what ties the oracle to something other than itself) live in
``tests/test_oracle_*.py`` and ``tests/golden/``: hand-computed blocks,
fp16/bf16 decoding against IEEE-754 definitions and numpy, closed forms
(single rounding, e_k columns), invariants (zero scale, affine in the code),
brute force with exact rational arithmetic, and planted-mistake checks.
GGUF byte compatibility with real llama.cpp files is *parity unpinned*: no
GGUF file, llama.cpp build or gguf package is available to compare against.
"""
from .formats import (BLOCK_BYTES, FORMATS, QK, dequant32, dequant64, pack,
                      packed_size, row_slice, unpack)
from .fp import bf16_bits_to_f64, f32_to_bf16_bits_rne, fp16_bits_to_f64
from .gemv import (elementwise_bound, elementwise_bound_rows, gamma, gemv64, gemv64_and_bound,
                   gemv64_rows,
                   normwise_rel_err, silu64, swiglu64, x_to_f64)

__all__ = [
    "BLOCK_BYTES", "FORMATS", "QK", "dequant32", "dequant64", "pack", "packed_size",
    "row_slice", "unpack", "bf16_bits_to_f64", "f32_to_bf16_bits_rne",
    "fp16_bits_to_f64", "elementwise_bound", "elementwise_bound_rows", "gamma", "gemv64",
    "gemv64_and_bound",
    "gemv64_rows",
    "normwise_rel_err", "silu64", "swiglu64", "x_to_f64",
]
