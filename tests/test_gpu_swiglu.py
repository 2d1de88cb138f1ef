"""qmv_gemv_swiglu on the GPU: h = silu(W_gate x) * (W_up x) in one launch.

Each case is checked two ways: against the float64 oracle's SwiGLU chain
(normwise 2e-3 per activation row, the gate of the GEMVs), and against the
unfused chain on the GPU -- the batch-1 GEMVs of the gate and up matrices
(qmv_gemv_multi per activation row), combined as silu(g) * u in float64.
The fused launch computes each (g, u) pair with the GEMV's two-row tile
arithmetic, so it differs from that chain only in the rounding of its fp32
epilogue (hardware exp2 and reciprocal, three products): elementwise within
4e-6 relative plus 1e-6 of the row's largest |h| (the exponent's rounding
grows with |g| where g is very negative and h tiny, and fp32 exp overflows
where float64 still holds a subnormal-sized result).  INT4's batch-1 GEMV uses
one-row tiles, whose reduction order differs, so there the chain is
compared normwise within 1e-5.  Shapes: every format and layout, each
activation dtype, ragged row counts (a single row, rows past one tile set),
several activation rows, rows at the widest K slice, inputs that push
silu's argument far out on both sides, all-zero activation rows, graph
capture, and the 7B FFN's gate and up at full size.
"""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_weight_qmv_amd import qmv
from gpu_util import DEV, Weights, say, to_dev_x
from synth import CONFIGS, gen_x, weight_seed, x_seed

pytestmark = pytest.mark.gpu

TOL = 2e-3
CASES = [("q8_0", "blocks"), ("q4_k", "blocks"), ("q4_k", "planes"), ("q5_k", "blocks"), ("q5_k", "planes"),
         ("q6_k", "blocks"), ("q6_k", "planes"), ("int4_g128", "blocks")]
# (rows, K in units of one wave's slice / 8, batch): K from one block to the widest slice
SHAPES = [(1, 1, 1), (67, 3, 1), (130, 8, 2), (4100, 5, 1), (33, 8, 3), (300, 2, 5)]
SLICE = {"q8_0": 2048, "q4_k": 4096, "q5_k": 4096, "q6_k": 4096, "int4_g128": 4096}


def _cols(fmt, eighths):
    qk = oracle.QK[fmt]
    return max(qk, SLICE[fmt] * eighths // 8 // qk * qk)


def _desc(w, layout):
    if layout == "blocks":
        return w.desc, None
    buf = torch.empty(qmv.qmv_planes_size(w.fmt, w.rows, w.cols), dtype=torch.uint8, device=DEV)
    return qmv.qmv_repack_planes(w.desc, buf), buf


def _chain(fmt, dg, du, xd, x_dtype, rows, batch):
    """The unfused chain on the GPU: batch-1 GEMVs of gate and up, then silu(g) * u in float64."""
    g = torch.empty(batch, rows, dtype=torch.float32, device=DEV)
    u = torch.empty_like(g)
    for b in range(batch):
        xb = xd[b:b + 1].clone()
        gb = torch.empty(1, rows, dtype=torch.float32, device=DEV)
        ub = torch.empty_like(gb)
        qmv.qmv_gemv_multi(fmt, x_dtype, 1, [(dg, xb, gb), (du, xb, ub)])
        g[b], u[b] = gb[0], ub[0]
    g, u = g.cpu().numpy().astype(np.float64), u.cpu().numpy().astype(np.float64)
    return oracle.silu64(g) * u


def _check(fmt, h, h64, hc):
    err = oracle.normwise_rel_err(h, h64)
    say(f"  oracle normwise err max {err.max():.3e}")
    assert np.all(err <= TOL), err
    if fmt == "int4_g128":
        apart = oracle.normwise_rel_err(h, hc)
        assert np.all(apart <= 1e-5), apart
    else:
        scale = np.max(np.abs(hc), axis=-1, keepdims=True)
        assert np.all(np.abs(h - hc) <= 4e-6 * np.abs(hc) + 1e-6 * scale)


@pytest.mark.parametrize("x_dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("rows,eighths,batch", SHAPES)
@pytest.mark.parametrize("fmt,layout", CASES)
def test_swiglu_matches_oracle_and_unfused_chain(fmt, layout, rows, eighths, batch, x_dtype):
    cols = _cols(fmt, eighths)
    say(f"swiglu {fmt} {layout} {rows}x{cols} batch {batch} x {x_dtype}")
    wg = Weights(fmt, rows, cols, seed=3100 + rows + eighths)
    wu = Weights(fmt, rows, cols, seed=3200 + rows + eighths)
    dg, kg = _desc(wg, layout)
    du, ku = _desc(wu, layout)
    x = gen_x(batch, cols, x_dtype, seed=310 + batch)
    xd = to_dev_x(x, x_dtype)
    h = torch.full((batch, rows), 9.0, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv_swiglu(fmt, dg, du, xd, x_dtype, h, rows, cols, batch)
    got = h.cpu().numpy()
    h64 = oracle.swiglu64(fmt, wg.oracle_bytes(), wu.oracle_bytes(), rows, cols, x, x_dtype)
    _check(fmt, got, h64, _chain(fmt, dg, du, xd, x_dtype, rows, batch))
    del kg, ku


@pytest.mark.parametrize("fmt", ["q4_k", "int4_g128"])
def test_swiglu_far_arguments_and_zero_rows(fmt):
    """Activation rows scaled so silu's argument reaches +-1e3 (silu(g) = g
    and -0 in fp32) and an all-zero row (h = 0 exactly)."""
    rows, cols = 260, _cols(fmt, 8)
    wg = Weights(fmt, rows, cols, seed=3300)
    wu = Weights(fmt, rows, cols, seed=3301)
    x_dtype = "f32"
    x = gen_x(4, cols, x_dtype, seed=330)
    x[1] *= 300.0
    x[2] *= -300.0
    x[3] = 0.0
    xd = to_dev_x(x, x_dtype)
    h = torch.full((4, rows), 9.0, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv_swiglu(fmt, wg.desc, wu.desc, xd, x_dtype, h, rows, cols, 4)
    got = h.cpu().numpy()
    assert np.all(np.isfinite(got)) and np.all(got[3] == 0.0)
    h64 = oracle.swiglu64(fmt, wg.oracle_bytes(), wu.oracle_bytes(), rows, cols, x, x_dtype)
    g64 = oracle.gemv64(fmt, wg.oracle_bytes(), rows, cols, x, x_dtype)
    say(f"swiglu far arguments {fmt}: |g| up to {np.abs(g64).max():.1f}")
    assert np.abs(g64[1:3]).max() > 100.0
    _check(fmt, got, h64, _chain(fmt, wg.desc, wu.desc, xd, x_dtype, rows, 4))


def test_swiglu_graph_replay():
    rows, cols = 1000, 14 * 256
    wg = Weights("q4_k", rows, cols, seed=3400)
    wu = Weights("q4_k", rows, cols, seed=3401)
    xd = to_dev_x(gen_x(1, cols, "f32", seed=340), "f32")
    h0 = torch.empty(1, rows, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv_swiglu("q4_k", wg.desc, wu.desc, xd, "f32", h0, rows, cols, 1)
    s = torch.cuda.Stream()
    hg = torch.zeros_like(h0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            qmv.qmv_gemv_swiglu("q4_k", wg.desc, wu.desc, xd, "f32", hg, rows, cols, 1, stream=s)
    for _ in range(3):
        hg.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(hg, h0)


@pytest.mark.parametrize("config", [3, 2])
def test_swiglu_full_size_ffn(config):
    """The 7B FFN's gate and up matrices (18944 x 3584; Q4_K in planes with
    fp32 activations, INT4 with fp16), every output against the oracle."""
    cfg = CONFIGS[config]
    names = [n for n, _, _ in cfg["mats"]]
    gi, ui = names.index("gate"), names.index("up")
    _, rows, cols = cfg["mats"][gi]
    fmt, x_dtype = cfg["fmt"], cfg["x_dtype"]
    layout = "planes" if fmt == "q4_k" else "blocks"
    say(f"swiglu full size {fmt} {layout} {rows}x{cols} x {x_dtype}")
    wg = Weights(fmt, rows, cols, seed=weight_seed(config, gi))
    wu = Weights(fmt, rows, cols, seed=weight_seed(config, ui))
    dg, kg = _desc(wg, layout)
    du, ku = _desc(wu, layout)
    x = gen_x(1, cols, x_dtype, x_seed(config, gi))
    xd = to_dev_x(x, x_dtype)
    h = torch.full((1, rows), 9.0, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv_swiglu(fmt, dg, du, xd, x_dtype, h, rows, cols, 1)
    got = h.cpu().numpy()
    h64 = oracle.swiglu64(fmt, wg.oracle_bytes(), wu.oracle_bytes(), rows, cols, x, x_dtype)
    _check(fmt, got, h64, _chain(fmt, dg, du, xd, x_dtype, rows, 1))
    del kg, ku
