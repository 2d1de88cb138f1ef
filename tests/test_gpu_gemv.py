"""qmv_gemv on the GPU against the float64 oracle.

The gate is the contract's: normwise relative error <= 2e-3 per batch row
(max_r |y - y64| / max_r |y64|).  Cases whose float32 result is unique are
checked exactly: x = e_k returns column k of the float32 weights, integer
inputs give integer outputs, scaling x by 2 scales y by 2 bitwise, and two
runs agree bitwise.
"""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_weight_qmv_amd import qmv
from gpu_util import DEV, Weights, oracle_y, say, to_dev_x
from synth import CONFIGS, gen_weights, gen_x, weight_seed, x_seed

pytestmark = pytest.mark.gpu

TOL = 2e-3
FMTS = ("q8_0", "q4_k", "q6_k", "int4_g128", "q5_k")
# (rows, blocks per row): single block, ragged wave tiles, several waves along K
SHAPES = {
    "q8_0": [(1, 1), (5, 3), (67, 48), (33, 65), (9, 200)],
    "q4_k": [(1, 1), (5, 3), (67, 14), (33, 17), (9, 74)],
    "q6_k": [(1, 1), (5, 3), (67, 14), (33, 17), (9, 74)],
    "int4_g128": [(1, 1), (5, 3), (67, 28), (33, 33), (9, 148)],
    "q5_k": [(1, 1), (5, 3), (67, 14), (33, 17), (9, 74)],
}
CASES = [(f, r, n) for f in FMTS for (r, n) in SHAPES[f]]


def _err(y, y64):
    return oracle.normwise_rel_err(y, y64)


@pytest.mark.parametrize("fmt,rows,nblk", CASES)
@pytest.mark.parametrize("x_dtype", ["f32", "f16", "bf16"])
def test_gemv_matches_oracle(fmt, rows, nblk, x_dtype):
    cols = nblk * oracle.QK[fmt]
    batch = 3 if rows < 40 else 1
    say(f"gemv {fmt} {rows}x{cols} batch {batch} x {x_dtype}")
    w = Weights(fmt, rows, cols, seed=1234 + rows + nblk)
    x = gen_x(batch, cols, x_dtype, seed=55 + nblk)
    y = w.gemv(to_dev_x(x, x_dtype), x_dtype, batch).cpu().numpy()
    y64 = oracle_y(w, x, x_dtype)
    err = _err(y, y64)
    say(f"  normwise err {err.max():.3e}")
    assert np.all(err <= TOL), err


@pytest.mark.parametrize("fmt", FMTS)
def test_unit_vectors_extract_columns_exactly(fmt):
    rows, cols = 21, 17 * oracle.QK[fmt] if fmt != "q8_0" else 70 * 32
    w = Weights(fmt, rows, cols, seed=31)
    ks = [0, 1, 31, 32, cols // 2 + 3, cols - 1]
    x = np.zeros((len(ks), cols), np.float32)
    for b, k in enumerate(ks):
        x[b, k] = 1.0
    say(f"e_k columns {fmt} {rows}x{cols}")
    y = w.gemv(to_dev_x(x, "f32"), "f32", len(ks)).cpu().numpy()
    w32 = oracle.dequant32(fmt, w.oracle_bytes(), rows, cols)
    for b, k in enumerate(ks):
        assert np.array_equal(y[b], w32[:, k]), (k, np.argwhere(y[b] != w32[:, k])[:4])


@pytest.mark.parametrize("fmt", FMTS)
def test_integer_case_is_exact(fmt):
    """Scales 1 and x in {-1, 0, 1}: every float32 partial sum is an exact integer."""
    rows, nblk = 40, {"q8_0": 70, "q4_k": 20, "q6_k": 20, "int4_g128": 40, "q5_k": 20}[fmt]
    cols = nblk * oracle.QK[fmt]
    f = gen_weights(fmt, rows, cols, 8)
    for k in ("d_bits", "dmin_bits", "s_bits"):
        if k in f:
            f[k][...] = 0x3C00
    w = Weights(fmt, rows, cols, fields=f)
    g = np.random.Generator(np.random.PCG64(4))
    x = g.integers(-1, 2, size=(2, cols)).astype(np.float32)
    y64 = oracle_y(w, x, "f32")
    w64 = oracle.dequant64(fmt, w.oracle_bytes(), rows, cols)
    assert np.all(np.abs(x) @ np.abs(w64).T < 2 ** 24)
    say(f"integer case {fmt}")
    y = w.gemv(to_dev_x(x, "f32"), "f32", 2).cpu().numpy()
    assert np.array_equal(y.astype(np.float64), y64)


@pytest.mark.parametrize("fmt", FMTS)
def test_scaling_x_by_two_and_determinism(fmt):
    rows, cols = 300, 14 * oracle.QK[fmt] if fmt != "q8_0" else 48 * 32
    w = Weights(fmt, rows, cols, seed=66)
    x = gen_x(1, cols, "f32", 67)
    say(f"2x / determinism {fmt}")
    y1 = w.gemv(to_dev_x(x, "f32"), "f32", 1).cpu().numpy()
    y1b = w.gemv(to_dev_x(x, "f32"), "f32", 1).cpu().numpy()
    y2 = w.gemv(to_dev_x(2 * x, "f32"), "f32", 1).cpu().numpy()
    assert np.array_equal(y1, y1b)
    assert np.array_equal(y2, 2 * y1)


@pytest.mark.parametrize("fmt", FMTS)
def test_output_canaries_untouched(fmt):
    rows, cols = 77, 3 * oracle.QK[fmt]
    w = Weights(fmt, rows, cols, seed=3)
    pad = 4
    # one contiguous [2][rows] window inside guard floats
    flat = torch.full((2 * rows + 2 * pad,), 12345.0, dtype=torch.float32, device=DEV)
    y = flat[pad:pad + 2 * rows]
    x = gen_x(2, cols, "f16", 9)
    say(f"canaries {fmt}")
    qmv.qmv_gemv(fmt, w.desc, to_dev_x(x, "f16"), "f16", y, rows, cols, 2)
    h = flat.cpu().numpy()
    assert np.all(h[:pad] == 12345.0) and np.all(h[pad + 2 * rows:] == 12345.0)
    assert np.all(_err(h[pad:pad + 2 * rows].reshape(2, rows), oracle_y(w, x, "f16")) <= TOL)


def test_graph_replay_matches_eager():
    """qmv_gemv captured in a HIP graph: every replay equals the eager result."""
    fmt, rows, cols = "q4_k", 512, 3584
    w = Weights(fmt, rows, cols, seed=12)
    x = to_dev_x(gen_x(1, cols, "f32", 13), "f32")
    y_eager = w.gemv(x, "f32", 1).clone()
    y = torch.empty(1, rows, dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph capture q4_k 512x3584")
    with torch.cuda.graph(g, stream=s):
        qmv.qmv_gemv(fmt, w.desc, x, "f32", y, rows, cols, 1, stream=s.cuda_stream)
    for i in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), i
        _ = (x * 2).sum().item()  # eager work between replays


# -- full-size workloads, sampled rows ----------------------------------------
def _sample_rows(rows, n=48, seed=0):
    g = np.random.Generator(np.random.PCG64(seed))
    ids = np.unique(np.concatenate([[0, 1, rows // 2, rows - 2, rows - 1],
                                    g.integers(0, rows, n)]))
    return ids


@pytest.mark.parametrize("config", [1, 2, 3, 4, 6])
def test_full_size_configs_sampled_rows(config):
    cfg = CONFIGS[config]
    for i, (name, rows, cols) in enumerate(cfg["mats"]):
        say(f"config {config} {cfg['fmt']} {name} {rows}x{cols} x {cfg['x_dtype']}")
        w = Weights(cfg["fmt"], rows, cols, seed=weight_seed(config, i))
        x = gen_x(1, cols, cfg["x_dtype"], x_seed(config, i))
        y = w.gemv(to_dev_x(x, cfg["x_dtype"]), cfg["x_dtype"], 1).cpu().numpy()
        ids = _sample_rows(rows, seed=config * 10 + i)
        y64 = oracle_y(w, x, cfg["x_dtype"], ids)
        # normwise over the sampled rows, scaled by the sampled maximum
        err = _err(y[:, ids], y64)
        say(f"  sampled normwise err {err.max():.3e}")
        assert np.all(err <= TOL)
        assert np.all(np.isfinite(y))
        del w
        torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt,layout", [("q4_k", "blocks"), ("q4_k", "planes"), ("q5_k", "blocks"),
                                        ("int4_g128", "blocks"), ("q8_0", "blocks"),
                                        ("q6_k", "blocks"), ("q6_k", "planes")])
@pytest.mark.parametrize("spread", ["wide", "large", "tiny"])
def test_bf16_activation_range(fmt, layout, spread):
    """Every format takes bf16 activations as fp16 after scaling each lane's
    activations by a power of two of their own: magnitudes far outside fp16's
    range (and a spread of twelve decades within one row) must still meet the
    gate."""
    rows, cols = 96, 17 * 256
    w = Weights(fmt, rows, cols, seed=808)
    g = np.random.Generator(np.random.PCG64({"wide": 1, "large": 2, "tiny": 3}[spread]))
    x = g.standard_normal((1, cols))
    if spread == "wide":
        x *= 10.0 ** g.uniform(-6, 6, size=x.shape)
    elif spread == "large":
        x *= 1e20
    else:
        x *= 1e-30
    x = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # bf16 bit patterns
    desc = w.desc
    if layout == "planes":
        dst = torch.empty(qmv.qmv_planes_size(fmt, rows, cols), dtype=torch.uint8, device=DEV)
        desc = qmv.qmv_repack_planes(w.desc, dst)
    say(f"{fmt} bf16 activation range {spread} ({layout})")
    y = torch.empty(1, rows, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv(fmt, desc, to_dev_x(x, "bf16"), "bf16", y, rows, cols, 1)
    got = y.cpu().numpy()
    assert np.all(np.isfinite(got))
    err = _err(got, oracle_y(w, x, "bf16"))
    say(f"  normwise err {err.max():.3e}")
    assert np.all(err <= TOL), err


@pytest.mark.parametrize("fmt,layout", [("q4_k", "blocks"), ("q4_k", "planes"), ("q5_k", "blocks"),
                                        ("int4_g128", "blocks"), ("q8_0", "blocks"),
                                        ("q6_k", "blocks"), ("q6_k", "planes")])
@pytest.mark.parametrize("spread", ["wide", "large", "tiny", "tinier", "mixed"])
@pytest.mark.parametrize("batch", [1, 2])
def test_f32_activation_range(fmt, layout, spread, batch):
    """fp32 activations far from N(0, 1): twelve decades within one row, all
    near 1e20, 1e-30 or 1e-36 (products of codes and activations below
    float32's normal range unless the kernel rescales), and a row mixing
    1e-36 and 1e+20 in different lanes.  Every case must meet the gate, in the
    single-row GEMV and in the two-row pass."""
    rows, cols = 96, 17 * 256
    w = Weights(fmt, rows, cols, seed=809)
    g = np.random.Generator(np.random.PCG64({"wide": 11, "large": 12, "tiny": 13, "tinier": 14,
                                             "mixed": 15}[spread]))
    x = g.standard_normal((batch, cols))
    if spread == "wide":
        x *= 10.0 ** g.uniform(-6, 6, size=x.shape)
    elif spread == "large":
        x *= 1e20
    elif spread == "tiny":
        x *= 1e-30
    elif spread == "tinier":
        x *= 1e-36
    else:
        x *= np.where((np.arange(cols) // 512) % 2 == 0, 1e-36, 1e20)[None, :]
    x = x.astype(np.float32)
    desc = w.desc
    if layout == "planes":
        dst = torch.empty(qmv.qmv_planes_size(fmt, rows, cols), dtype=torch.uint8, device=DEV)
        desc = qmv.qmv_repack_planes(w.desc, dst)
    say(f"{fmt} f32 activation range {spread} ({layout}) batch {batch}")
    y = torch.empty(batch, rows, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv(fmt, desc, to_dev_x(x, "f32"), "f32", y, rows, cols, batch)
    got = y.cpu().numpy()
    assert np.all(np.isfinite(got))
    err = _err(got, oracle_y(w, x, "f32"))
    say(f"  normwise err {err.max():.3e}")
    assert np.all(err <= TOL), err


# longest rows a GEMV launch accepts (16 waves along K): the 1024-thread
# kernel, and a 10-wave split in between
LONG = [("q8_0", 16 * 64 * 32), ("q4_k", 16 * 16 * 256), ("q5_k", 10 * 16 * 256),
        ("q6_k", 16 * 16 * 256), ("int4_g128", 16 * 64 * 64)]


@pytest.mark.parametrize("fmt,cols", LONG)
@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("layout", ["blocks", "planes"])
def test_longest_rows(fmt, cols, x_dtype, layout):
    if layout == "planes" and fmt not in ("q4_k", "q5_k", "q6_k"):
        pytest.skip("no plane layout for this format")
    rows = 37
    say(f"longest rows {fmt} {rows}x{cols} x {x_dtype} {layout}")
    w = Weights(fmt, rows, cols, seed=515)
    desc = w.desc
    if layout == "planes":
        buf = torch.empty(qmv.qmv_planes_size(fmt, rows, cols), dtype=torch.uint8, device=DEV)
        desc = qmv.qmv_repack_planes(w.desc, buf)
    x = gen_x(1, cols, x_dtype, seed=516)
    y = torch.full((1, rows), 5.0, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv(fmt, desc, to_dev_x(x, x_dtype), x_dtype, y, rows, cols, 1)
    err = _err(y.cpu().numpy(), oracle_y(w, x, x_dtype))
    say(f"  normwise err {err.max():.3e}")
    assert np.all(err <= TOL), err
    if layout == "planes":
        assert torch.equal(y, w.gemv(to_dev_x(x, x_dtype), x_dtype, 1))
