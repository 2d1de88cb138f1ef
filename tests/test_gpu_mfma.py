"""Batched Q4_K x bf16 on the matrix-core path, and Q4_K x fp16 on its
streaming kernel (5-16 rows with X in LDS) and tile kernels (17 rows up);
with a caller workspace, from 65 rows (17 against 8192 columns and more)
against 256 weight rows and more, the register-dequantized kernels (fp16
weight fragments formed per wave, activations converted once; every form
the launcher picks, with K whole or in slices).  Calls through the test
helper pass the workspace the library asks for; shapes the register path
would take also run as plain calls (no workspace: the tile kernels).

Gate: normwise relative error <= 2e-3 per batch row against the float64 oracle.
The matrix cores take the 4-bit codes and the activations exactly and the
sub-block scales are applied in fp32, so results are not bitwise those of the
fp32 GEMV; inputs whose products and sums are small integers are exact on both
paths and are checked exactly.  Shapes cover the three kernels behind the call
(batch <= 16 with X in LDS: one to eight 16-row tiles per workgroup and more
workgroups than CUs; batch <= 32 or K too long for LDS: K split over waves;
larger batches: 64 x 64 tiles; the register-dequantized kernels),
ragged rows and batches, the smallest batch routed here (2: matrices wider
than eight waves along K; narrower ones take the multi-row GEMV at batch 2,
and at 3-4 those within one wave's K slice), and the full-size batched
workload (18944 x 3584 at M = 4, 16, 64, 256 and 512, and 3584 x 18944 at
M = 512) on sampled rows.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from block_quantized_weight_qmv_amd import qmv
from gpu_util import DEV, Weights, gemv_ws, oracle_y, say, to_dev_x
from synth import CONFIGS, gen_weights, gen_x, weight_seed, x_seed

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from bench import dqreg_plan as bench_plan  # noqa: E402  (the form named in the test output)

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.mark.parametrize("rows,nblk,batch", [(64, 1, 64), (67, 14, 64), (130, 3, 65), (33, 5, 100),
                                             (200, 14, 128), (1, 2, 64), (70, 3, 3), (67, 5, 4),
                                             (96, 2, 16), (65, 3, 17), (40, 2, 32), (33, 4, 33),
                                             (17, 74, 8), (300, 9, 24), (1, 1, 3), (16, 1, 31),
                                             (4100, 2, 5), (40000, 1, 9), (3, 16, 16), (33, 17, 12),
                                             (70, 3, 2), (4100, 2, 2), (1, 1, 2), (17, 74, 2), (5, 130, 2),
                                             (300, 3, 130), (257, 2, 256), (1, 1, 128), (520, 5, 300),
                                             (256, 14, 129), (33, 74, 200), (300, 3, 384), (257, 2, 400),
                                             (520, 5, 390), (256, 14, 385), (1, 3, 400),
                                             # per-wave register fragments, 2..5 tiles per wave
                                             (10000, 1, 300), (10001, 3, 300), (18944, 1, 640), (18950, 2, 630),
                                             (30000, 1, 512), (30001, 1, 500), (18944, 2, 512), (18900, 3, 509),
                                             # LDS-shared tiles (grids of half to all compute units)
                                             (4100, 1, 1000), (8200, 2, 520), (6000, 3, 700), (4099, 2, 1000)])
def test_mfma_matches_oracle(rows, nblk, batch):
    cols = nblk * 256
    say(f"mfma q4_k {rows}x{cols} batch {batch}")
    w = Weights("q4_k", rows, cols, seed=700 + rows + nblk)
    x = gen_x(batch, cols, "bf16", seed=71 + batch)
    y = torch.full((batch, rows), 3.5, dtype=torch.float32, device=DEV)
    xd = to_dev_x(x, "bf16")
    w.gemv(xd, "bf16", batch, y=y)
    y = y.cpu().numpy()
    y64 = oracle_y(w, x, "bf16")
    err = oracle.normwise_rel_err(y, y64)
    say(f"  normwise err max {err.max():.3e}")
    assert np.all(err <= TOL), err
    if qmv.qmv_workspace_size("q4_k", "bf16", batch, [(w.desc, xd, y)]):
        # with a workspace this took the register-dequantized kernels; the
        # plain call takes the exact-product tile kernels
        err = oracle.normwise_rel_err(w.gemv(xd, "bf16", batch, ws=False).cpu().numpy(), y64)
        say(f"  plain call: normwise err max {err.max():.3e}")
        assert np.all(err <= TOL), err


# One shape per form of the register-dequantized kernels the launcher's model
# picks (T tiles per wave, 64 or 128 activation rows per workgroup, K whole
# or in slices summed afterwards), ragged where the form allows.
DQREG_FORMS = [(256, 5, 128), (520, 14, 512), (4100, 1, 200), (520, 14, 384), (8200, 1, 200), (520, 14, 768),
               (24000, 1, 200), (4100, 14, 256), (3000, 14, 160), (4100, 14, 200), (6000, 20, 160),
               (24000, 1, 300), (3001, 14, 161), (4099, 14, 201), (257, 5, 129)]


@pytest.mark.parametrize("rows,nblk,batch", DQREG_FORMS)
def test_dqreg_forms_match_oracle(rows, nblk, batch):
    cols = nblk * 256
    say(f"dqreg form {bench_plan(rows, cols, batch)} q4_k {rows}x{cols} batch {batch}")
    w = Weights("q4_k", rows, cols, seed=2100 + rows + nblk)
    x = gen_x(batch, cols, "bf16", seed=210 + batch)
    y = torch.full((batch, rows), 3.5, dtype=torch.float32, device=DEV)
    w.gemv(to_dev_x(x, "bf16"), "bf16", batch, y=y)
    err = oracle.normwise_rel_err(y.cpu().numpy(), oracle_y(w, x, "bf16"))
    say(f"  normwise err max {err.max():.3e}")
    assert np.all(err <= TOL), err


@pytest.mark.parametrize("rows,batch", [(96, 64), (96, 128), (300, 384), (300, 400), (4100, 1000)])
def test_mfma_integer_case_is_exact(rows, batch):
    # d = dmin = 1 and x in {-1, 0, 1}: every product and partial sum is an
    # integer below 2^24, so the fp32 result is exact on any summation order
    # (on the register-dequantized kernels the fp16 weights sc u - m are
    # exact integers too, and the power-of-two activation scale is exact).
    cols = 4 * 256
    f = gen_weights("q4_k", rows, cols, 5)
    f["d_bits"][:] = 0x3C00
    f["dmin_bits"][:] = 0x3C00
    w = Weights("q4_k", rows, cols, fields=f)
    g = np.random.Generator(np.random.PCG64(9))
    xf = g.integers(-1, 2, size=(batch, cols)).astype(np.float32)
    x = (xf.view(np.uint32) >> 16).astype(np.uint16)
    y = w.gemv(to_dev_x(x, "bf16"), "bf16", batch).cpu().numpy()
    y64 = oracle_y(w, x, "bf16")
    assert np.abs(y64).max() < 2 ** 24
    np.testing.assert_array_equal(y, y64.astype(np.float32))


@pytest.mark.parametrize("batch", [16, 64])
def test_mfma_deterministic_and_graph_replay(batch):
    rows, cols = 256, 14 * 256
    w = Weights("q4_k", rows, cols, seed=11)
    x = to_dev_x(gen_x(batch, cols, "bf16", seed=12), "bf16")
    y1 = w.gemv(x, "bf16", batch)
    y2 = w.gemv(x, "bf16", batch)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    s = torch.cuda.Stream()
    yg = torch.zeros_like(y1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            w.gemv(x, "bf16", batch, y=yg, stream=s)
    for _ in range(3):
        yg.fill_(-2.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y1)


@pytest.mark.parametrize("config,mat,batch", [(5, 0, 4), (5, 0, 16), (5, 0, 64), (5, 0, 256), (5, 0, 512),
                                              (3, 6, 512)])
def test_full_size_batched_ffn_sampled_rows(config, mat, batch):
    # the 7B FFN's gate (18944 x 3584) and down (3584 x 18944) matrices
    _, rows, cols = CONFIGS[config]["mats"][mat]
    say(f"full-size mfma {rows}x{cols} batch {batch}")
    w = Weights("q4_k", rows, cols, seed=weight_seed(config, mat))
    x = gen_x(batch, cols, "bf16", x_seed(config, 0))
    y = w.gemv(to_dev_x(x, "bf16"), "bf16", batch).cpu().numpy()
    g = np.random.Generator(np.random.PCG64(batch))
    ids = np.sort(g.choice(rows, size=48, replace=False))
    ids[0], ids[-1] = 0, rows - 1
    y64 = oracle_y(w, x, "bf16", ids)
    err = oracle.normwise_rel_err(y[:, ids], y64)
    say(f"  sampled normwise err max {err.max():.3e}")
    assert np.all(err <= TOL)
    assert np.all(np.isfinite(y))
    del w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layout", ["blocks", "planes"])
@pytest.mark.parametrize("rows,nblk,batch", [(67, 14, 5), (130, 3, 16), (1, 1, 8), (33, 16, 9), (200, 14, 12),
                                             (16, 2, 7), (40, 5, 17), (70, 3, 33), (33, 14, 64), (9, 2, 100),
                                             (17, 74, 20), (130, 3, 129), (33, 74, 5), (70, 20, 16), (5, 130, 9),
                                             (300, 3, 400), (257, 5, 390)])
def test_mfma_f16_matches_oracle(layout, rows, nblk, batch):
    # Q4_K x fp16 from 5 rows: the streaming kernel (5-16 rows, X in LDS),
    # the K-split kernel (5-16 rows, K > 4096) or the tile kernels (17 rows
    # up, any K; ragged batch tiles) with fp16 operands (codes as
    # fp16(1024 + u), exact; fp32 sums)
    cols = nblk * 256
    say(f"mfma fp16 q4_k {layout} {rows}x{cols} batch {batch}")
    w = Weights("q4_k", rows, cols, seed=900 + rows + nblk)
    desc = w.desc
    if layout == "planes":
        buf = torch.empty(qmv.qmv_planes_size("q4_k", rows, cols), dtype=torch.uint8, device=DEV)
        desc = qmv.qmv_repack_planes(w.desc, buf)
        desc.keep = buf
    x = gen_x(batch, cols, "f16", seed=91 + batch)
    y = torch.full((batch, rows), 3.5, dtype=torch.float32, device=DEV)
    xd = to_dev_x(x, "f16")
    qmv.qmv_gemv("q4_k", desc, xd, "f16", y, rows, cols, batch)
    y64 = oracle_y(w, x, "f16")
    err = oracle.normwise_rel_err(y.cpu().numpy(), y64)
    say(f"  normwise err max {err.max():.3e}")
    assert np.all(err <= TOL), err
    if qmv.qmv_workspace_size("q4_k", "f16", batch, [(desc, xd, y)]):
        # with a workspace: the register-dequantized kernels
        y.fill_(3.5)
        ws = gemv_ws("q4_k", [(desc, xd, y)], "f16", batch)
        err = oracle.normwise_rel_err(y.cpu().numpy(), y64)
        del ws
        say(f"  with a workspace: normwise err max {err.max():.3e}")
        assert np.all(err <= TOL), err


def test_mfma_f16_integer_case_is_exact():
    # d = dmin = 1 and x in {-1, 0, 1}: every product and partial sum is an
    # integer below 2^24, so the fp32 result is exact on any summation order
    rows, cols, batch = 96, 4 * 256, 12
    f = gen_weights("q4_k", rows, cols, 6)
    f["d_bits"][:] = 0x3C00
    f["dmin_bits"][:] = 0x3C00
    w = Weights("q4_k", rows, cols, fields=f)
    g = np.random.Generator(np.random.PCG64(10))
    x = g.integers(-1, 2, size=(batch, cols)).astype(np.float16)
    y = w.gemv(to_dev_x(x, "f16"), "f16", batch).cpu().numpy()
    y64 = oracle_y(w, x, "f16")
    assert np.abs(y64).max() < 2 ** 24
    np.testing.assert_array_equal(y, y64.astype(np.float32))


@pytest.mark.parametrize("batch", [5, 16, 64, 256, 512])
def test_full_size_f16_batched_ffn_sampled_rows(batch):
    cfg = CONFIGS[5]
    _, rows, cols = cfg["mats"][0]
    say(f"full-size mfma fp16 {rows}x{cols} batch {batch}")
    w = Weights("q4_k", rows, cols, seed=weight_seed(5, 0))
    x = gen_x(batch, cols, "f16", x_seed(5, 0))
    y = w.gemv(to_dev_x(x, "f16"), "f16", batch).cpu().numpy()
    g = np.random.Generator(np.random.PCG64(100 + batch))
    ids = np.sort(g.choice(rows, size=48, replace=False))
    ids[0], ids[-1] = 0, rows - 1
    err = oracle.normwise_rel_err(y[:, ids], oracle_y(w, x, "f16", ids))
    say(f"  sampled normwise err max {err.max():.3e}")
    assert np.all(err <= TOL)
    del w
    torch.cuda.empty_cache()


def test_mfma_f16_tile_graph_replay():
    # 40 fp16 rows on the tile kernel; a captured graph of the call must equal
    # the eager result on every replay
    rows, cols, batch = 300, 14 * 256, 40
    say("mfma fp16 tile graph replay")
    w = Weights("q4_k", rows, cols, seed=1900)
    x = to_dev_x(gen_x(batch, cols, "f16", seed=190), "f16")
    y0 = w.gemv(x, "f16", batch)
    s = torch.cuda.Stream()
    yg = torch.zeros(batch, rows, dtype=torch.float32, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        w.gemv(x, "f16", batch, y=yg, stream=s)  # warm-up outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            w.gemv(x, "f16", batch, y=yg, stream=s)
    for _ in range(3):
        yg.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y0)


@pytest.mark.parametrize("layout", ["blocks", "planes"])
@pytest.mark.parametrize("spread", ["wide", "large", "tiny", "rising", "falling", "zero_blocks"])
@pytest.mark.parametrize("rows,nblk,batch", [(300, 9, 400), (18944, 3, 512), (4100, 3, 1000)])
def test_dq_bf16_activation_range(layout, spread, rows, nblk, batch):
    """On the register-dequantized kernels the activations enter the matrix
    cores as fp16, each row scaled by the power of two that brings its
    largest |x| into [2^14, 2^15).  Rows far outside fp16's range, twelve
    decades within a row, magnitudes rising or falling by 2^20 per block
    along K, and all-zero blocks must all meet the gate, in forms with one to
    five tiles per wave and K whole or in slices."""
    cols = nblk * 256
    w = Weights("q4_k", rows, cols, seed=1300)
    g = np.random.Generator(np.random.PCG64({"wide": 1, "large": 2, "tiny": 3, "rising": 4, "falling": 5,
                                             "zero_blocks": 6}[spread]))
    x = g.standard_normal((batch, cols))
    blk = np.arange(cols) // 256
    if spread == "wide":
        x *= 10.0 ** g.uniform(-6, 6, size=x.shape)
    elif spread == "large":
        x *= 1e30
    elif spread == "tiny":
        x *= 1e-33
    elif spread == "rising":
        x *= 2.0 ** (20.0 * blk - 80.0)
    elif spread == "falling":
        x *= 2.0 ** (80.0 - 20.0 * blk)
    else:
        x[:, (blk % 3) == 1] = 0.0
        x[::7] = 0.0  # some rows all zero
    x = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # bf16 bit patterns
    desc = w.desc
    keep = None
    if layout == "planes":
        keep = torch.empty(qmv.qmv_planes_size("q4_k", rows, cols), dtype=torch.uint8, device=DEV)
        desc = qmv.qmv_repack_planes(w.desc, keep)
    say(f"dq bf16 activation range {spread} ({layout}) {rows}x{cols} batch {batch}")
    y = torch.full((batch, rows), 3.5, dtype=torch.float32, device=DEV)
    ws = gemv_ws("q4_k", [(desc, to_dev_x(x, "bf16"), y)], "bf16", batch)
    got = y.cpu().numpy()
    del ws
    assert np.all(np.isfinite(got))
    err = oracle.normwise_rel_err(got, oracle_y(w, x, "bf16"))
    say(f"  normwise err max {err.max():.3e}")
    assert np.all(err <= TOL), err


@pytest.mark.parametrize("x_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("rows,cols,batch", [(520, 6 * 256, 400), (4100, 2 * 256, 1000), (18944, 2 * 256, 512)])
def test_dq_deterministic_and_graph_replay(x_dtype, rows, cols, batch):
    # the register-dequantized kernels (K in slices, 64-row activation
    # tiles, five tiles per wave): bitwise equal on a second call and on
    # every replay of a captured graph
    say(f"dq {x_dtype} determinism and graph replay {rows}x{cols} batch {batch}")
    w = Weights("q4_k", rows, cols, seed=1400)
    x = to_dev_x(gen_x(batch, cols, x_dtype, seed=140), x_dtype)
    y0 = w.gemv(x, x_dtype, batch)
    assert torch.equal(w.gemv(x, x_dtype, batch), y0)
    s = torch.cuda.Stream()
    yg = torch.zeros(batch, rows, dtype=torch.float32, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        w.gemv(x, x_dtype, batch, y=yg, stream=s)  # warm-up outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            w.gemv(x, x_dtype, batch, y=yg, stream=s)
    for _ in range(3):
        yg.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y0)


def test_dqreg_caller_workspace():
    """The register-dequantized kernels run only with a workspace from the
    caller: qmv_workspace_size names its bytes, one byte fewer fails with
    QMV_ERR_SIZE before anything is launched (y keeps its values), no
    workspace gives the exact-product kernels of plain qmv_gemv (bit for
    bit), and a capture on a fresh stream needs no earlier call: every
    replay equals the eager result, also after a larger call has used
    another workspace."""
    rows, cols, batch = 3584, 14 * 256, 128
    w = Weights("q4_k", rows, cols, seed=2300)
    x = to_dev_x(gen_x(batch, cols, "bf16", seed=230), "bf16")
    y = torch.full((batch, rows), 7.0, dtype=torch.float32, device=DEV)
    items = [(w.desc, x, y)]
    n = qmv.qmv_workspace_size("q4_k", "bf16", batch, items)
    assert n >= cols * batch * 2 + rows * batch * 4
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    with pytest.raises(qmv.QmvError, match="workspace") as e:
        qmv.qmv_gemv_multi_ws("q4_k", "bf16", batch, items, ws, n - 1)
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
    plain = w.gemv(x, "bf16", batch, ws=False)
    qmv.qmv_gemv_multi_ws("q4_k", "bf16", batch, items, None, 0)
    assert torch.equal(y, plain)
    y0 = w.gemv(x, "bf16", batch)
    assert not torch.equal(y0, plain)  # fp16 weights on the register path
    s = torch.cuda.Stream()
    yg = torch.zeros(batch, rows, dtype=torch.float32, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            qmv.qmv_gemv_multi_ws("q4_k", "bf16", batch, [(w.desc, x, yg)], ws, n, stream=s)
    big = 512
    xb = to_dev_x(gen_x(big, cols, "bf16", seed=231), "bf16")
    yb = w.gemv(xb, "bf16", big)
    for _ in range(3):
        yg.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y0)
    err = oracle.normwise_rel_err(yb.cpu().numpy()[::37], oracle_y(w, gen_x(big, cols, "bf16", seed=231)[::37],
                                                                    "bf16"))
    assert np.all(err <= TOL), err
