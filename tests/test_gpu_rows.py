"""Every format with several activation rows: the multi-row GEMV.

qmv_gemv routes two or more activation rows (Q4_K x bf16: 2-4 rows; larger
bf16 batches take the matrix cores) against matrices within one wave's K
slice (4096 columns; Q8_0 2048) to a GEMV that reads W once per two or four
rows (fp32: two), and fp16/bf16 rows against matrices of two to eight waves
along K (Q4_K x bf16: two rows only) to its K-split form, W once per two
rows; fp32 rows against those run the GEMV once per row.  Each row's products and sums are the batch-1 GEMV's operations
in the same order and the wave reduction adds in the same order, so every
output row must equal the batch-1 GEMV of that activation row bit for bit,
and the float64 oracle within the 2e-3 normwise gate.  Shapes: one block,
ragged tiles, a full wave K slice, odd block counts (the widest of them take
the once-per-row route for Q8_0, which must agree as well); batches 2, 3 (a
partial group of four) and 4, and batches of several groups; every layout of
the format; several matrices in one launch, one of them wider than a wave's K
slice (routed as its own call); matrices of two to nine waves along K (the
K-split form, two rows per pass); graph replay; full-size shapes (Q4_K and
INT4 18944 x 3584, Q6_K 152064 x 3584, Q8_0 1536 x 1536 at M = 2, 3, 4; the
INT4, Q5_K and Q4_K down projections 3584 x 18944 at M = 2, 3), all rows
against the batch-1 GEMV, sampled rows against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_weight_qmv_amd import qmv
from gpu_util import DEV, Weights, oracle_y, say, to_dev_x
from synth import CONFIGS, gen_x, weight_seed, x_seed

pytestmark = pytest.mark.gpu

TOL = 2e-3
FMTS = ["q4_k", "q6_k", "int4_g128", "q5_k", "q8_0"]
LAYOUTS = {"q4_k": ["blocks", "planes"], "q6_k": ["blocks", "planes"], "int4_g128": ["blocks"],
           "q5_k": ["blocks", "planes"], "q8_0": ["blocks"]}
FMT_LAYOUTS = [(f, lay) for f in FMTS for lay in LAYOUTS[f]]
SHAPES = [(1, 1), (3, 1), (5, 3), (67, 14), (9, 16), (40, 5), (130, 2)]


def _planes(w: Weights):
    buf = torch.empty(qmv.qmv_planes_size(w.fmt, w.rows, w.cols), dtype=torch.uint8, device=DEV)
    desc = qmv.qmv_repack_planes(w.desc, buf)
    desc.keep = buf
    return desc


def _desc(w: Weights, layout):
    return w.desc if layout == "blocks" else _planes(w)


def _per_row(fmt, desc, rows, cols, xd, x_dtype, batch):
    """The batch-1 GEMV of each activation row."""
    out = []
    for i in range(batch):
        y = torch.empty(1, rows, dtype=torch.float32, device=DEV)  # own buffer: 16-byte aligned
        qmv.qmv_gemv(fmt, desc, xd[i:i + 1].clone(), x_dtype, y, rows, cols, 1)
        out.append(y)
    return torch.cat(out)


def _check(fmt, layout, rows, cols, batch, x_dtype, seed):
    w = Weights(fmt, rows, cols, seed=seed)
    desc = _desc(w, layout)
    x = gen_x(batch, cols, x_dtype, seed=seed + 7)
    xd = to_dev_x(x, x_dtype)
    # one row past the batch: must stay untouched
    y = torch.full((batch + 1, rows), 7.25, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv(fmt, desc, xd, x_dtype, y, rows, cols, batch)
    got = y.cpu().numpy()
    assert np.all(got[batch] == 7.25)
    np.testing.assert_array_equal(got[:batch], _per_row(fmt, desc, rows, cols, xd, x_dtype, batch).cpu().numpy())
    err = oracle.normwise_rel_err(got[:batch], oracle_y(w, x, x_dtype))
    say(f"  normwise err max {err.max():.3e}")
    assert np.all(err <= TOL), err


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS)
@pytest.mark.parametrize("x_dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("batch", [2, 3, 4])
@pytest.mark.parametrize("rows,nblk", SHAPES)
def test_rows_equal_batch1_and_oracle(fmt, layout, x_dtype, batch, rows, nblk):
    cols = nblk * 256
    say(f"multi-row {fmt} {layout} {rows}x{cols} batch {batch} x {x_dtype}")
    _check(fmt, layout, rows, cols, batch, x_dtype, seed=1300 + rows + nblk)


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS)
@pytest.mark.parametrize("x_dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("batch", [5, 8, 9, 30])
@pytest.mark.parametrize("rows,nblk", [(3, 1), (67, 14), (130, 2)])
def test_rows_groups_of_four(fmt, layout, x_dtype, batch, rows, nblk):
    # batches above four: one pass over W per group of four rows (fp32: two),
    # the last group partial unless the group size divides the batch (Q4_K x
    # bf16 batches above four take the matrix cores and are not this kernel's)
    if fmt == "q4_k" and x_dtype == "bf16":
        pytest.skip("Q4_K x bf16 batches above four run on the matrix cores (test_gpu_mfma.py)")
    if fmt == "q4_k" and x_dtype == "f16":
        pytest.skip("Q4_K x fp16 batches from 5 rows run on the matrix cores (test_gpu_mfma.py)")
    cols = nblk * 256
    say(f"multi-row {fmt} {layout} {rows}x{cols} batch {batch} x {x_dtype}")
    _check(fmt, layout, rows, cols, batch, x_dtype, seed=1600 + rows + nblk)


# (rows, 256-column blocks): two, three, five and nine waves along K for the
# 4096-column formats (Q8_0, 2048 columns per wave: three, five and ten; its
# widest shape is above its limit); more than eight waves take the
# once-per-row route, which must agree as well
SPLIT_SHAPES = [(67, 20), (9, 40), (33, 74), (5, 130)]


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS)
@pytest.mark.parametrize("x_dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("batch", [2, 3, 5])
@pytest.mark.parametrize("rows,nblk", SPLIT_SHAPES)
def test_rows_split_k_equal_batch1_and_oracle(fmt, layout, x_dtype, batch, rows, nblk):
    # matrices wider than a wave's K slice: the K-split form, two activation
    # rows per pass (odd batches end in a half-used pass)
    cols = nblk * 256
    if fmt == "q4_k" and x_dtype == "f16" and batch >= 5:
        pytest.skip("Q4_K x fp16 from 5 rows runs on the matrix cores (test_gpu_mfma.py)")
    if fmt == "q4_k" and x_dtype == "bf16" and (batch > 2 or cols > 8 * 4096):
        pytest.skip("Q4_K x bf16 of wide matrices above two rows, or above eight waves along K, "
                    "runs on the matrix cores (test_gpu_mfma.py)")
    if fmt == "q8_0" and cols > 16 * 2048:
        pytest.skip("above the Q8_0 GEMV's 32768-column limit")
    say(f"multi-row split-K {fmt} {layout} {rows}x{cols} batch {batch} x {x_dtype}")
    _check(fmt, layout, rows, cols, batch, x_dtype, seed=1700 + rows + nblk)


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS)
@pytest.mark.parametrize("batch", [2, 4])
def test_rows_multi_matrix_launch(fmt, layout, batch):
    # q, k, v-shaped matrices (scaled down) and one wider than a wave's K
    # slice in one launch, each with its own x; every item must equal its own
    # call's result bitwise
    shapes = [(96, 14), (16, 14), (16, 14), (33, 3), (9, 20)]
    say(f"multi-row multi-matrix {fmt} {layout} batch {batch}")
    ws, descs, xs, ys, items = [], [], [], [], []
    for i, (rows, nblk) in enumerate(shapes):
        w = Weights(fmt, rows, nblk * 256, seed=1400 + i)
        d = _desc(w, layout)
        x = gen_x(batch, nblk * 256, "bf16", seed=140 + i)
        ws.append(w)
        descs.append(d)
        xs.append((x, to_dev_x(x, "bf16")))
        ys.append(torch.full((batch, rows), -1.0, dtype=torch.float32, device=DEV))
        items.append((d, xs[-1][1], ys[-1]))
    qmv.qmv_gemv_multi(fmt, "bf16", batch, items)
    for w, d, (x, xd), y in zip(ws, descs, xs, ys):
        got = y.cpu().numpy()
        alone = torch.empty(batch, w.rows, dtype=torch.float32, device=DEV)
        qmv.qmv_gemv(fmt, d, xd, "bf16", alone, w.rows, w.cols, batch)
        np.testing.assert_array_equal(got, alone.cpu().numpy())
        if not (fmt == "q4_k" and w.cols > 4096 and batch > 2):  # Q4_K x bf16 wide, M > 2: matrix cores
            ref = _per_row(fmt, d, w.rows, w.cols, xd, "bf16", batch).cpu().numpy()
            np.testing.assert_array_equal(got, ref)
        assert np.all(oracle.normwise_rel_err(got, oracle_y(w, x, "bf16")) <= TOL)


@pytest.mark.parametrize("fmt", FMTS)
def test_rows_graph_replay(fmt):
    rows, cols, batch = 300, 14 * 256, 4
    say(f"multi-row graph replay {fmt}")
    w = Weights(fmt, rows, cols, seed=1500)
    xd = to_dev_x(gen_x(batch, cols, "bf16", seed=150), "bf16")
    y0 = w.gemv(xd, "bf16", batch)
    s = torch.cuda.Stream()
    yg = torch.zeros(batch, rows, dtype=torch.float32, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        w.gemv(xd, "bf16", batch, y=yg, stream=s)  # warm-up outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            w.gemv(xd, "bf16", batch, y=yg, stream=s)
    for _ in range(3):
        yg.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y0)


# full-size shapes: the Q4_K FFN gate (bf16 and fp32 x), the INT4 FFN gate (fp16
# x), the Q6_K lm-head (bf16 and fp32 x), the Q8_0 1536 x 1536 matrix (fp16 x)
FULL = [("q4_k", 5, "bf16", "blocks"), ("q4_k", 5, "bf16", "planes"), ("int4_g128", 2, "f16", "blocks"),
        ("q6_k", 4, "bf16", "planes"), ("q8_0", 1, "f16", "blocks"), ("q4_k", 5, "f32", "planes"),
        ("q6_k", 4, "f32", "planes")]


# the down projections (3584 x 18944, five waves along K): INT4 (fp16 x), Q5_K
# (bf16 x), Q4_K (fp16 x); matrix index into the configuration's list
FULL_SPLIT = [("int4_g128", 2, "f16", "blocks", 2), ("q5_k", 6, "bf16", "planes", 0),
              ("q4_k", 3, "f16", "planes", 6), ("q4_k", 3, "bf16", "planes", 6)]


@pytest.mark.parametrize("fmt,config,x_dtype,layout", FULL)
@pytest.mark.parametrize("batch", [2, 3, 4])
def test_rows_full_size(fmt, config, x_dtype, layout, batch):
    _full_size(fmt, config, x_dtype, layout, batch, 0)


@pytest.mark.parametrize("fmt,config,x_dtype,layout,mat", FULL_SPLIT)
@pytest.mark.parametrize("batch", [2, 3])
def test_rows_split_k_full_size(fmt, config, x_dtype, layout, mat, batch):
    if fmt == "q4_k" and x_dtype == "bf16" and batch > 2:
        pytest.skip("Q4_K x bf16 above two rows: the matrix cores (test_gpu_mfma.py)")
    _full_size(fmt, config, x_dtype, layout, batch, mat)


def _full_size(fmt, config, x_dtype, layout, batch, mat):
    cfg = CONFIGS[config]
    rows, cols = cfg["mats"][mat][1], cfg["mats"][mat][2]
    say(f"full-size multi-row {fmt} {layout} {rows}x{cols} batch {batch} x {x_dtype}")
    w = Weights(fmt, rows, cols, seed=weight_seed(config, mat))
    desc = _desc(w, layout)
    x = gen_x(batch, cols, x_dtype, x_seed(config, mat))
    xd = to_dev_x(x, x_dtype)
    y = torch.empty(batch, rows, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv(fmt, desc, xd, x_dtype, y, rows, cols, batch)
    got = y.cpu().numpy()
    np.testing.assert_array_equal(got, _per_row(fmt, desc, rows, cols, xd, x_dtype, batch).cpu().numpy())
    g = np.random.Generator(np.random.PCG64(40 + batch))
    ids = np.sort(g.choice(rows, size=48, replace=False))
    ids = np.unique(np.concatenate([ids, [0, rows - 1]]))
    ref = oracle_y(w, x, x_dtype, row_ids=ids)
    err = oracle.normwise_rel_err(got[:, ids], ref)
    say(f"  sampled normwise err max {err.max():.3e}")
    assert np.all(err <= TOL), err
    del w, desc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["q4_k", "int4_g128"])
@pytest.mark.parametrize("x_dtype,batch", [("f16", 3), ("bf16", 2), ("f32", 2)])
def test_rows_sixteen_items(fmt, x_dtype, batch):
    # the largest launch: 16 matrices, narrow ones and ones split along K
    # (fp32: those run once per row), each equal to its own call bitwise
    say(f"multi-row 16 items {fmt} batch {batch} x {x_dtype}")
    ws, items, ys = [], [], []
    for i in range(16):
        rows, nblk = 3 + 13 * i, (5 if i % 3 else 20)
        w = Weights(fmt, rows, nblk * 256, seed=1800 + i)
        x = to_dev_x(gen_x(batch, nblk * 256, x_dtype, seed=180 + i), x_dtype)
        y = torch.full((batch, rows), -2.0, dtype=torch.float32, device=DEV)
        ws.append((w, x))
        ys.append(y)
        items.append((w.desc, x, y))
    qmv.qmv_gemv_multi(fmt, x_dtype, batch, items)
    for (w, x), y in zip(ws, ys):
        alone = w.gemv(x, x_dtype, batch)
        assert torch.equal(y, alone), (w.rows, w.cols)
