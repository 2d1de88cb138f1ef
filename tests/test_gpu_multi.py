"""qmv_gemv_multi on the GPU: several matrices in one launch.

Each item is checked against the float64 oracle with the same normwise bound
as qmv_gemv (2e-3), and against a separate qmv_gemv call of the same matrix
(same per-row arithmetic, so the two agree to float32 rounding).  Items mix
shapes with one and several waves along K, ragged row counts and shared or
distinct activations; y buffers carry canaries between items.
"""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_weight_qmv_amd import qmv
from gpu_util import DEV, Weights, gemv_ws, oracle_y, say, to_dev_x
from synth import gen_x

pytestmark = pytest.mark.gpu

TOL = 2e-3
FMTS = ("q8_0", "q4_k", "q6_k", "int4_g128", "q5_k")
# (rows, blocks per row) per item; the last item spans several waves along K
ITEMS = {
    "q8_0": [(67, 48), (5, 48), (130, 48), (33, 300)],
    "q4_k": [(67, 14), (5, 14), (130, 14), (33, 40)],
    "q6_k": [(67, 14), (5, 14), (130, 14), (33, 40)],
    "int4_g128": [(67, 28), (5, 28), (130, 28), (33, 80)],
    "q5_k": [(67, 14), (5, 14), (130, 14), (33, 40)],
}


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("x_dtype", ["f32", "f16", "bf16"])
def test_multi_matches_oracle_and_single_calls(fmt, x_dtype):
    qk = oracle.QK[fmt]
    batch = 2
    ws, xs_np, xs, ys = [], [], [], []
    # one flat y buffer with a canary gap of 16..19 floats after each item
    # (each item's y starts 16-byte aligned)
    sizes = [batch * r for r, _ in ITEMS[fmt]]
    offs = np.cumsum([0] + [(s + 16 + 3) // 4 * 4 for s in sizes])
    ybuf = torch.full((int(offs[-1]),), 7.25, dtype=torch.float32, device=DEV)
    shared = None
    for i, (rows, nblk) in enumerate(ITEMS[fmt]):
        cols = nblk * qk
        w = Weights(fmt, rows, cols, seed=900 + 7 * i)
        if i in (0, 1, 2):  # q/k/v-style items read one activation
            if shared is None:
                shared = gen_x(batch, cols, x_dtype, seed=77)
            x = shared
        else:
            x = gen_x(batch, cols, x_dtype, seed=78 + i)
        ws.append(w)
        xs_np.append(x)
        xs.append(to_dev_x(x, x_dtype))
        ys.append(ybuf[int(offs[i]):int(offs[i]) + sizes[i]])
    say(f"multi {fmt} x {x_dtype}: " + ", ".join(f"{w.rows}x{w.cols}" for w in ws))
    qmv.qmv_gemv_multi(fmt, x_dtype, batch, [(w.desc, x, y) for w, x, y in zip(ws, xs, ys)])
    torch.cuda.synchronize()
    host = ybuf.cpu().numpy()
    for i, w in enumerate(ws):
        gap = host[int(offs[i]) + sizes[i]:int(offs[i + 1])]
        assert np.all(gap == 7.25), f"canary after item {i} overwritten"
        y = host[int(offs[i]):int(offs[i]) + sizes[i]].reshape(batch, w.rows)
        err = oracle.normwise_rel_err(y, oracle_y(w, xs_np[i], x_dtype))
        say(f"  item {i} {w.rows}x{w.cols}: normwise err {err.max():.3e}")
        assert np.all(err <= TOL), err
        single = w.gemv(xs[i], x_dtype, batch).cpu().numpy()
        np.testing.assert_allclose(y, single, rtol=1e-5, atol=1e-5 * np.abs(single).max())


@pytest.mark.parametrize("fmt", FMTS)
def test_multi_sixteen_items(fmt):
    qk = oracle.QK[fmt]
    nblk = {"q8_0": 40, "q4_k": 5, "q6_k": 5, "int4_g128": 10, "q5_k": 5}[fmt]
    cols = nblk * qk
    ws = [Weights(fmt, 3 + 11 * i, cols, seed=500 + i) for i in range(16)]
    x_np = gen_x(1, cols, "f32", seed=5)
    x = to_dev_x(x_np, "f32")
    ys = [torch.empty(1, w.rows, dtype=torch.float32, device=DEV) for w in ws]
    say(f"multi16 {fmt} cols {cols}")
    qmv.qmv_gemv_multi(fmt, "f32", 1, [(w.desc, x, y) for w, y in zip(ws, ys)])
    for w, y in zip(ws, ys):
        err = oracle.normwise_rel_err(y.cpu().numpy(), oracle_y(w, x_np, "f32"))
        assert np.all(err <= TOL), err


def test_multi_graph_replay_matches_eager():
    fmt, x_dtype = "q4_k", "bf16"
    ws = [Weights(fmt, r, 14 * 256, seed=40 + r) for r in (96, 16, 16)]
    x_np = gen_x(1, 14 * 256, x_dtype, seed=9)
    x = to_dev_x(x_np, x_dtype)
    ys = [torch.zeros(1, w.rows, dtype=torch.float32, device=DEV) for w in ws]
    items = [(w.desc, x, y) for w, y in zip(ws, ys)]
    qmv.qmv_gemv_multi(fmt, x_dtype, 1, items)
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            qmv.qmv_gemv_multi(fmt, x_dtype, 1, items, stream=s)
    for rep in range(3):
        for y in ys:
            y.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert torch.equal(y, e), f"replay {rep} differs"


@pytest.mark.parametrize("batch", [2, 4, 24, 64])
def test_multi_q4_k_bf16_batches_per_item_routing(batch):
    """Q4_K x bf16 with batch >= 2: each item runs the kernel its own call
    takes (the multi-row GEMV for matrices of at most 4096 columns at batch
    2-4, the matrix cores otherwise), whatever the other items of the launch;
    results match the oracle and the same item called alone (same kernel,
    same arithmetic: bitwise)."""
    items = [(67, 14), (16, 14), (130, 3), (33, 20)]
    ws, xs_np, xs, ys = [], [], [], []
    for i, (rows, nblk) in enumerate(items):
        cols = nblk * 256
        w = Weights("q4_k", rows, cols, seed=1500 + 11 * i)
        x = gen_x(batch, cols, "bf16", seed=1600 + i)
        ws.append(w)
        xs_np.append(x)
        xs.append(to_dev_x(x, "bf16"))
        ys.append(torch.full((batch, rows), -3.0, dtype=torch.float32, device=DEV))
    say(f"multi q4_k bf16 batch {batch}: " + ", ".join(f"{w.rows}x{w.cols}" for w in ws))
    qmv.qmv_gemv_multi("q4_k", "bf16", batch, [(w.desc, x, y) for w, x, y in zip(ws, xs, ys)])
    torch.cuda.synchronize()
    for w, x_np, x, y in zip(ws, xs_np, xs, ys):
        got = y.cpu().numpy()
        err = oracle.normwise_rel_err(got, oracle_y(w, x_np, "bf16"))
        assert np.all(err <= TOL), (w.rows, w.cols, err.max())
        alone = w.gemv(x, "bf16", batch).cpu().numpy()
        assert np.array_equal(got, alone), (w.rows, w.cols)


@pytest.mark.parametrize("x_dtype,batch", [("bf16", 5), ("bf16", 8), ("f16", 16)])
def test_multi_small_q4_k_matrices_share_one_multi_row_launch(x_dtype, batch):
    """Several small Q4_K matrices (q, k, v shaped, scaled down) at 5-16 rows:
    one multi-row launch, so every output row equals the batch-1 GEMV of that
    activation row bitwise, and the oracle within the gate."""
    items = [(192, 14), (32, 14), (32, 14)]
    x_np = gen_x(batch, 14 * 256, x_dtype, seed=2100 + batch)
    xd = to_dev_x(x_np, x_dtype)
    ws = [Weights("q4_k", r, nb * 256, seed=2000 + i) for i, (r, nb) in enumerate(items)]
    ys = [torch.full((batch, w.rows), -3.0, dtype=torch.float32, device=DEV) for w in ws]
    say(f"multi small q4_k x {x_dtype} batch {batch}")
    qmv.qmv_gemv_multi("q4_k", x_dtype, batch, [(w.desc, xd, y) for w, y in zip(ws, ys)])
    torch.cuda.synchronize()
    for w, y in zip(ws, ys):
        got = y.cpu().numpy()
        for i in range(batch):
            one = torch.empty(1, w.rows, dtype=torch.float32, device=DEV)
            w.gemv(xd[i:i + 1].clone(), x_dtype, 1, y=one)
            np.testing.assert_array_equal(got[i], one.cpu().numpy()[0])
        assert np.all(oracle.normwise_rel_err(got, oracle_y(w, x_np, x_dtype)) <= TOL)


@pytest.mark.parametrize("x_dtype,batch", [("bf16", 17), ("bf16", 32), ("bf16", 128), ("f16", 64), ("bf16", 300)])
def test_multi_register_dequantized_runs(x_dtype, batch):
    """With a workspace, consecutive Q4_K items of at least 256 rows on one
    activation share one register-dequantized launch from 17 rows (a q+k+v-like run of three, then
    a lone matrix of another width that runs alone): every item meets the
    oracle gate, as its own call does (below 65 rows a lone call of these
    matrices takes the exact-product kernels, so the two differ by the fp16
    rounding of the weights; above, by float32 summation order).  Without a
    workspace the launch gives each item its plain call's result, bit for
    bit."""
    items = [(520, 14), (256, 14), (300, 14), (257, 9)]
    ws = [Weights("q4_k", r, n * 256, seed=1700 + 13 * i) for i, (r, n) in enumerate(items)]
    x14 = gen_x(batch, 14 * 256, x_dtype, seed=1800 + batch)
    x9 = gen_x(batch, 9 * 256, x_dtype, seed=1900 + batch)
    xd14, xd9 = to_dev_x(x14, x_dtype), to_dev_x(x9, x_dtype)
    ys = [torch.full((batch, w.rows), -3.0, dtype=torch.float32, device=DEV) for w in ws]
    xs = [xd14, xd14, xd14, xd9]
    say(f"multi q4_k {x_dtype} batch {batch}: run of three on one activation, one more")
    buf = gemv_ws("q4_k", [(w.desc, x, y) for w, x, y in zip(ws, xs, ys)], x_dtype, batch)
    torch.cuda.synchronize()
    del buf
    # without a workspace every item takes the exact-product kernels of its own plain call
    yp = [torch.full_like(y, -5.0) for y in ys]
    qmv.qmv_gemv_multi("q4_k", x_dtype, batch, [(w.desc, x, y) for w, x, y in zip(ws, xs, yp)])
    for w, x_np, xd, y, y_plain in zip(ws, [x14, x14, x14, x9], xs, ys, yp):
        got = y.cpu().numpy()
        err = oracle.normwise_rel_err(got, oracle_y(w, x_np, x_dtype))
        assert np.all(err <= TOL), (w.rows, w.cols, err.max())
        alone = w.gemv(xd, x_dtype, batch).cpu().numpy()
        apart = oracle.normwise_rel_err(got, alone.astype(np.float64))
        assert np.all(apart <= (2 * TOL if batch < 65 else 1e-5)), (w.rows, w.cols, apart.max())
        assert torch.equal(y_plain, w.gemv(xd, x_dtype, batch, ws=False)), (w.rows, w.cols)


PAIR_CASES = [("q8_0", "blocks"), ("q4_k", "blocks"), ("q4_k", "planes"), ("q5_k", "planes"), ("q6_k", "blocks"),
              ("q6_k", "planes"), ("int4_g128", "blocks")]


@pytest.mark.parametrize("x_dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("rows,eighths,batch", [(1, 8, 1), (67, 3, 1), (4100, 8, 1), (67, 3, 2), (130, 8, 2),
                                                (1, 8, 3), (67, 5, 3), (300, 8, 4)])
@pytest.mark.parametrize("fmt,layout", PAIR_CASES)
def test_multi_pair_of_one_shape(fmt, layout, rows, eighths, batch, x_dtype):
    """Two matrices of one shape on the same activation rows (gate and up):
    at one row they run as one launch whose two-row tiles pair row i of
    each; at two or more rows as two items of the multi-row GEMV.  Every
    output against the oracle, and against each matrix called alone -- bit
    for bit, except INT4 at one row, whose lone call runs one-row tiles and
    so another reduction order."""
    qk = oracle.QK[fmt]
    slice_cols = 2048 if fmt == "q8_0" else 4096
    cols = max(qk, slice_cols * eighths // 8 // qk * qk)
    ws = [Weights(fmt, rows, cols, seed=2600 + 5 * i + rows) for i in range(2)]
    keep, descs = [], []
    for w in ws:
        d = w.desc
        if layout == "planes":
            buf = torch.empty(qmv.qmv_planes_size(fmt, rows, cols), dtype=torch.uint8, device=DEV)
            d = qmv.qmv_repack_planes(w.desc, buf)
            keep.append(buf)
        descs.append(d)
    x = gen_x(batch, cols, x_dtype, seed=2700 + rows)
    xd = to_dev_x(x, x_dtype)
    n = batch * rows
    off = (n + 4 + 3) // 4 * 4  # the second output 16-byte aligned, a canary gap between
    ybuf = torch.full((off + n + 4,), 7.25, dtype=torch.float32, device=DEV)
    ys = [ybuf[:n], ybuf[off:off + n]]
    say(f"multi pair {fmt} {layout} {rows}x{cols} batch {batch} x {x_dtype}")
    qmv.qmv_gemv_multi(fmt, x_dtype, batch, [(d, xd, y) for d, y in zip(descs, ys)])
    torch.cuda.synchronize()
    host = ybuf.cpu().numpy()
    assert np.all(host[n:off] == 7.25) and np.all(host[off + n:] == 7.25)
    for w, d, y in zip(ws, descs, ys):
        got = y.cpu().numpy().reshape(batch, rows)
        err = oracle.normwise_rel_err(got, oracle_y(w, x, x_dtype))
        assert np.all(err <= TOL), err
        alone = torch.empty(batch, rows, dtype=torch.float32, device=DEV)
        qmv.qmv_gemv(fmt, d, xd, x_dtype, alone, rows, cols, batch)
        alone = alone.cpu().numpy()
        if fmt == "int4_g128" and batch == 1:
            np.testing.assert_allclose(got, alone, rtol=1e-5, atol=1e-5 * np.abs(alone).max())
        else:
            np.testing.assert_array_equal(got, alone)
    del keep
