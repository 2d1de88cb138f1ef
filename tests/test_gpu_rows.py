"""Q4_K with several fp16 or bf16 activation rows: the multi-row GEMV.

qmv_gemv routes Q4_K with two or more fp16 activation rows, or 2-4 bf16 rows,
against matrices of at most 4096 columns to a GEMV that reads W once per two
or four rows.  Each row's products and sums are the batch-1 GEMV's operations
in the same order and the wave reduction adds in the same order, so every
output row must equal the batch-1 GEMV of that activation row bit for bit,
and the float64 oracle within the 2e-3 normwise gate.  Shapes: one block,
ragged tiles, a full wave K slice, odd block counts; batches 2, 3 (a partial
group of four) and 4, fp16 batches of several groups; both layouts; several
matrices in one launch; graph replay; the full 18944 x 3584 batched workload
at M = 2, 3, 4 (all rows compared with the batch-1 GEMV, sampled rows with
the oracle).
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
SHAPES = [(1, 1), (3, 1), (5, 3), (67, 14), (9, 16), (40, 5), (130, 2)]


def _planes(w: Weights):
    buf = torch.empty(qmv.qmv_planes_size(w.fmt, w.rows, w.cols), dtype=torch.uint8, device=DEV)
    desc = qmv.qmv_repack_planes(w.desc, buf)
    desc.keep = buf
    return desc


def _per_row(desc, rows, cols, xd, x_dtype, batch):
    """The batch-1 GEMV of each activation row."""
    out = []
    for i in range(batch):
        y = torch.empty(1, rows, dtype=torch.float32, device=DEV)  # own buffer: 16-byte aligned
        qmv.qmv_gemv("q4_k", desc, xd[i:i + 1].clone(), x_dtype, y, rows, cols, 1)
        out.append(y)
    return torch.cat(out)


@pytest.mark.parametrize("layout", ["blocks", "planes"])
@pytest.mark.parametrize("x_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("batch", [2, 3, 4])
@pytest.mark.parametrize("rows,nblk", SHAPES)
def test_rows_equal_batch1_and_oracle(layout, x_dtype, batch, rows, nblk):
    cols = nblk * 256
    say(f"multi-row q4_k {layout} {rows}x{cols} batch {batch} x {x_dtype}")
    w = Weights("q4_k", rows, cols, seed=1300 + rows + nblk)
    desc = w.desc if layout == "blocks" else _planes(w)
    x = gen_x(batch, cols, x_dtype, seed=130 + batch + nblk)
    xd = to_dev_x(x, x_dtype)
    # one row past the batch: must stay untouched
    y = torch.full((batch + 1, rows), 7.25, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv("q4_k", desc, xd, x_dtype, y, rows, cols, batch)
    got = y.cpu().numpy()
    assert np.all(got[batch] == 7.25)
    np.testing.assert_array_equal(got[:batch], _per_row(desc, rows, cols, xd, x_dtype, batch).cpu().numpy())
    err = oracle.normwise_rel_err(got[:batch], oracle_y(w, x, x_dtype))
    say(f"  normwise err max {err.max():.3e}")
    assert np.all(err <= TOL), err


@pytest.mark.parametrize("layout", ["blocks", "planes"])
@pytest.mark.parametrize("batch", [5, 8, 9, 30])
@pytest.mark.parametrize("rows,nblk", [(3, 1), (67, 14), (130, 2)])
def test_rows_f16_groups_of_four(layout, batch, rows, nblk):
    # fp16 batches above four: one pass over W per group of four rows, the
    # last group partial unless four divides the batch
    cols = nblk * 256
    say(f"multi-row q4_k {layout} {rows}x{cols} batch {batch} x f16")
    w = Weights("q4_k", rows, cols, seed=1600 + rows + nblk)
    desc = w.desc if layout == "blocks" else _planes(w)
    x = gen_x(batch, cols, "f16", seed=160 + batch + nblk)
    xd = to_dev_x(x, "f16")
    y = torch.full((batch + 1, rows), 7.25, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv("q4_k", desc, xd, "f16", y, rows, cols, batch)
    got = y.cpu().numpy()
    assert np.all(got[batch] == 7.25)
    np.testing.assert_array_equal(got[:batch], _per_row(desc, rows, cols, xd, "f16", batch).cpu().numpy())
    assert np.all(oracle.normwise_rel_err(got[:batch], oracle_y(w, x, "f16")) <= TOL)


@pytest.mark.parametrize("layout", ["blocks", "planes"])
@pytest.mark.parametrize("batch", [2, 4])
def test_rows_multi_matrix_launch(layout, batch):
    # q, k, v-shaped matrices (scaled down) in one launch, each with its own x
    shapes = [(96, 14), (16, 14), (16, 14), (33, 3)]
    say(f"multi-row multi-matrix {layout} batch {batch}")
    ws, descs, xs, ys, items = [], [], [], [], []
    for i, (rows, nblk) in enumerate(shapes):
        w = Weights("q4_k", rows, nblk * 256, seed=1400 + i)
        d = w.desc if layout == "blocks" else _planes(w)
        x = gen_x(batch, nblk * 256, "bf16", seed=140 + i)
        ws.append(w)
        descs.append(d)
        xs.append((x, to_dev_x(x, "bf16")))
        ys.append(torch.full((batch, rows), -1.0, dtype=torch.float32, device=DEV))
        items.append((d, xs[-1][1], ys[-1]))
    qmv.qmv_gemv_multi("q4_k", "bf16", batch, items)
    for w, d, (x, xd), y in zip(ws, descs, xs, ys):
        got = y.cpu().numpy()
        ref = _per_row(d, w.rows, w.cols, xd, "bf16", batch).cpu().numpy()
        np.testing.assert_array_equal(got, ref)
        assert np.all(oracle.normwise_rel_err(got, oracle_y(w, x, "bf16")) <= TOL)


def test_rows_graph_replay():
    rows, cols, batch = 300, 14 * 256, 4
    say("multi-row graph replay")
    w = Weights("q4_k", rows, cols, seed=1500)
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


@pytest.mark.parametrize("layout", ["blocks", "planes"])
@pytest.mark.parametrize("batch", [2, 3, 4])
def test_rows_full_size_batched_ffn(layout, batch):
    cfg = CONFIGS[5]
    rows, cols = cfg["mats"][0][1], cfg["mats"][0][2]
    say(f"full-size multi-row {layout} {rows}x{cols} batch {batch}")
    w = Weights("q4_k", rows, cols, seed=weight_seed(5, 0))
    desc = w.desc if layout == "blocks" else _planes(w)
    x = gen_x(batch, cols, "bf16", x_seed(5, 0))
    xd = to_dev_x(x, "bf16")
    y = torch.empty(batch, rows, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv("q4_k", desc, xd, "bf16", y, rows, cols, batch)
    got = y.cpu().numpy()
    np.testing.assert_array_equal(got, _per_row(desc, rows, cols, xd, "bf16", batch).cpu().numpy())
    g = np.random.Generator(np.random.PCG64(40 + batch))
    ids = np.sort(g.choice(rows, size=48, replace=False))
    ids = np.unique(np.concatenate([ids, [0, rows - 1]]))
    ref = oracle_y(w, x, "bf16", row_ids=ids)
    err = oracle.normwise_rel_err(got[:, ids], ref)
    say(f"  sampled normwise err max {err.max():.3e}")
    assert np.all(err <= TOL), err
