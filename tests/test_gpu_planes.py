"""Q4_K, Q5_K and Q6_K in the plane layout (qmv_repack_planes) on the GPU.

The repack only moves bytes, so dequantization from planes must equal the
canonical layout's bit for bit (and the oracle's).  The plane GEMV runs the
canonical GEMV's arithmetic in the same order with the same launch shape, so
its outputs must equal the canonical layout's bitwise, and the oracle's
within the 2e-3 normwise gate.  The full 7B decoder-layer shapes are checked
in the launch grouping the benchmark times (q+k+v, o, gate+up, down), the
Q6_K lm-head and the Q5_K down projection at full size.
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
# (rows, blocks per row): one block, ragged tiles, a wave's full K slice plus
# one, several waves along K, an odd block count per row
SHAPES = [(1, 1), (3, 1), (5, 3), (67, 14), (33, 17), (9, 74), (40, 5)]


FMTS = ["q4_k", "q5_k", "q6_k"]


def _planes(w: Weights, align_pad=0):
    n = qmv.qmv_planes_size(w.fmt, w.rows, w.cols)
    buf = torch.full((n + align_pad,), 0xA5, dtype=torch.uint8, device=DEV)
    dst = buf[align_pad:] if align_pad else buf
    desc = qmv.qmv_repack_planes(w.desc, dst)
    desc.keep = buf
    return desc


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,nblk", SHAPES)
def test_repack_dequant_bit_exact(fmt, rows, nblk):
    cols = nblk * 256
    say(f"planes dequant {fmt} {rows}x{cols}")
    w = Weights(fmt, rows, cols, seed=900 + rows + nblk)
    p = _planes(w, align_pad=16 if rows == 5 else 0)  # one case off 256-byte alignment
    assert p.layout == 1 and p.nbytes == qmv.qmv_planes_size(fmt, rows, cols)
    a = torch.empty(rows, cols, dtype=torch.float32, device=DEV)
    b = torch.empty_like(a)
    qmv.qmv_dequant(w.desc, a, "f32")
    qmv.qmv_dequant(p, b, "f32")
    got = b.cpu().numpy()
    assert np.array_equal(got, a.cpu().numpy())
    assert np.array_equal(got, oracle.dequant32(fmt, w.oracle_bytes(), rows, cols))
    for dt, tdt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        c = torch.empty(rows, cols, dtype=tdt, device=DEV)
        d = torch.empty_like(c)
        qmv.qmv_dequant(w.desc, c, dt)
        qmv.qmv_dequant(p, d, dt)
        assert torch.equal(c.view(torch.int16), d.view(torch.int16)), dt


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,nblk", SHAPES)
@pytest.mark.parametrize("x_dtype", ["f32", "f16", "bf16"])
def test_planes_gemv_equals_blocks_and_oracle(fmt, rows, nblk, x_dtype):
    cols = nblk * 256
    batch = 3 if rows < 40 else 1  # Q4_K x bf16 with batch >= 2: the matrix-core path
    say(f"planes gemv {fmt} {rows}x{cols} batch {batch} x {x_dtype}")
    w = Weights(fmt, rows, cols, seed=700 + rows + nblk)
    p = _planes(w)
    x = gen_x(batch, cols, x_dtype, seed=77 + nblk)
    xd = to_dev_x(x, x_dtype)
    y_blocks = w.gemv(xd, x_dtype, batch)
    y_planes = torch.full((batch, rows), 123.0, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv(fmt, p, xd, x_dtype, y_planes, rows, cols, batch)
    got = y_planes.cpu().numpy()
    assert np.array_equal(got, y_blocks.cpu().numpy())
    err = oracle.normwise_rel_err(got, oracle_y(w, x, x_dtype))
    say(f"  normwise err {err.max():.3e}")
    assert np.all(err <= TOL), err


@pytest.mark.parametrize("fmt", FMTS)
def test_planes_multi_matches_separate_calls(fmt):
    items = [(67, 14), (16, 14), (130, 14), (33, 14)]
    ws, ps, ys = [], [], []
    x = gen_x(1, 14 * 256, "f32", seed=5)
    xd = to_dev_x(x, "f32")
    for i, (rows, nblk) in enumerate(items):
        w = Weights(fmt, rows, nblk * 256, seed=1100 + i)
        ws.append(w)
        ps.append(_planes(w))
        ys.append(torch.full((1, rows), -2.0, dtype=torch.float32, device=DEV))
    say(f"planes multi {fmt}: " + ", ".join(f"{w.rows}x{w.cols}" for w in ws))
    qmv.qmv_gemv_multi(fmt, "f32", 1, [(p, xd, y) for p, y in zip(ps, ys)])
    ref = []
    for w in ws:
        ref.append(torch.empty(1, w.rows, dtype=torch.float32, device=DEV))
    qmv.qmv_gemv_multi(fmt, "f32", 1, [(w.desc, xd, y) for w, y in zip(ws, ref)])
    torch.cuda.synchronize()
    for w, y, r in zip(ws, ys, ref):
        assert torch.equal(y, r), (w.rows, w.cols)
        err = oracle.normwise_rel_err(y.cpu().numpy(), oracle_y(w, x, "f32"))
        assert np.all(err <= TOL)


@pytest.mark.parametrize("fmt", FMTS)
def test_planes_multi_mixed_widths(fmt):
    """One launch over plane-layout matrices of different widths (one wave's
    K slice, two and five waves along K), each with its own activation:
    bitwise equal to the canonical layout's launch, within the gate."""
    items = [(67, 14), (16, 17), (33, 74), (5, 3)]
    ws, ps, xs_np, xs, yp, yb = [], [], [], [], [], []
    for i, (rows, nblk) in enumerate(items):
        w = Weights(fmt, rows, nblk * 256, seed=1300 + i)
        ws.append(w)
        ps.append(_planes(w))
        x = gen_x(1, nblk * 256, "f32", seed=1400 + i)
        xs_np.append(x)
        xs.append(to_dev_x(x, "f32"))
        yp.append(torch.full((1, rows), -4.0, dtype=torch.float32, device=DEV))
        yb.append(torch.full((1, rows), -4.0, dtype=torch.float32, device=DEV))
    say(f"planes multi mixed widths {fmt}: " + ", ".join(f"{w.rows}x{w.cols}" for w in ws))
    qmv.qmv_gemv_multi(fmt, "f32", 1, [(p, x, y) for p, x, y in zip(ps, xs, yp)])
    qmv.qmv_gemv_multi(fmt, "f32", 1, [(w.desc, x, y) for w, x, y in zip(ws, xs, yb)])
    torch.cuda.synchronize()
    for w, x, a, b in zip(ws, xs_np, yp, yb):
        assert torch.equal(a, b), (w.rows, w.cols)
        err = oracle.normwise_rel_err(a.cpu().numpy(), oracle_y(w, x, "f32"))
        assert np.all(err <= TOL), (w.rows, w.cols, err.max())


@pytest.mark.parametrize("fmt", FMTS)
def test_kept_planes_rewrapped(fmt):
    """Planes copied to a new buffer and wrapped with qmv_create_weights_planes
    compute what the repack's own descriptor computes, bitwise."""
    w = Weights(fmt, 50, 20 * 256, seed=21)
    p = _planes(w)
    copy = p.keep[:p.nbytes].clone()
    q = qmv.qmv_create_weights_planes(fmt, w.rows, w.cols, copy)
    x = to_dev_x(gen_x(1, w.cols, "f32", seed=22), "f32")
    ya = torch.empty(1, w.rows, dtype=torch.float32, device=DEV)
    yb = torch.empty_like(ya)
    qmv.qmv_gemv(fmt, p, x, "f32", ya, w.rows, w.cols, 1)
    qmv.qmv_gemv(fmt, q, x, "f32", yb, w.rows, w.cols, 1)
    assert torch.equal(ya, yb)


def test_planes_graph_replay_equals_eager():
    w = Weights("q4_k", 300, 14 * 256, seed=12)
    p = _planes(w)
    x = to_dev_x(gen_x(1, w.cols, "f32", seed=3), "f32")
    eager = torch.empty(1, w.rows, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv("q4_k", p, x, "f32", eager, w.rows, w.cols, 1)
    y = torch.empty_like(eager)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            qmv.qmv_gemv("q4_k", p, x, "f32", y, w.rows, w.cols, 1, stream=s)
    for rep in range(3):
        y.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {rep} differs"


@pytest.mark.parametrize("rows,nblk,batch", [(16, 2, 4), (70, 14, 16), (33, 20, 5),
                                             (130, 3, 17), (67, 14, 64), (40, 5, 130)])
def test_planes_on_the_matrix_core_path(rows, nblk, batch):
    """Q4_K x bf16 batches (every batched kernel: stream, K split, tile) read
    the plane layout with the canonical arithmetic: results equal bitwise."""
    cols = nblk * 256
    say(f"planes matrix cores {rows}x{cols} batch {batch}")
    w = Weights("q4_k", rows, cols, seed=60 + rows)
    p = _planes(w)
    x = gen_x(batch, cols, "bf16", seed=61 + batch)
    xd = to_dev_x(x, "bf16")
    yp = torch.full((batch, rows), 3.0, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv("q4_k", p, xd, "bf16", yp, rows, cols, batch)
    yb = w.gemv(xd, "bf16", batch)
    torch.cuda.synchronize()
    assert torch.equal(yp, yb)
    err = oracle.normwise_rel_err(yp.cpu().numpy(), oracle_y(w, x, "bf16"))
    assert np.all(err <= TOL), err


def _sample_rows(rows, n=48, seed=0):
    g = np.random.Generator(np.random.PCG64(seed))
    return np.unique(np.concatenate([[0, 1, rows // 2, rows - 2, rows - 1], g.integers(0, rows, n)]))


def test_full_size_layer_in_planes_sampled_rows():
    """The 7B Q4_K decoder layer, repacked, in the benchmark's four launches;
    every output equals the canonical layout's and sampled rows meet the gate."""
    cfg = CONFIGS[3]
    mats = cfg["mats"]
    names = [m[0] for m in mats]
    groups = [["q", "k", "v"], ["o"], ["gate", "up"], ["down"]]
    ws, ps, xs_np, xs = {}, {}, {}, {}
    for i, (name, rows, cols) in enumerate(mats):
        ws[name] = Weights("q4_k", rows, cols, seed=weight_seed(3, i))
        ps[name] = _planes(ws[name])
    for g in groups:
        lead = names.index(g[0])
        x = gen_x(1, mats[lead][2], "f32", x_seed(3, lead))
        for name in g:
            xs_np[name], xs[name] = x, to_dev_x(x, "f32")
    for g in groups:
        say("planes full-size launch " + "+".join(g))
        yp = {n: torch.empty(1, ws[n].rows, dtype=torch.float32, device=DEV) for n in g}
        yb = {n: torch.empty(1, ws[n].rows, dtype=torch.float32, device=DEV) for n in g}
        qmv.qmv_gemv_multi("q4_k", "f32", 1, [(ps[n], xs[n], yp[n]) for n in g])
        qmv.qmv_gemv_multi("q4_k", "f32", 1, [(ws[n].desc, xs[n], yb[n]) for n in g])
        torch.cuda.synchronize()
        for n in g:
            assert torch.equal(yp[n], yb[n]), n
            got = yp[n].cpu().numpy()
            ids = _sample_rows(ws[n].rows, seed=names.index(n))
            err = oracle.normwise_rel_err(got[:, ids], oracle_y(ws[n], xs_np[n], "f32", ids))
            say(f"  {n}: sampled normwise err {err.max():.3e}")
            assert np.all(err <= TOL)
    del ws, ps
    torch.cuda.empty_cache()


def test_full_size_q6_k_lm_head_in_planes_sampled_rows():
    """The Q6_K lm-head (152064 x 3584), repacked: every output equals the
    canonical layout's, and sampled rows meet the gate."""
    cfg = CONFIGS[4]
    name, rows, cols = cfg["mats"][0]
    say(f"planes full-size q6_k {name} {rows}x{cols}")
    w = Weights("q6_k", rows, cols, seed=weight_seed(4, 0))
    p = _planes(w)
    x = gen_x(1, cols, "f32", x_seed(4, 0))
    xd = to_dev_x(x, "f32")
    yp = torch.empty(1, rows, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv("q6_k", p, xd, "f32", yp, rows, cols, 1)
    yb = w.gemv(xd, "f32", 1)
    torch.cuda.synchronize()
    assert torch.equal(yp, yb)
    ids = _sample_rows(rows, seed=4)
    err = oracle.normwise_rel_err(yp.cpu().numpy()[:, ids], oracle_y(w, x, "f32", ids))
    say(f"  sampled normwise err {err.max():.3e}")
    assert np.all(err <= TOL)
    del w, p
    torch.cuda.empty_cache()


def test_full_size_q5_k_down_in_planes_sampled_rows():
    """The Q5_K down projection (3584 x 18944), repacked: every output equals
    the canonical layout's, and sampled rows meet the gate."""
    cfg = CONFIGS[6]
    name, rows, cols = cfg["mats"][0]
    say(f"planes full-size q5_k {name} {rows}x{cols}")
    w = Weights("q5_k", rows, cols, seed=weight_seed(6, 0))
    p = _planes(w)
    x = gen_x(1, cols, "f32", x_seed(6, 0))
    xd = to_dev_x(x, "f32")
    yp = torch.empty(1, rows, dtype=torch.float32, device=DEV)
    qmv.qmv_gemv("q5_k", p, xd, "f32", yp, rows, cols, 1)
    yb = w.gemv(xd, "f32", 1)
    torch.cuda.synchronize()
    assert torch.equal(yp, yb)
    ids = _sample_rows(rows, seed=6)
    err = oracle.normwise_rel_err(yp.cpu().numpy()[:, ids], oracle_y(w, x, "f32", ids))
    say(f"  sampled normwise err {err.max():.3e}")
    assert np.all(err <= TOL)
