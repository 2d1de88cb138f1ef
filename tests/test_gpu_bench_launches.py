"""The benchmark's own launches, at full size, against the oracle.

For every configuration bench.py times, the matrices are generated from the
same seeds, laid out as bench.py lays them out (plane layout where it uses
one) and issued in its launch grouping (q+k+v, o, gate+up, down as
multi-matrix launches; the matrix-core path for Q4_K x bf16 batches), taken
from bench.workload_plan itself.  Sampled output rows of every matrix meet
the 2e-3 normwise gate against the float64 oracle.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from block_quantized_weight_qmv_amd import qmv
from gpu_util import DEV, Weights, oracle_y, say, to_dev_x
from synth import gen_x, weight_seed, x_seed

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _sample_rows(rows, n=32, seed=0):
    g = np.random.Generator(np.random.PCG64(seed))
    return np.unique(np.concatenate([[0, 1, rows // 2, rows - 2, rows - 1], g.integers(0, rows, n)]))


@pytest.mark.parametrize("config,batch", [(1, None), (2, None), (3, None), (4, None), (6, None),
                                          (5, 1), (5, 4), (5, 64)])
def test_bench_launches_match_oracle(config, batch):
    layout = bench.default_layout(config, batch)
    plan = bench.workload_plan(config, batch, False, layout)
    fmt, x_dtype, b = plan["fmt"], plan["x_dtype"], plan["batch"]
    mats, groups = plan["mats"], plan["groups"]
    say(f"bench launches config {config} batch {b} {fmt} x {x_dtype} {layout}: {plan['launch_names']}")
    ws, descs, keep = [], [], []
    for i, (name, rows, cols) in enumerate(mats):
        w = Weights(fmt, rows, cols, seed=weight_seed(config, i))
        d = w.desc
        if layout == "planes":
            buf = torch.empty(qmv.qmv_planes_size(fmt, rows, cols), dtype=torch.uint8, device=DEV)
            d = qmv.qmv_repack_planes(w.desc, buf)
            keep.append(buf)
        ws.append(w)
        descs.append(d)
    for gi, g in enumerate(groups):
        lead = g[0]
        x = gen_x(b, mats[lead][2], x_dtype, x_seed(config, lead))
        xd = to_dev_x(x, x_dtype)
        ys = [torch.full((b, mats[m][1]), 7.0, dtype=torch.float32, device=DEV) for m in g]
        if len(g) == 1:
            m = g[0]
            qmv.qmv_gemv(fmt, descs[m], xd, x_dtype, ys[0], mats[m][1], mats[m][2], b)
        else:
            qmv.qmv_gemv_multi(fmt, x_dtype, b, [(descs[m], xd, y) for m, y in zip(g, ys)])
        torch.cuda.synchronize()
        for m, y in zip(g, ys):
            ids = _sample_rows(mats[m][1], seed=config * 31 + m)
            got = y.cpu().numpy()[:, ids]
            err = oracle.normwise_rel_err(got, oracle_y(ws[m], x, x_dtype, ids))
            say(f"  {mats[m][0]}: sampled normwise err {err.max():.3e}")
            assert np.all(err <= TOL), (mats[m][0], err.max())
    del ws, descs, keep
    torch.cuda.empty_cache()
