"""The benchmark's own launches, at full size, against the oracle: every row.

For every configuration bench.py times, the matrices are generated from the
same seeds, laid out as bench.py lays them out (plane layout where it uses
one) and issued in its launch grouping (q+k+v, o, gate+up, down as
multi-matrix launches; the matrix-core path for Q4_K batches), taken from
bench.workload_plan itself.  Every output of every matrix is compared with
the float64 oracle, decoded in row chunks: the 2e-3 normwise gate per
activation row is asserted, and the a-priori elementwise diagnostic
max |y - y64| / (gamma_{K+1} sum_k |w x|) is printed, not gated (kernels
that apply the block scales after partial sums may exceed it).
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from block_quantized_weight_qmv_amd import qmv
from gpu_util import DEV, Weights, gemv_ws, say, to_dev_x
from synth import gen_x, weight_seed, x_seed

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 2e-3

CASES = [(1, None, None), (2, None, None), (3, None, None), (4, None, None), (6, None, None),
         (5, 1, None), (5, 4, None), (5, 16, None), (5, 64, None), (5, 512, None),
         (3, 8, "bf16"), (3, 8, "f16")]


@pytest.mark.parametrize("config,batch,x_dtype", CASES,
                         ids=[f"c{c}-m{b}-{x}" for c, b, x in CASES])
def test_bench_launches_match_oracle(config, batch, x_dtype):
    layout = bench.default_layout(config, batch, x_dtype)
    plan = bench.workload_plan(config, batch, False, layout, x_dtype)
    fmt, xd_name, b = plan["fmt"], plan["x_dtype"], plan["batch"]
    mats, groups = plan["mats"], plan["groups"]
    say(f"bench launches config {config} batch {b} {fmt} x {xd_name} {layout}: {plan['launch_names']}")
    for gi, g in enumerate(groups):
        lead = g[0]
        x = gen_x(b, mats[lead][2], xd_name, x_seed(config, lead))
        xd = to_dev_x(x, xd_name)
        ws, descs, keep = [], [], []
        for m in g:
            name, rows, cols = mats[m]
            w = Weights(fmt, rows, cols, seed=weight_seed(config, m))
            d = w.desc
            if layout == "planes":
                buf = torch.empty(qmv.qmv_planes_size(fmt, rows, cols), dtype=torch.uint8, device=DEV)
                d = qmv.qmv_repack_planes(w.desc, buf)
                keep.append(buf)
            ws.append(w)
            descs.append(d)
        ys = [torch.full((b, mats[m][1]), 7.0, dtype=torch.float32, device=DEV) for m in g]
        say(f"  launch {plan['launch_names'][gi]} ({plan['kname'][gi]})")
        # as the benchmark issues it: one launch with the workspace it asks for
        wsbuf = gemv_ws(fmt, [(d, xd, y) for d, y in zip(descs, ys)], xd_name, b)
        torch.cuda.synchronize()
        del wsbuf
        for w, m, y in zip(ws, g, ys):
            name, rows, cols = mats[m]
            got = y.cpu().numpy().astype(np.float64)
            y64, bound = oracle.gemv64_and_bound(fmt, w.oracle_bytes(), rows, cols, x, xd_name)
            err = oracle.normwise_rel_err(got, y64)
            diag = np.max(np.abs(got - y64) / np.where(bound > 0, bound, np.inf))
            say(f"    {name} {rows}x{cols}: all {rows} rows x {b}: normwise err {err.max():.3e}, "
                f"max |y - y64| / elementwise bound {diag:.3f}")
            assert np.all(err <= TOL), (name, err.max())
        del ws, descs, keep, ys
        torch.cuda.empty_cache()


@pytest.mark.parametrize("config,m,layout", [(4, 0, "blocks"), (4, 0, "planes"), (3, 4, "blocks"),
                                             (3, 4, "planes")],
                         ids=["lm-head-blocks", "lm-head-planes", "gate-blocks", "gate-planes"])
def test_full_size_dequant_bit_exact(config, m, layout):
    """qmv_dequant of a whole benchmark matrix (the 152064 x 3584 lm-head's fp32
    output is 2.18 GB, past 2^31 byte offsets) against the oracle, bit for bit
    (+0 and -0 equal), compared in row chunks."""
    from synth import CONFIGS
    cfg = CONFIGS[config]
    fmt = cfg["fmt"]
    name, rows, cols = cfg["mats"][m]
    say(f"full-size dequant {fmt} {name} {rows}x{cols} {layout}")
    w = Weights(fmt, rows, cols, seed=weight_seed(config, m))
    d = w.desc
    keep = None
    if layout == "planes":
        keep = torch.empty(qmv.qmv_planes_size(fmt, rows, cols), dtype=torch.uint8, device=DEV)
        d = qmv.qmv_repack_planes(w.desc, keep)
    out = torch.full((rows, cols), float("nan"), dtype=torch.float32, device=DEV)
    qmv.qmv_dequant(d, out, "f32")
    torch.cuda.synchronize()
    data = w.oracle_bytes()
    chunk = 8192
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        want = oracle.dequant32(fmt, oracle.row_slice(fmt, data, rows, cols, r0, r1), r1 - r0, cols)
        got = out[r0:r1].cpu().numpy()
        eq = (got == want) | ((got == 0) & (want == 0))
        assert eq.all(), (r0, np.argwhere(~eq)[:5])
    say(f"  {rows} rows bit-exact")
    del out, keep
    torch.cuda.empty_cache()
