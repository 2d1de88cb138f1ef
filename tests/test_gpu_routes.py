"""bench.py's names for the kernels it times are the kernels the library runs.

bench.kernel_name restates the library's dispatch rules (which kernel serves a
launch, by format, activation type, batch, widths and layout) to label its
figures and to pick the dominant kernel.  For every benchmarked launch plan,
one eager step of bench.py is traced with rocprofv3 (kernel trace only) in a
child process, and the GEMV dispatches of that step, in order, must carry the
names the plan gives (the load-time repacks and the probes are left out).  A
launch group served by the matrix-core kernels dispatches per matrix, named
for that matrix's shape (the register-dequantized kernel with its activation
conversion before it and, with K in slices, the partial-output sum after
it); every other group is one dispatch.
"""
import csv
import glob
import os
import subprocess
import sys
import tempfile

import pytest

from gpu_util import say

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

pytestmark = pytest.mark.gpu

PLANS = [(1, None, None), (2, None, None), (3, None, None), (4, None, None), (6, None, None),
         (5, 1, None), (5, 4, None), (5, 16, None), (5, 64, None), (5, 256, None), (5, 512, None),
         (3, 8, "bf16"), (3, 8, "f16"), (5, 512, "f16"), (5, 100, "f16"), (2, 4, None), (3, 256, "bf16"),
         (3, 17, "bf16"), (3, 32, "bf16"), (3, 64, "bf16"), (3, 128, "f16"), (3, 512, "bf16"), (5, 32, None)]


def _dispatched(trace_dir):
    files = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True))
    assert files, f"no kernel trace under {trace_dir}"
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                rows.append((int(r["Start_Timestamp"]), bench.kernel_display_name(r["Kernel_Name"])))
    rows.sort()
    return [n for _, n in rows if n.startswith("qmv::") and "repack" not in n and "probe" not in n]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("config,batch,x_dtype", PLANS, ids=[f"c{c}-m{b}-{x}" for c, b, x in PLANS])
def test_bench_kernel_names_are_dispatched(config, batch, x_dtype):
    layout = bench.default_layout(config, batch, x_dtype)
    plan = bench.workload_plan(config, batch, False, layout, x_dtype)
    say(f"route config {config} batch {plan['batch']} x {plan['x_dtype']} {layout}: {plan['kname']}")
    cmd = ["rocprofv3", "--kernel-trace", "--output-format", "csv", "-d", None, "-o", "run", "--",
           sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--eager-pass", "--steps", "1", "--warmup", "0",
           "--config", str(config)]
    if batch is not None:
        cmd += ["--batch", str(batch)]
    if x_dtype is not None:
        cmd += ["--x-dtype", x_dtype]
    with tempfile.TemporaryDirectory(dir="/tmp") as td:
        cmd[cmd.index(None)] = td
        env = dict(os.environ, TMPDIR="/tmp", PYTHONPATH=ROOT)
        r = subprocess.run(cmd, cwd=td, env=env, capture_output=True, text=True, timeout=240)
        assert r.returncode == 0, (r.returncode, r.stdout[-2000:], r.stderr[-2000:])
        got = _dispatched(td)
    want = [k for _, _, k in plan["dispatches"]]
    say(f"  dispatched {got}")
    assert got == want, (got, want)
