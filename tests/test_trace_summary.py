"""The kernel-trace summarizer of bench.py assigns every traced dispatch to
its matrix, also where several matrices share a kernel and a grid and the
timing replays run them alone (here o and down of a 7B decoder layer at 512
bf16 rows: one register-dequantized kernel, one grid)."""
import argparse
import csv
import io
import contextlib

import bench

DUR = {"q": 46.0, "k": 43.0, "v": 43.5, "o": 45.0, "gate": 111.0, "up": 112.0, "down": 208.0}


def _trace(tmp_path, plan):
    disp = plan["dispatches"]
    names = plan["names"]
    grid = {"q": 14336, "k": 2048, "v": 2048, "o": 14336, "gate": 15360, "up": 15360, "down": 14336}
    seq = []
    full = list(range(len(disp)))
    for _ in range(3):
        seq += full
    for gis in plan["by_kernel"].values():  # per-kernel timing replays
        for _ in range(4):
            seq += [si for si, d in enumerate(disp) if d[0] in gis]
    for gi in range(len(plan["groups"])):  # per-launch timing replays
        for _ in range(5):
            seq += [si for si, d in enumerate(disp) if d[0] == gi]
    t = 1000
    rows = []
    for j, si in enumerate(seq):
        _, m, kname = disp[si]
        d = DUR[names[m]] + (0.5 if j % 7 == 0 else 0.0)
        rows.append({"Kernel_Name": f"void {kname}(unsigned char const*)", "Grid_Size_X": grid[names[m]],
                     "Grid_Size_Y": 4, "Grid_Size_Z": 1, "Start_Timestamp": t,
                     "End_Timestamp": t + int(d * 1000)})
        t += int(d * 1000) + 2000
    rows.append({"Kernel_Name": "void qmv::probe_read_kernel(float*)", "Grid_Size_X": 262144, "Grid_Size_Y": 1,
                 "Grid_Size_Z": 1, "Start_Timestamp": t, "End_Timestamp": t + 300000})
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)
    return str(d)


def test_trace_summary_assigns_lookalike_dispatches(tmp_path):
    plan = bench.workload_plan(3, 512, False, "blocks", "bf16")
    assert [n for _, _, n in plan["dispatches"]].count(plan["kname"][1]) == 5  # q, k, v, o, down alike
    args = argparse.Namespace(summarize_trace=_trace(tmp_path, plan), config=3, batch=512, separate=False,
                              layout="blocks", x_dtype="bf16")
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        assert bench.summarize_trace(args) == 0
    text = out.getvalue()
    med = {}
    for line in text.splitlines():
        cells = [c.strip() for c in line.split("|")]
        if len(cells) > 7 and cells[2] and cells[2].split()[0] in DUR:
            med[cells[2].split()[0]] = (int(cells[5]), float(cells[6]))
    assert {k: v[1] for k, v in med.items()} == DUR
    # q, k, v: 3 full steps + 4 kernel replays + 5 launch replays; o and down the same
    assert all(n == 12 for n, _ in med.values()), med
    assert "matched no replay" not in text
    assert "223.000 us" in text  # gate + up, the dominant kernel's one launch
