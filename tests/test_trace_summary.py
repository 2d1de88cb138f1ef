"""The kernel-trace summarizer of bench.py assigns every traced dispatch to
its matrix, also where several matrices share a kernel and a grid and the
timing replays run them alone (a 7B-layer-like step: q, k, v in one launch,
o, gate+up, down; q, k, v, o and down on one kernel, o and down on one grid,
and a helper kernel before two of the launches)."""
import argparse
import contextlib
import csv
import io

import bench

K1, K2, AUX = "qmv::kern_a<1>", "qmv::kern_b<2>", "qmv::helper"
DUR = {"q": 46.0, "k": 43.0, "v": 43.5, "o": 45.0, "gate": 111.0, "up": 112.0, "down": 208.0, "aux": 3.0}
GRID = {"q": 14336, "k": 2048, "v": 2048, "o": 14336, "gate": 15360, "up": 15360, "down": 14336, "aux": 512}


def _plan():
    names = ["q", "k", "v", "o", "gate", "up", "down"]
    mats = [(n, 1, 1) for n in names]
    groups = [[0, 1, 2], [3], [4, 5], [6]]
    disp = [(0, 0, AUX), (0, 0, K1), (0, 1, K1), (0, 2, K1), (1, 3, K1), (2, 4, AUX), (2, 4, K2), (2, 5, K2),
            (3, 6, K1)]
    return {"dispatches": disp, "names": names, "mats": mats, "groups": groups,
            "launch_names": ["q+k+v", "o", "gate+up", "down"], "by_kernel": {K1: [0, 1, 3], K2: [2]}, "dom": K2,
            "gbytes": [1.0, 1.0, 2.0e8, 1.0], "gflops": [1.0, 1.0, 2.23e11, 1.0],
            "bound": ["mfma"] * 4}


def _trace(tmp_path, plan):
    disp = plan["dispatches"]
    names = plan["names"]
    seq = []
    for _ in range(3):  # full steps
        seq += list(range(len(disp)))
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
        key = "aux" if kname == AUX else names[m]
        d = DUR[key] + (0.5 if j % 7 == 0 else 0.0)
        rows.append({"Kernel_Name": f"void {kname}(unsigned char const*)", "Grid_Size_X": GRID[key],
                     "Grid_Size_Y": 4, "Grid_Size_Z": 1, "Start_Timestamp": t, "End_Timestamp": t + int(d * 1000)})
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


def test_trace_summary_assigns_lookalike_dispatches(tmp_path, monkeypatch):
    plan = _plan()
    monkeypatch.setattr(bench, "workload_plan", lambda *a, **k: plan)
    args = argparse.Namespace(summarize_trace=_trace(tmp_path, plan), config=3, batch=512, separate=False,
                              layout="blocks", x_dtype="bf16")
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        assert bench.summarize_trace(args) == 0
    text = out.getvalue()
    med = {}
    for line in text.splitlines():
        cells = [c.strip() for c in line.split("|")]
        if len(cells) > 7 and cells[2] and cells[2].split()[0] in DUR and cells[3].strip("`") != AUX:
            med[cells[2].split()[0]] = (int(cells[5]), float(cells[6]))
    assert {k: v[1] for k, v in med.items()} == {k: v for k, v in DUR.items() if k != "aux"}
    # q, k, v, o, down: 3 full steps + 4 kernel replays + 5 launch replays
    assert all(n == 12 for n, _ in med.values()), med
    assert "matched no replay" not in text
    assert "226.000 us" in text  # gate + up and the helper before them: the dominant kernel's launch
