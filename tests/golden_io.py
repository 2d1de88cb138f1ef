"""Reader for the hand-computed block fixtures in tests/golden/ (format in its README)."""
import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _hex_tokens(tokens):
    out = []
    for tok in tokens:
        if "*" in tok:
            b, n = tok.split("*")
            out.extend([int(b, 16)] * int(n))
        else:
            out.append(int(tok, 16))
    return out


def load(name):
    fmt = rows = cols = None
    data, fills, ramps, points, sums = [], [], [], [], []
    with open(os.path.join(GOLDEN_DIR, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].split()
            if not line:
                continue
            key, args = line[0], line[1:]
            if key == "format":
                fmt = args[0]
            elif key == "rows":
                rows = int(args[0])
            elif key == "cols":
                cols = int(args[0])
            elif key == "bytes":
                data.extend(_hex_tokens(args))
            elif key == "fill":
                fills.append((int(args[0]), int(args[1]), int(args[2]), float(args[3])))
            elif key == "ramp":
                ramps.append((int(args[0]), int(args[1]), int(args[2]), float(args[3]), float(args[4])))
            elif key == "w":
                points.append((int(args[0]), int(args[1]), float(args[2])))
            elif key == "gemv_ones":
                sums.append((int(args[0]), float(args[1])))
            else:
                raise ValueError(f"{name}: unknown directive {key}")
    w = np.full((rows, cols), np.nan)
    for r, t0, t1, v in fills:
        w[r, t0:t1] = v
    for r, t0, t1, a, b in ramps:
        w[r, t0:t1] = a + b * np.arange(t1 - t0)
    for r, t, v in points:
        w[r, t] = v
    if np.isnan(w).any():
        raise ValueError(f"{name}: not every weight has an expected value")
    return {"fmt": fmt, "rows": rows, "cols": cols,
            "data": np.array(data, np.uint8), "w": w, "row_sums": sums}


def all_names():
    return sorted(f for f in os.listdir(GOLDEN_DIR) if f.endswith(".txt"))
