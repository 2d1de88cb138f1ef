#!/usr/bin/env python3
"""Decode-GEMV benchmark on one MI355X: achieved HBM GB/s and µs per GEMV.

Default workload (one "step"): the seven batch-1 Q4_K GEMVs of one 7B-shaped
decoder layer -- q, o 3584x3584; k, v 512x3584; gate, up 18944x3584;
down 3584x18944 -- with fp32 activations ~ N(0, 1), seeded synthetic weights
(synth/), packed by the library's host packer and resident in HBM before the
timed region starts.  Distinct copies of the layer (>= 1.25 GiB in total) are
cycled so that the 256 MB Infinity Cache cannot serve repeated reads.

Output: one JSON line.  `value` is algorithmic bytes (packed weights + x + y)
per step divided by the measured time per step.  `roofline` covers the
dominant kernel (most time per step), timed with HIP events recorded on the
launch stream around each of its launches inside the timed region.
`cpu_baseline` times the CPU oracle (float64 decode + dot) on a bounded sample
of the same matrices.

    python bench.py [--steps K] [--warmup W] [--config {1,2,3,4,5}] [--batch M]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
CSRC = os.path.join(ROOT, "block_quantized_weight_qmv_amd", "csrc")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def kernel_name(fmt: str, cols: int, x_dtype: str) -> str:
    """Instantiation the library launches for this shape (mirrors the launcher's choice)."""
    per_wave = {"q8_0": 2048, "q4_k": 4096, "q6_k": 4096, "int4_g128": 4096}[fmt]
    kw = -(-cols // per_wave)
    threads = 64 * kw * (4 if kw == 1 else 1)
    cfg = "4, 256" if threads <= 256 else ("4, 512" if threads <= 512 else "2, 1024")
    pol = {"q8_0": "Q80Policy", "q4_k": "Q4KPolicy", "q6_k": "Q6KPolicy",
           "int4_g128": "Int4G128Policy"}[fmt]
    xt = {"f32": "float", "f16": "_Float16", "bf16": "qmv::bf16_t"}[x_dtype]
    return f"gemv_kernel<qmv::{pol}, {xt}, {cfg}>"


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter runs, if the kernels are unchanged."""
    try:
        with open(COUNTERS_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    rec = data.get(workload, {})
    if rec.get("kernel") != kernel or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(mats, fmt, x_dtype, fields_list, xs, seconds):
    """Time the CPU oracle (decode to float64 + float64 dot) on row chunks of the workload."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    chunk = 512
    done_bytes, spent, rows_done = 0, 0.0, 0
    it = 0
    while spent < seconds and it < 10000:
        m = it % len(mats)
        name, rows, cols = mats[m]
        r0 = (it // len(mats)) * chunk % rows
        r1 = min(rows, r0 + chunk)
        ids = np.arange(r0, r1)
        sub = {k: v[ids] for k, v in fields_list[m].items()}
        data = oracle.pack(fmt, sub, len(ids), cols)
        t0 = time.perf_counter()
        oracle.gemv64(fmt, data, len(ids), cols, xs[m], x_dtype)
        spent += time.perf_counter() - t0
        xb = {"f32": 4, "f16": 2, "bf16": 2}[x_dtype]
        done_bytes += data.size + cols * xb + len(ids) * 4
        rows_done += len(ids)
        it += 1
    return {"value": done_bytes / spent / 1e9, "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": (f"{rows_done} rows in {chunk}-row chunks cycling over the workload's "
                       f"matrices, {spent:.1f} s; numpy float64 decode (1 thread) + float64 "
                       f"matrix-vector product (BLAS, {blas_threads} threads); packing excluded")}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--batch", type=int, default=None, help="activation rows (config 5 only)")
    ap.add_argument("--rotate-gib", type=float, default=1.25)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single GPU: this library has no multi-GPU path "
              "(sharding is described in DESIGN.md). Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from block_quantized_weight_qmv_amd import qmv
    from synth import CONFIGS, gen_weights, gen_x, weight_seed, x_seed

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = CONFIGS[args.config]
    fmt, x_dtype = cfg["fmt"], cfg["x_dtype"]
    batch = args.batch or cfg["batch"][0]
    mats = cfg["mats"]
    xb = {"f32": 4, "f16": 2, "bf16": 2}[x_dtype]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[x_dtype]

    # -- inputs: synthesize, pack on the host with the library packer, upload ---
    fields_list, packed_dev, xs, xs_dev, ys = [], [], [], [], []
    for i, (name, rows, cols) in enumerate(mats):
        f = gen_weights(fmt, rows, cols, weight_seed(args.config, i))
        fields_list.append(f)
        packed_dev.append(torch.from_numpy(qmv.pack_fields(fmt, f, rows, cols)).to(dev))
        x = gen_x(batch, cols, x_dtype, x_seed(args.config, i))
        xs.append(x)
        xt = torch.from_numpy(x.view(np.int16) if x_dtype == "bf16" else x).to(dev)
        xs_dev.append(xt.view(tdt) if x_dtype == "bf16" else xt)
        ys.append(torch.empty(batch, rows, dtype=torch.float32, device=dev))
    step_w_bytes = sum(p.numel() for p in packed_dev)
    step_bytes = sum(p.numel() + batch * c * xb + batch * r * 4
                     for p, (_, r, c) in zip(packed_dev, mats))
    copies = max(1, int(np.ceil(args.rotate_gib * 2 ** 30 / step_w_bytes)))
    descs = []  # descs[c][m]
    keep = []
    for c in range(copies):
        row = []
        for m, (name, rows, cols) in enumerate(mats):
            t = packed_dev[m] if c == 0 else packed_dev[m].clone()
            keep.append(t)
            row.append(qmv.qmv_create_weights(fmt, rows, cols, t))
        descs.append(row)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def launch(c, m):
        _, rows, cols = mats[m]
        qmv.qmv_gemv(fmt, descs[c][m], xs_dev[m], x_dtype, ys[m], rows, cols, batch, sp)

    # dominant kernel: the instantiation with the most algorithmic bytes per step
    kname = {m: kernel_name(fmt, mats[m][2], x_dtype) for m in range(len(mats))}
    by_kernel = {}
    for m in range(len(mats)):
        by_kernel.setdefault(kname[m], []).append(m)
    mbytes = [packed_dev[m].numel() + batch * mats[m][2] * xb + batch * mats[m][1] * 4
              for m in range(len(mats))]
    dom = max(by_kernel, key=lambda k: sum(mbytes[m] for m in by_kernel[k]))
    dom_ms = set(by_kernel[dom])

    for s in range(args.warmup):
        for m in range(len(mats)):
            launch(s % copies, m)
    torch.cuda.synchronize()

    # -- timed region ------------------------------------------------------------
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(mats) + 1)]
          for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        c = (args.warmup + s) % copies
        ev[s][0].record(stream)
        for m in range(len(mats)):
            launch(c, m)
            ev[s][m + 1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    per_launch_ms = np.array([[ev[s][m].elapsed_time(ev[s][m + 1]) for m in range(len(mats))]
                              for s in range(args.steps)])
    med_us = np.median(per_launch_ms, axis=0) * 1e3
    detail = {mats[m][0]: {"shape": f"{mats[m][1]}x{mats[m][2]}", "bytes": int(mbytes[m]),
                           "median_us": round(float(med_us[m]), 3),
                           "GBps": round(mbytes[m] / (med_us[m] * 1e-6) / 1e9, 1)}
              for m in range(len(mats))}
    dom_time_s = per_launch_ms[:, sorted(dom_ms)].sum() / 1e3
    dom_launches = args.steps * len(dom_ms)
    dom_avg_us = dom_time_s / dom_launches * 1e6
    dom_bytes_per_launch = sum(mbytes[m] for m in dom_ms) / len(dom_ms)
    achieved = dom_bytes_per_launch / (dom_avg_us * 1e-6) / 1e9

    # -- HBM read ceiling on this GPU (128-bit streaming read of 2 GiB) ----------------
    nb = 2 * 2 ** 30
    buf = torch.empty(nb, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    out = torch.empty(qmv.qmv_probe_read_outputs(nb), dtype=torch.float32, device=dev)
    for _ in range(3):
        qmv.qmv_probe_read(buf, nb, out, sp)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(10):
        qmv.qmv_probe_read(buf, nb, out, sp)
    b.record(stream)
    torch.cuda.synchronize()
    read_ceiling = nb * 10 / (a.elapsed_time(b) * 1e-3) / 1e9
    del buf, out

    workload = cfg["name"] + (f"_m{batch}" if args.config == 5 else "")
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    rec = {
        "metric": "achieved HBM GB/s (% of peak) and µs per GEMV, batch-1 7B-shaped Q4_K",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": workload, "format": fmt, "batch": batch, "x_dtype": x_dtype,
                   "matrices": {n: f"{r}x{c}" for n, r, c in mats},
                   "bytes_per_step": int(step_bytes), "weight_copies": copies},
        "pct_of_peak": round(100 * value / PEAK_GBPS, 1),
        "us_per_gemv": round(ms_per_step * 1e3 / len(mats), 3),
        "per_matrix": detail,
        "read_ceiling_GBps": round(read_ceiling, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4),
                     "traffic": measured_traffic(dom, workload),
                     "kernel": dom, "avg_launch_us": round(dom_avg_us, 3),
                     "launches_per_step": len(dom_ms),
                     "bytes_per_launch": round(dom_bytes_per_launch, 1)},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(mats, fmt, x_dtype, fields_list, xs, args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
