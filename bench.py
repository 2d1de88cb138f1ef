#!/usr/bin/env python3
"""Decode-GEMV benchmark on one MI355X: achieved HBM GB/s and µs per GEMV.

Default workload (one "step"): the seven batch-1 Q4_K GEMVs of one 7B-shaped
decoder layer -- q, o 3584x3584; k, v 512x3584; gate, up 18944x3584;
down 3584x18944 -- with fp32 activations ~ N(0, 1), seeded synthetic weights
(synth/), packed by the library's host packer and resident in HBM before the
timed region starts.  Distinct copies of the layer (>= 1.25 GiB in total) are
cycled so that the 256 MB Infinity Cache cannot serve repeated reads.

The step issues the layer's GEMVs in decode order, one launch per group of
projections that read the same activation (qmv_gemv_multi_ws, with one
caller-owned workspace sized by qmv_workspace_size): [q, k, v], [o],
[gate, up], [down].  `--separate` issues one launch per matrix instead.

Output: one JSON line.  `value` is algorithmic bytes (packed weights + x + y)
per step divided by the measured time per step.  For the default workload the
line also carries `batched`: the same measurement, run first in child
processes, of the batched bf16 workloads (the FFN gate at 64 and 512 rows,
the whole layer at 17, 64, 128 and 512 rows, with one caller workspace),
their step and launch times and their dominant kernel's roofline.
`swiglu_fused` times gate and up as one launch that writes silu(gate) * up
(qmv_gemv_swiglu) next to the unfused gate+up launch.
`roofline` covers the dominant kernel (most bytes per step): a graph of the
same K steps restricted to that kernel's launches, replayed between HIP
events on the replay stream.
`cpu_baseline` times the CPU oracle (float64 decode + dot) on a bounded sample
of the same matrices.

    python bench.py [--steps K] [--warmup W] [--config {1,2,3,4,5,6}] [--batch M]
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


# Sources each kernel family is built from: a change to any of them voids the
# committed counter figures for that family (and only for it).
_KERNEL_SOURCES = {
    "gemv_kernel": ["gemv_skeleton.h", "device_util.h"],
    "gemv_rows_kernel": ["gemv_skeleton.h", "device_util.h"],
    "gemv_pair_kernel": ["gemv_skeleton.h", "device_util.h"],
    "gemv_glu_kernel": ["gemv_skeleton.h", "device_util.h"],
    "gemm_q4_k_stream": ["gemm_q4_k_mfma.hip", "device_util.h"],
    "gemm_q4_k_ksplit": ["gemm_q4_k_mfma.hip", "device_util.h"],
    "gemm_q4_k_tile": ["gemm_q4_k_mfma.hip", "device_util.h"],
}
_POLICY_SOURCE = {"Q80Policy": "gemv_q8_0.hip", "Q4KPolicy": "gemv_q4_k.hip",
                  "Q4KPlanesPolicy": "gemv_q4_k.hip", "Q5KPlanesPolicy": "gemv_q5_k.hip",
                  "Q6KPlanesPolicy": "gemv_q6_k.hip",
                  "Q5KPolicy": "gemv_q5_k.hip", "Q6KPolicy": "gemv_q6_k.hip",
                  "Int4G128Policy": "gemv_int4_g128.hip"}


def kernel_source_hash(kernel: str) -> str:
    """Hash of the source files the named kernel instantiation is compiled from."""
    fam = kernel.split("::")[1].split("<")[0] if "::" in kernel else kernel
    files = list(_KERNEL_SOURCES.get(fam, sorted(os.listdir(CSRC))))
    for pol, src in _POLICY_SOURCE.items():
        if pol in kernel:
            files.append(src)
    h = hashlib.sha256()
    for name in sorted(files):
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


# Compute units of the MI355X; the register-dequantized plans depend on it.
DEVICE_CUS = 256
# Q4_K x fp16/bf16 batches take the register-dequantized kernels for
# matrices of at least DQ_MIN_ROWS rows: from DQ_MIN_BATCH_RUN rows for runs
# of two or more matrices of a launch and for matrices of at least DQ_LONGK
# columns, from DQ_MIN_BATCH rows for any matrix.
DQ_MIN_BATCH, DQ_MIN_BATCH_RUN, DQ_LONGK, DQ_MIN_ROWS = 65, 17, 8192, 256


def dq_eligible(rows: int, cols: int, batch: int, layout: str) -> bool:
    """The launcher's dqreg_eligible for a Q4_K matrix and fp16/bf16 rows
    (byte offsets of weights and activations within 32 bits)."""
    if rows < DQ_MIN_ROWS or batch < DQ_MIN_BATCH_RUN:
        return False
    nb = cols // 256
    a = -(-16 * rows * nb // 256) * 256  # the plane unit
    wbytes = (5 * a + 64 * rows * nb) if layout == "planes" else 144 * rows * nb
    return wbytes < 2 ** 32 and 2 * batch * cols < 2 ** 32


def dqreg_plan(rows, cols: int, batch: int, cus: int = DEVICE_CUS):
    """(T, NB, slices, blocks per slice) of gemm_q4_k_dqreg for one matrix of
    `rows` rows, or a run of matrices (a list of row counts) in one launch:
    the launcher's model, rounds of workgroups over the compute units times a
    workgroup's time ((14 + 17 / T) ns per product of a wave at NB = 8,
    (20 + 16 / T) at NB = 4, 5.5 us fixed), plus the sum of the partial
    outputs when K is sliced (3 us and its bytes at 8 TB/s).  Ties keep the
    first in the order NB = 8 then 4, smaller T, fewer slices."""
    rows_list = list(rows) if isinstance(rows, (list, tuple)) else [rows]
    nb = cols // 256
    best = None
    for nbt in (8, 4):
        for t in (1, 2, 3, 4, 5):
            for s in range(1, min(8, nb) + 1):
                bps = -(-nb // s)
                splits = -(-nb // bps)
                if splits != s:
                    continue
                tiles = sum(-(-r // (64 * t)) for r in rows_list)
                wgs = tiles * -(-batch // (16 * nbt)) * splits
                products = float(bps * 8 * nbt * t)
                per = 20.0 + 16.0 / t if nbt == 4 else 14.0 + 17.0 / t
                us = float(-(-wgs // cus)) * (products * per * 1e-3 + 5.5)
                if splits > 1:
                    us += 3.0 + float(splits + 1) * sum(rows_list) * batch * 4 / 8e6
                if best is None or us < best[0]:
                    best = (us, t, nbt, splits, bps)
    return best[1:]


def dq_run(mats, batch: int, layout: str):
    """How many of the leading matrices (rows, cols) one register-dequantized
    launch covers: those eligible with the first one's width, up to four; 0
    if the first is not eligible, or is alone below DQ_MIN_BATCH rows with
    fewer than DQ_LONGK columns."""
    if not mats or not dq_eligible(mats[0][0], mats[0][1], batch, layout):
        return 0
    k = 1
    while k < min(len(mats), 4) and mats[k][1] == mats[0][1] and dq_eligible(mats[k][0], mats[k][1], batch, layout):
        k += 1
    if k == 1 and batch < DQ_MIN_BATCH and mats[0][1] < DQ_LONGK:
        return 0
    return k


def dq_kernel_name(rows, cols: int, batch: int, layout: str) -> str:
    """The register-dequantized kernel for one matrix or a run of matrices."""
    pl = "true" if layout == "planes" else "false"
    t, nbt = dqreg_plan(rows, cols, batch)[:2]
    d = 1 if t >= 3 else 2
    return f"qmv::gemm_q4_k_dqreg<{t}, {nbt}, {d}, {d}, {pl}>"


def group_dispatches(fmt: str, mats, x_dtype: str, batch: int, layout: str):
    """(kernel, first matrix, matrices) of each dispatch the matrices (rows,
    cols) of one launch on the matrix-core path make, in order: a run of up
    to four register-dequantized matrices of one width is one product
    launch, after the activation conversion (skipped when the previous run
    converted the same activations: a launch's matrices share them) and,
    with K in slices, before one sum of the partial outputs; the other
    matrices take one matrix-core kernel each."""
    out = []
    prev = None
    i = 0
    while i < len(mats):
        rows, cols = mats[i]
        k = dq_run(mats[i:], batch, layout) if fmt == "q4_k" and x_dtype in ("f16", "bf16") else 0
        if k:
            run_rows = [m[0] for m in mats[i:i + k]]
            if prev != cols:
                out.append((f"qmv::act_rows_f16<{'false' if x_dtype == 'f16' else 'true'}>", i, k))
            out.append((dq_kernel_name(run_rows, cols, batch, layout), i, k))
            if dqreg_plan(run_rows, cols, batch)[2] > 1:
                out.append(("qmv::dqreg_sum", i, k))
            prev = cols
            i += k
        else:
            out.append((kernel_name(fmt, [cols], x_dtype, batch, layout, [rows]), i, 1))
            prev = None
            i += 1
    return out


def kernel_name(fmt: str, cols_list, x_dtype: str, batch: int = 1, layout: str = "blocks",
                rows_list=None) -> str:
    """Instantiation the library launches for matrices of these widths in one
    launch (mirrors the dispatch in api.cpp and the GEMV launcher: Q4_K x bf16
    with batch >= 2 not taken by the multi-row GEMV (below) -> one of the
    matrix-core kernels, chosen by batch and by
    whether X fits in LDS; otherwise waves per workgroup = max(4, widest K
    split), and the shared-activation kernel when no matrix splits K; Q4_K
    weights in the plane layout take the plane policy; two or more rows
    (Q4_K x bf16: 2-4 rows) against matrices within one wave's K slice (4096
    columns, Q8_0 2048) -> the multi-row GEMV (fp32: two rows per pass);
    fp16/bf16 against two to eight waves along K -> its K-split form, except
    Q4_K x bf16 above two rows; Q4_K x fp16 from 5 rows -> the matrix-core
    kernels of bf16 with fp16 operands; two or more small Q4_K matrices at
    5-16 fp16/bf16 rows (rows_list summing to at most 8192) -> one multi-row
    launch; Q4_K x fp16/bf16 from 128 rows (from 64 against 8192 columns and
    more) against matrices of at least 256 rows -> gemm_q4_k_dqreg in the
    form dqreg_plan picks; one activation row against two matrices of one
    shape within one wave's K slice (gate, up) -> the paired kernel; the
    first matrix of a group names the group)."""
    nb_max = max(cols_list) // 256
    if (fmt == "q4_k" and x_dtype in ("f16", "bf16") and 5 <= batch <= 16 and len(cols_list) >= 2
            and max(cols_list) <= 4096 and rows_list is not None and sum(rows_list) <= 8192):
        # several small matrices (q, k, v): one multi-row launch, groups of four rows
        pol = "Q4KPlanesPolicy" if layout == "planes" else "Q4KPolicy"
        xt = "_Float16" if x_dtype == "f16" else "qmv::bf16_t"
        return f"qmv::gemv_rows_kernel<qmv::{pol}, {xt}, 1, 3, 256, 4>"
    if fmt == "q4_k" and x_dtype in ("f16", "bf16") and rows_list is not None:  # the register-dequantized kernels
        k = dq_run(list(zip(rows_list, cols_list)), batch, layout)
        if k:
            return dq_kernel_name(list(rows_list[:k]), cols_list[0], batch, layout)
    if fmt == "q4_k" and x_dtype == "f16" and batch >= 17:  # fp16 on the tile kernels
        pl = "true" if layout == "planes" else "false"
        mb = 1 if batch <= 32 else (2 if batch <= 64 else 4)
        return f"qmv::gemm_q4_k_tile<1, {mb}, 2, 5, {pl}, true>"
    if fmt == "q4_k" and x_dtype == "f16" and batch >= 5:  # fp16 on the matrix cores, up to 16 rows
        pl = "true" if layout == "planes" else "false"
        if nb_max * 8 * 1088 + 8 * 2 * 4 * 64 * 4 <= 160 * 1024:  # X fits the stream kernel's LDS
            return f"qmv::gemm_q4_k_stream<{pl}, true>"
        return f"qmv::gemm_q4_k_ksplit<1, 1, {pl}, true>"
    wave_cols = 2048 if fmt == "q8_0" else 4096
    kw_max = -(-max(cols_list) // wave_cols)
    q4k_bf16 = fmt == "q4_k" and x_dtype == "bf16"
    half = x_dtype in ("f16", "bf16")
    if (batch >= 2 and not (q4k_bf16 and batch > 4)
            and (kw_max == 1 or (2 <= kw_max <= 8 and half and not (q4k_bf16 and batch > 2)))):
        pol = {"q8_0": "Q80Policy", "q4_k": "Q4KPolicy", "q5_k": "Q5KPolicy", "q6_k": "Q6KPolicy",
               "int4_g128": "Int4G128Policy"}[fmt]
        if layout == "planes":
            pol = {"q4_k": "Q4KPlanesPolicy", "q5_k": "Q5KPlanesPolicy", "q6_k": "Q6KPlanesPolicy"}[fmt]
        xt = {"f32": "float", "f16": "_Float16", "bf16": "qmv::bf16_t"}[x_dtype]
        if kw_max > 1:  # K-split form, two rows per pass
            r = 1 if fmt == "q5_k" else 2
            return f"qmv::gemv_rows_split_kernel<qmv::{pol}, {xt}, {r}, 2, {256 if max(kw_max, 4) <= 4 else 512}>"
        shape = "2, 2, 256, 2" if batch == 2 or not half else ("1, 3, 256, 3" if batch == 3 else "1, 3, 256, 4")
        return f"qmv::gemv_rows_kernel<qmv::{pol}, {xt}, {shape}>"
    if fmt == "q4_k" and x_dtype == "bf16" and batch >= 2:
        nb = max(cols_list) // 256
        pl = "true" if layout == "planes" else "false"
        if batch <= 16 and nb * 8 * 1088 + 8 * 2 * 4 * 64 * 4 <= 160 * 1024:  # X fits in LDS
            return f"qmv::gemm_q4_k_stream<{pl}, false>"
        if batch <= 16:
            return f"qmv::gemm_q4_k_ksplit<1, 1, {pl}, false>"
        if batch <= 32:
            return f"qmv::gemm_q4_k_tile<1, 1, 2, 5, {pl}, false>"
        return (f"qmv::gemm_q4_k_tile<1, 2, 2, 5, {pl}, false>" if batch <= 64
                else f"qmv::gemm_q4_k_tile<1, 4, 2, 5, {pl}, false>")
    per_wave = {"q8_0": 2048, "q4_k": 4096, "q6_k": 4096, "int4_g128": 4096, "q5_k": 4096}[fmt]
    waves = max([4] + [-(-c // per_wave) for c in cols_list])
    kw = max(-(-c // per_wave) for c in cols_list)
    pol = {"q8_0": "Q80Policy", "q4_k": "Q4KPolicy", "q6_k": "Q6KPolicy",
           "int4_g128": "Int4G128Policy", "q5_k": "Q5KPolicy"}[fmt]
    if layout == "planes":
        pol = {"q4_k": "Q4KPlanesPolicy", "q5_k": "Q5KPlanesPolicy", "q6_k": "Q6KPlanesPolicy"}[fmt]
    xt = {"f32": "float", "f16": "_Float16", "bf16": "qmv::bf16_t"}[x_dtype]
    if len(cols_list) == 1 and 2 <= kw <= 8:   # one matrix split along K: slices in LDS
        return f"qmv::gemv_lx_kernel<qmv::{pol}, {xt}, 2, 2, 512>"
    if (batch == 1 and kw == 1 and len(cols_list) == 2 and cols_list[0] == cols_list[1]
            and rows_list is not None and rows_list[0] == rows_list[1]):
        # two matrices of one shape on one activation (gate, up): rows paired per tile
        return f"qmv::gemv_pair_kernel<qmv::{pol}, {xt}, 256>"
    if kw == 1:   # the shared-activation kernel; INT4 with one-row tiles, three in flight
        cfg = "1, 3, 256, true" if fmt == "int4_g128" else "2, 2, 256, true"
    else:
        cfg = "2, 2, 256, false" if waves <= 4 else ("2, 2, 512, false" if waves <= 8 else "1, 2, 1024, false")
    pol = {"q8_0": "Q80Policy", "q4_k": "Q4KPolicy", "q6_k": "Q6KPolicy",
           "int4_g128": "Int4G128Policy", "q5_k": "Q5KPolicy"}[fmt]
    if layout == "planes":
        pol = {"q4_k": "Q4KPlanesPolicy", "q5_k": "Q5KPlanesPolicy", "q6_k": "Q6KPlanesPolicy"}[fmt]
    xt = {"f32": "float", "f16": "_Float16", "bf16": "qmv::bf16_t"}[x_dtype]
    return f"qmv::gemv_kernel<qmv::{pol}, {xt}, {cfg}>"


def decode_groups(names):
    """Launch groups in decode order: consecutive projections that read the same
    activation (q/k/v, gate/up) form one group; every other matrix is alone."""
    shared = [("q", "k", "v"), ("gate", "up")]
    groups, i = [], 0
    while i < len(names):
        for tup in shared:
            if tuple(names[i:i + len(tup)]) == tup:
                groups.append(list(range(i, i + len(tup))))
                i += len(tup)
                break
        else:
            groups.append([i])
            i += 1
    return groups


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter runs, if the kernels are unchanged."""
    try:
        with open(COUNTERS_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    rec = data.get(workload, {})
    if rec.get("kernel") != kernel or rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def _cpu_model() -> dict:
    """The host CPU as /proc/cpuinfo names it (model name, family, model, stepping)."""
    info = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if not ln.strip():
                    break   # first processor only
                k, _, v = ln.partition(":")
                info[k.strip()] = v.strip()
    except OSError:
        pass
    return {"model_name": info.get("model name", ""), "family": info.get("cpu family", ""),
            "model": info.get("model", ""), "stepping": info.get("stepping", ""),
            "vendor": info.get("vendor_id", "")}


def _median_of_3(fn):
    """Median of three timed calls after one untimed warm-up call (seconds)."""
    fn()
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return sorted(ts)[1]


def cpu_baseline(mats, fmt, x_dtype, fields_list, xs, sample_rows):
    """Time the CPU oracle on a bounded sample of every matrix of the workload.

    For each matrix, a block of `sample_rows` rows (all rows if fewer) is packed
    by the oracle and timed in two parts, each the median of three runs after
    one warm-up: the float64 decode (oracle.dequant64, numpy, one thread) and
    the float64 matrix-vector product of the decoded rows (BLAS).  Per-row times
    are scaled to the whole matrix, so the figures describe one full pass over
    the workload (one step).  The product is timed again with BLAS limited to
    one thread."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threadpool_limits, blas_threads = None, 1
    xb = {"f32": 4, "f16": 2, "bf16": 2}[x_dtype]
    dq_s = gemv_s = gemv1_s = 0.0
    step_bytes = 0
    rows_timed = 0
    t_all = time.perf_counter()
    for m, (name, rows, cols) in enumerate(mats):
        n = min(rows, sample_rows)
        ids = np.arange(n)
        sub = {k: v[ids] for k, v in fields_list[m].items()}
        data = oracle.pack(fmt, sub, n, cols)
        x64 = oracle.x_to_f64(xs[m], x_dtype).reshape(-1, cols)
        w = {}

        def dq():
            w["w"] = oracle.dequant64(fmt, data, n, cols)

        t_dq = _median_of_3(dq)
        t_mv = _median_of_3(lambda: x64 @ w["w"].T)
        if threadpool_limits is not None:
            with threadpool_limits(limits=1, user_api="blas"):
                t_mv1 = _median_of_3(lambda: x64 @ w["w"].T)
        else:
            t_mv1 = t_mv
        scale = rows / n
        dq_s += t_dq * scale
        gemv_s += t_mv * scale
        gemv1_s += t_mv1 * scale
        rows_timed += n
        step_bytes += data.size * scale + x64.size * xb + x64.shape[0] * rows * 4
    wall = time.perf_counter() - t_all
    step = dq_s + gemv_s
    step1 = dq_s + gemv1_s
    return {"value": step_bytes / step / 1e9, "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle",
            "dequant_ms_per_step": round(dq_s * 1e3, 3),
            "gemv64_ms_per_step": round(gemv_s * 1e3, 3),
            "gemv_per_s": round(len(mats) / step, 3),
            "single_thread": {"value": step_bytes / step1 / 1e9, "unit": "GB/s",
                              "gemv64_ms_per_step": round(gemv1_s * 1e3, 3),
                              "gemv_per_s": round(len(mats) / step1, 3)},
            "blas_threads": int(blas_threads), "affinity_cores": len(os.sched_getaffinity(0)),
            "cpu": _cpu_model(),
            "sample": (f"the first {sample_rows} rows of each of the workload's {len(mats)} matrices "
                       f"({rows_timed} rows, {wall:.1f} s of wall time); per matrix the oracle's "
                       "float64 decode (numpy, 1 thread) and its float64 matrix-vector product "
                       f"(BLAS, {blas_threads} threads; again with 1) each timed as the median of 3 "
                       "after 1 warm-up, per-row times scaled to the full matrices; packing excluded")}


PEAK_TFLOPS_BF16 = 2500.0   # MI355X dense bf16 matrix cores, vendor figure


def default_layout(config: int, batch: int | None = None, x_dtype: str | None = None) -> str:
    """Q4_K, Q5_K and Q6_K on the GEMV path stream the plane layout (repacked
    once at load, as a decode layout replacing the blocks); Q4_K x bf16
    batches on the matrix cores read the canonical blocks, which they stream
    3-17 % faster than planes (they accept both); Q8_0 and INT4 read their
    canonical layouts."""
    from synth import CONFIGS
    cfg = CONFIGS[config]
    b = batch or cfg["batch"][0]
    xd = x_dtype or cfg["x_dtype"]
    # Q4_K x bf16 batches of 5 or more run on the matrix cores; 2-4 rows take the multi-row GEMV
    gemv = not (cfg["fmt"] == "q4_k" and xd in ("bf16", "f16") and b >= 5)
    return "planes" if cfg["fmt"] in ("q4_k", "q5_k", "q6_k") and gemv else "blocks"


def workload_plan(config: int, batch: int | None, separate: bool, layout: str = "blocks",
                  x_dtype: str | None = None) -> dict:
    """Launches of one step and their algorithmic bytes and flops (no GPU needed).

    Bytes per launch = packed weights + each activation once + y; flops =
    2 * batch * rows * cols over the launch's matrices.  Each launch's bound is
    the roofline the kernel runs against: matrix cores when its arithmetic
    intensity exceeds the machine balance (dense bf16 peak / HBM peak), HBM
    otherwise."""
    from block_quantized_weight_qmv_amd import qmv
    from synth import CONFIGS
    cfg = CONFIGS[config]
    fmt = cfg["fmt"]
    x_dtype = x_dtype or cfg["x_dtype"]
    batch_given = batch is not None and batch != cfg["batch"][0]
    batch = batch or cfg["batch"][0]
    mats = cfg["mats"]
    names = [n for n, _, _ in mats]
    groups = [[m] for m in range(len(mats))] if separate else decode_groups(names)
    xb = {"f32": 4, "f16": 2, "bf16": 2}[x_dtype]
    size = qmv.qmv_planes_size if layout == "planes" else qmv.qmv_packed_size
    wbytes = [int(size(fmt, r, c)) for _, r, c in mats]
    gbytes = [sum(wbytes[m] + batch * mats[m][1] * 4 for m in g) + batch * mats[g[0]][2] * xb
              for g in groups]
    gflops = [sum(2.0 * batch * mats[m][1] * mats[m][2] for m in g) for g in groups]
    kname = [kernel_name(fmt, [mats[m][2] for m in g], x_dtype, batch, layout, [mats[m][1] for m in g])
             for g in groups]
    balance = PEAK_TFLOPS_BF16 * 1e12 / (PEAK_GBPS * 1e9)
    bound = ["mfma" if kname[i].startswith("qmv::gemm") and gflops[i] / gbytes[i] > balance
             else "hbm" for i in range(len(groups))]
    by_kernel = {}
    for gi in range(len(groups)):
        by_kernel.setdefault(kname[gi], []).append(gi)
    dom = max(by_kernel, key=lambda k: sum(gbytes[gi] for gi in by_kernel[k]))
    # the dispatches of one step in order: per matrix where a group runs on
    # the matrix-core kernels (each named for its matrix, with the register
    # kernel's conversion and sum kernels), else one per group
    dispatches = []
    for gi, g in enumerate(groups):
        if kname[gi].startswith("qmv::gemm"):
            # each dispatch is credited to the matrix it serves (None: several)
            for k, i0, n in group_dispatches(fmt, [(mats[m][1], mats[m][2]) for m in g], x_dtype, batch, layout):
                dispatches.append((gi, g[i0] if n == 1 else None, k))
        else:
            dispatches.append((gi, None, kname[gi]))
    workload = (cfg["name"] + (f"_m{batch}" if config == 5 or batch_given else "")
                + (f"_x{x_dtype}" if x_dtype != cfg["x_dtype"] else ""))
    return {"cfg": cfg, "fmt": fmt, "x_dtype": x_dtype, "batch": batch, "mats": mats,
            "names": names, "groups": groups, "wbytes": wbytes, "gbytes": gbytes,
            "gflops": gflops, "kname": kname, "bound": bound, "by_kernel": by_kernel,
            "dom": dom, "workload": workload, "layout": layout, "dispatches": dispatches,
            "launch_names": ["+".join(names[m] for m in g) for g in groups]}


_F16_FORMS = [
    (r"_ZN3qmv11gemv_kernelINS_\d+(\w+?)EDF16_Li(\d+)ELi(\d+)ELi(\d+)ELb([01])EEEvNS_10GemvLaunchE",
     lambda m: f"qmv::gemv_kernel<qmv::{m[1]}, _Float16, {m[2]}, {m[3]}, {m[4]}, {'true' if m[5] == '1' else 'false'}>"),
    (r"_ZN3qmv14gemv_lx_kernelINS_\d+(\w+?)EDF16_Li(\d+)ELi(\d+)ELi(\d+)EEEvNS_10GemvLxArgsE",
     lambda m: f"qmv::gemv_lx_kernel<qmv::{m[1]}, _Float16, {m[2]}, {m[3]}, {m[4]}>"),
    (r"_ZN3qmv16gemv_rows_kernelINS_\d+(\w+?)EDF16_Li(\d+)ELi(\d+)ELi(\d+)ELi(\d+)EEEvNS_10GemvLaunchEi",
     lambda m: f"qmv::gemv_rows_kernel<qmv::{m[1]}, _Float16, {m[2]}, {m[3]}, {m[4]}, {m[5]}>"),
    (r"_ZN3qmv22gemv_rows_split_kernelINS_\d+(\w+?)EDF16_Li(\d+)ELi(\d+)ELi(\d+)EEEvNS_10GemvLaunchEi",
     lambda m: f"qmv::gemv_rows_split_kernel<qmv::{m[1]}, _Float16, {m[2]}, {m[3]}, {m[4]}>"),
    (r"_ZN3qmv16gemv_pair_kernelINS_\d+(\w+?)EDF16_Li(\d+)EEEvNS_10GemvLaunchE",
     lambda m: f"qmv::gemv_pair_kernel<qmv::{m[1]}, _Float16, {m[2]}>"),
    (r"_ZN3qmv15gemv_glu_kernelINS_\d+(\w+?)EDF16_Li(\d+)EEEvNS_10GemvLaunchE",
     lambda m: f"qmv::gemv_glu_kernel<qmv::{m[1]}, _Float16, {m[2]}>"),
]


def kernel_display_name(name: str) -> str:
    """A kernel name as the traces print it, in bench.py's form: without
    'void ' and the argument list; the _Float16 instantiations, which the
    demangler leaves mangled, spelled out."""
    import re
    name = name.split("(")[0]
    name = name[5:] if name.startswith("void ") else name
    for pat, fmt in _F16_FORMS:
        m = re.fullmatch(pat, name)
        if m:
            return fmt(m)
    return name


def _counter_csv(d: str):
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    return files


def _per_dispatch(d: str, counter: str):
    """[(kernel name without 'void ' and arguments, summed counter value)] in dispatch order."""
    import csv
    acc = {}
    for f in _counter_csv(d):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (f, int(r["Dispatch_Id"]))
                name = kernel_display_name(r["Kernel_Name"])
                prev = acc.get(key, (name, 0.0, int(r.get("Grid_Size", 0) or 0)))
                acc[key] = (name, prev[1] + float(r["Counter_Value"]), prev[2])
    return [acc[k] for k in sorted(acc)]


def summarize_counters(args) -> int:
    """Turn four rocprofv3 --pmc runs into HBM bytes per launch (profiles/counters.json).

    Runs: FETCH_SIZE and WRITE_SIZE of `bench.py --eager-pass` for the workload,
    and of `python -m block_quantized_weight_qmv_amd.probe copy --mib N` for the
    scale factors (a copy of N MiB reads and writes N MiB)."""
    fetch_d, write_d, cfetch_d, cwrite_d = args.summarize_counters
    plan = workload_plan(args.config, args.batch, args.separate, _layout(args), args.x_dtype)
    groups, kname, gbytes = plan["groups"], plan["kname"], plan["gbytes"]
    copy_kib = args.copy_mib * 1024.0

    def copy_mean(d, counter):
        v = [val for name, val, _ in _per_dispatch(d, counter) if "probe_copy" in name]
        v = v[1:] or v
        return sum(v) / len(v)
    fetch_scale = copy_kib / copy_mean(cfetch_d, "FETCH_SIZE")
    write_scale = copy_kib / copy_mean(cwrite_d, "WRITE_SIZE")

    # expected dispatch sequence of one step (launch of each dispatch): the
    # GEMV kernel once per launch, the matrix-core kernels per matrix
    seq = [d[0] for d in plan["dispatches"]]
    per_launch = []
    for counter, d in (("FETCH_SIZE", fetch_d), ("WRITE_SIZE", write_d)):
        # GEMV / matrix-core dispatches only (the plane repack runs at load)
        ds = [x for x in _per_dispatch(d, counter)
              if x[0].startswith("qmv::") and "repack" not in x[0]]
        n_steps = len(ds) // len(seq)
        if n_steps * len(seq) != len(ds) or n_steps <= args.warmup:
            raise SystemExit(f"{counter}: {len(ds)} qmv dispatches, not a whole number of "
                             f"{len(seq)}-dispatch steps after {args.warmup} warmup steps")
        sums = [[0.0, 0, 0] for _ in groups]
        for i, (name, val, grid) in enumerate(ds):
            gi = seq[i % len(seq)]
            if name != kname[gi]:
                raise SystemExit(f"dispatch {i}: kernel {name!r}, expected {kname[gi]!r}")
            if i // len(seq) >= args.warmup:
                sums[gi][0] += val
                sums[gi][1] += 1
                sums[gi][2] = grid
        steps = n_steps - args.warmup
        for gi in range(len(groups)):
            if counter == "FETCH_SIZE":
                per_launch.append({"kernel": kname[gi], "launch": plan["launch_names"][gi],
                                   "grid": sums[gi][2]})
            per_launch[gi][counter.split("_")[0].lower() + "_kib"] = round(sums[gi][0] / steps, 3)
    for gi, pl in enumerate(per_launch):
        pl["fetch_bytes"] = round(pl["fetch_kib"] * 1024 * fetch_scale)
        pl["write_bytes"] = round(pl["write_kib"] * 1024 * write_scale)
        pl["algorithmic_bytes"] = int(gbytes[gi])
        pl["ratio"] = round((pl["fetch_bytes"] + pl["write_bytes"]) / gbytes[gi], 4)
    dom = plan["dom"]
    gis = plan["by_kernel"][dom]

    def avg(key):
        return sum(per_launch[gi][key] for gi in gis) / len(gis)
    rec = {"kernel": dom, "source_hash": kernel_source_hash(dom), "launches_per_step": len(gis),
           "hbm_bytes_per_launch": round(avg("fetch_bytes") + avg("write_bytes")),
           "fetch_bytes_per_launch": round(avg("fetch_bytes")),
           "write_bytes_per_launch": round(avg("write_bytes")),
           "algorithmic_bytes_per_launch": round(avg("algorithmic_bytes")),
           "fetch_scale": round(fetch_scale, 5), "write_scale": round(write_scale, 5),
           "per_launch": per_launch, "summary": args.summary_file}
    try:
        with open(COUNTERS_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        data = {}
    data[plan["workload"]] = rec
    with open(COUNTERS_FILE, "w") as fh:
        json.dump(data, fh, indent=1)
        fh.write("\n")
    print(f"scale: HBM bytes = {fetch_scale:.5f} x FETCH_SIZE x 1024 + {write_scale:.5f} x WRITE_SIZE x 1024")
    print("| kernel | launch | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes | algorithmic bytes | ratio |")
    print("|---|---|---:|---:|---:|---:|---:|")
    for pl in per_launch:
        print(f"| `{pl['kernel']}` | {pl['launch']} | {pl['fetch_kib']:.1f} | {pl['write_kib']:.1f} | "
              f"{pl['fetch_bytes'] + pl['write_bytes']} | {pl['algorithmic_bytes']} | {pl['ratio']:.3f} |")
    print(f"dominant `{dom}`: {rec['hbm_bytes_per_launch']} HBM bytes per launch, "
          f"{rec['algorithmic_bytes_per_launch']} algorithmic (ratio "
          f"{rec['hbm_bytes_per_launch'] / rec['algorithmic_bytes_per_launch']:.3f}); "
          f"source hash {rec['source_hash']}")
    return 0


def summarize_trace(args) -> int:
    """Kernel durations of a rocprofv3 --kernel-trace run of bench.py, per launch.

    The trace holds full steps, the timing replays restricted to one kernel's
    launches or to one launch, and load-time work.  The first full step in it
    fixes each dispatch's grid; the dispatches are then read in time order as
    a chain of those replays (at each point the replay just matched if it
    matches again, as a graph repeats one pattern, else the longest that
    matches by kernel name and grid), which assigns every dispatch to its
    matrix even where several matrices share a kernel and a grid (a run of
    replays that could be any of several goes to the one whose durations in
    the full steps are nearest).  Every dispatch of a
    step is summarized by count and median / mean / min duration; a launch
    takes the sum of its dispatches' medians.  For the dominant kernel these
    launch times are averaged with equal weight, as bench.py's per-kernel
    figure weighs every launch of a step once, and turned into the roofline
    fraction of the same algorithmic bytes or flops."""
    import csv
    import glob
    import statistics
    files = sorted(glob.glob(os.path.join(args.summarize_trace, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *kernel_trace.csv under {args.summarize_trace}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                name = kernel_display_name(r["Kernel_Name"])
                grid = (int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]))
                start = int(r["Start_Timestamp"])
                rows.append((start, name, grid, (int(r["End_Timestamp"]) - start) * 1e-3))  # ns -> us
    rows.sort()
    plan = workload_plan(args.config, args.batch, args.separate, _layout(args), args.x_dtype)
    disp = plan["dispatches"]
    step_names = [n for _, _, n in disp]
    toks = [(n, g, d) for _, n, g, d in rows if n in step_names]
    others = {}
    for _, n, g, d in rows:
        if n not in step_names and n.startswith("qmv::"):
            others.setdefault((n, g), []).append(d)
    first = next((i for i in range(len(toks) - len(disp) + 1)
                  if [t[0] for t in toks[i:i + len(disp)]] == step_names), None)
    if first is None:
        raise SystemExit("no full step in the trace")
    slot_tok = [(n, toks[first + si][1]) for si, n in enumerate(step_names)]
    pats = {tuple(range(len(disp)))}
    for gis in plan["by_kernel"].values():
        pats.add(tuple(si for si, d in enumerate(disp) if d[0] in gis))
    for gi in range(len(plan["groups"])):
        pats.add(tuple(si for si, d in enumerate(disp) if d[0] == gi))
    # replays whose dispatches look alike (say two matrices of one kernel and
    # grid, each timed alone) form one class; a run of such replays goes to
    # the member whose durations in the full steps are nearest
    classes = {}
    for pat in pats:
        classes.setdefault(tuple(slot_tok[si] for si in pat), []).append(pat)
    order = sorted(classes, key=len, reverse=True)
    durs = [[] for _ in disp]
    runs = []  # (class key, [dispatch durations per replay]) for ambiguous classes
    def matches(key, at):
        return at + len(key) <= len(toks) and all(toks[at + k][:2] == key[k] for k in range(len(key)))

    def continues(at):
        return at == len(toks) or any(matches(key, at) for key in order)

    p = unmatched = 0
    prev = None
    while p < len(toks):
        # a graph replays one pattern many times over: the pattern just seen
        # first, then the longest; a pattern is taken only if another (or the
        # end of the trace) follows it, so that the tail of one replay and the
        # head of the next are not read as a longer pattern
        cands = [c for c in ([prev] if prev else []) + order if matches(c, p)]
        key = next((c for c in cands if continues(p + len(c))), cands[0] if cands else None)
        if key is None:
            unmatched += 1
            p += 1
            prev = None
            continue
        prev = key
        ds = [toks[p + k][2] for k in range(len(key))]
        if len(classes[key]) == 1:
            for k, si in enumerate(classes[key][0]):
                durs[si].append(ds[k])
        elif runs and runs[-1][0] == key and runs[-1][2] == p:
            runs[-1][1].append(ds)
            runs[-1][2] = p + len(key)
        else:
            runs.append([key, [ds], p + len(key)])
        p += len(key)
    ref = [statistics.median(d) if d else None for d in durs]
    for key, reps, _ in runs:
        run_med = [statistics.median(r[k] for r in reps) for k in range(len(key))]

        def miss(pat):
            return sum(abs(run_med[k] / ref[si] - 1.0) if ref[si] else 1e9 for k, si in enumerate(pat))
        best = min(classes[key], key=miss)
        for r in reps:
            for k, si in enumerate(best):
                durs[si].append(r[k])
    names, mats = plan["names"], plan["mats"]
    print("| launch | matrix | kernel | grid (work-items) | dispatches | median us | mean us | min us |")
    print("|---|---|---|---|---:|---:|---:|---:|")
    launch_us = [0.0] * len(plan["groups"])
    for si, (gi, m, name) in enumerate(disp):
        d = durs[si]
        grid = slot_tok[si][1]
        med = statistics.median(d)
        launch_us[gi] += med
        mat = f"{names[m]} {mats[m][1]}x{mats[m][2]}" if m is not None else "all"
        print(f"| {plan['launch_names'][gi]} | {mat} | `{name}` | {grid[0]}x{grid[1]} | {len(d)} | {med:.3f} | "
              f"{statistics.mean(d):.3f} | {min(d):.3f} |")
    for (name, grid), d in sorted(others.items()):
        print(f"| (other) | | `{name}` | {grid[0]}x{grid[1]} | {len(d)} | {statistics.median(d):.3f} | "
              f"{statistics.mean(d):.3f} | {min(d):.3f} |")
    if unmatched:
        print(f"\n{unmatched} dispatches of these kernels matched no replay of the step and are left out.")
    dom = plan["dom"]
    gis = plan["by_kernel"][dom]
    nl = len(gis)
    avg = sum(launch_us[gi] for gi in gis) / nl
    bpl = sum(plan["gbytes"][gi] for gi in gis) / nl
    fpl = sum(plan["gflops"][gi] for gi in gis) / nl
    if plan["bound"][gis[0]] == "mfma":
        ach, peak, unit = fpl / (avg * 1e-6) / 1e12, PEAK_TFLOPS_BF16, "TFLOP/s"
    else:
        ach, peak, unit = bpl / (avg * 1e-6) / 1e9, PEAK_GBPS, "GB/s"
    print(f"\ndominant `{dom}`: {nl} launches per step, equal-weight mean of their durations (sums of their "
          f"dispatch medians) {avg:.3f} us; {bpl:.0f} algorithmic bytes and {fpl:.3e} flops per launch -> "
          f"{ach:.1f} {unit} = {ach / peak:.4f} of {peak:g}")
    return 0


SQ_DERIVED = ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16",
              "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU",
              "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAVES", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_VMEM_RD")


def summarize_sq(args) -> int:
    """Per-launch SQ counters of rocprofv3 --pmc runs of `bench.py --eager-pass`.

    Every directory given may hold one pass (a handful of SQ counters each).
    Values are summed over counter instances per dispatch and averaged over
    the timed steps (after --warmup).  Derived: VALU instructions per weight
    and lane (SQ_INSTS_VALU x 64 / weights: every wave instruction covers 64
    lanes), matrix-core operations against the launch's flops, and the
    fractions of wave cycles spent waiting (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES)
    and issuing VALU (SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES), VALU instructions
    per matrix-core instruction, and LDS bank-conflict cycles per LDS
    instruction."""
    plan = workload_plan(args.config, args.batch, args.separate, _layout(args), args.x_dtype)
    groups, kname = plan["groups"], plan["kname"]
    # launch of each dispatch of a step; only the kernel that names the
    # launch is counted (not the activation conversion or the partial sums)
    seq = [d[0] for d in plan["dispatches"]]
    counted = [d[2] == kname[d[0]] for d in plan["dispatches"]]
    vals = [{} for _ in groups]
    for d in args.summarize_sq:
        for counter in SQ_DERIVED:
            ds = [x for x in _per_dispatch_any(d, counter) if x[0].startswith("qmv::") and "repack" not in x[0]]
            if not ds:
                continue
            n_steps = len(ds) // len(seq)
            if n_steps * len(seq) != len(ds) or n_steps <= args.warmup:
                raise SystemExit(f"{d} {counter}: {len(ds)} qmv dispatches, not whole {len(seq)}-dispatch steps")
            acc = [0.0] * len(groups)
            for i, (name, val, _grid) in enumerate(ds):
                gi = seq[i % len(seq)]
                want = plan["dispatches"][i % len(seq)][2]
                if name != want:
                    raise SystemExit(f"dispatch {i}: kernel {name!r}, expected {want!r}")
                if i // len(seq) >= args.warmup and counted[i % len(seq)]:
                    acc[gi] += val
            steps = n_steps - args.warmup
            for gi in range(len(groups)):
                vals[gi][counter] = acc[gi] / steps
    print("| launch | kernel | " + " | ".join(c for c in SQ_DERIVED if any(c in v for v in vals))
          + " | VALU / weight / lane | wait / wave cycles | VALU issue / wave cycles | VALU / MFMA |"
          " LDS conflict cycles / LDS instruction |")
    cols = [c for c in SQ_DERIVED if any(c in v for v in vals)]
    print("|---|---|" + "---:|" * (len(cols) + 5))
    for gi, g in enumerate(groups):
        v = vals[gi]
        weights = sum(plan["mats"][m][1] * plan["mats"][m][2] for m in g)
        per_w = v["SQ_INSTS_VALU"] * 64 / weights if "SQ_INSTS_VALU" in v else float("nan")
        wait = v["SQ_WAIT_INST_ANY"] / v["SQ_WAVE_CYCLES"] if v.get("SQ_WAVE_CYCLES") and "SQ_WAIT_INST_ANY" in v else float("nan")
        act = v["SQ_ACTIVE_INST_VALU"] / v["SQ_WAVE_CYCLES"] if v.get("SQ_WAVE_CYCLES") and "SQ_ACTIVE_INST_VALU" in v else float("nan")
        per_mfma = v["SQ_INSTS_VALU"] / v["SQ_INSTS_MFMA"] if v.get("SQ_INSTS_MFMA") and "SQ_INSTS_VALU" in v else float("nan")
        conf = (v["SQ_LDS_BANK_CONFLICT"] / v["SQ_INSTS_LDS"]
                if v.get("SQ_INSTS_LDS") and "SQ_LDS_BANK_CONFLICT" in v else float("nan"))
        print(f"| {plan['launch_names'][gi]} | `{kname[gi]}` | " + " | ".join(f"{v.get(c, float('nan')):.4g}" for c in cols)
              + f" | {per_w:.3f} | {wait:.3f} | {act:.3f} | {per_mfma:.2f} | {conf:.2f} |")
    return 0


def _per_dispatch_any(d, counter):
    """_per_dispatch, or [] when the directory's runs hold no such counter."""
    try:
        return _per_dispatch(d, counter)
    except SystemExit:
        return []


def _layout(args) -> str:
    return (default_layout(args.config, args.batch, args.x_dtype) if args.layout == "auto"
            else args.layout)


# Batched workloads reported beside the decode line: (configuration, rows).
# Configuration 5 is the 7B FFN gate matrix (18944 x 3584), configuration 3
# the whole 7B decoder layer (its down projection is 3584 x 18944), both
# with bf16 rows here.
BATCHED_RUNS = [(5, 64), (5, 512), (3, 17), (3, 64), (3, 128), (3, 512)]


def batched_lines(args) -> list:
    """Time each batched workload in a child run of this script (one GPU
    process at a time) and keep the figures of its line: step time, launch
    times and the dominant kernel's roofline."""
    import subprocess
    out = []
    for config, batch in BATCHED_RUNS:
        cmd = [sys.executable, "-u", os.path.abspath(__file__), "--config", str(config), "--batch", str(batch),
               "--x-dtype", "bf16", "--steps", "50", "--warmup", "5", "--no-cpu-baseline", "--batched", "off",
               "--settle-ms", str(args.settle_ms), "--replays", str(args.replays)]
        print(f"batched workload: config {config}, {batch} bf16 rows", file=sys.stderr, flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
        if r.returncode != 0 or not lines:
            msg = f"exit {r.returncode}: {r.stderr[-1500:]}"
            print(f"batched workload failed: {msg}", file=sys.stderr, flush=True)
            out.append({"config": config, "batch": batch, "x_dtype": "bf16", "error": msg})
            continue
        d = json.loads(lines[-1])
        rf = d["roofline"]
        out.append({"workload": d["config"]["workload"], "batch": batch, "x_dtype": "bf16",
                    "layout": d["config"]["layout"], "launches": d["config"]["launches"],
                    "steps": d["steps"], "ms_per_step": d["ms_per_step"],
                    "per_launch_us": {k: v["us"] for k, v in (d["per_launch"] or {}).items()},
                    "roofline": {k: rf[k] for k in ("bound", "achieved", "peak", "unit", "frac", "kernel",
                                                    "avg_launch_us")}})
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5, 6])
    ap.add_argument("--batch", type=int, default=None,
                    help="activation rows (default: the configuration's; config 5 is quoted at 1, 4, 16, 64, 512)")
    ap.add_argument("--x-dtype", choices=["f32", "f16", "bf16"], default=None,
                    help="activation dtype in place of the configuration's (same seeded values)")
    ap.add_argument("--rotate-gib", type=float, default=1.25)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed graph replays before each timed one (steady-state clocks)")
    ap.add_argument("--cpu-sample-rows", type=int, default=2048,
                    help="rows of each matrix the CPU oracle baseline times")
    ap.add_argument("--replays", type=int, default=11,
                    help="timed graph replays per region; the median is reported")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate", action="store_true", help="one launch per matrix")
    ap.add_argument("--layout", choices=["auto", "blocks", "planes"], default="auto",
                    help="weight layout in HBM (auto: planes for Q4_K, Q5_K and Q6_K on the GEMV path, else blocks)")
    ap.add_argument("--eager-pass", action="store_true",
                    help="only issue warmup + steps eagerly (no graphs, no timing): for counter runs")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 --pmc output dirs of the eager pass (same --config/--batch/"
                         "--separate/--warmup) and of the probe copy: write profiles/counters.json")
    ap.add_argument("--copy-mib", type=int, default=256, help="size of the calibration copy")
    ap.add_argument("--summary-file", default="", help="profiles/ summary recorded with the counters")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="rocprofv3 --kernel-trace output dir of a bench.py run: per-launch durations "
                         "(grouped by kernel and grid) and the dominant kernel's roofline fraction")
    ap.add_argument("--summarize-sq", nargs="+", metavar="DIR",
                    help="rocprofv3 --pmc output dirs (SQ counters) of the eager pass: per-launch table")
    ap.add_argument("--batched", choices=["auto", "on", "off"], default="auto",
                    help="also time the batched bf16 workloads (the FFN gate at 64 and 512 rows, the "
                         "layer at 17, 64, 128 and 512 rows), each in a child run before this one, and add "
                         "their figures to the line as \"batched\" (auto: for the default workload)")
    args = ap.parse_args()
    if args.summarize_counters:
        return summarize_counters(args)
    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_sq:
        return summarize_sq(args)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single GPU: this library has no multi-GPU path (over P GPUs "
              "each would hold rows/P of every matrix, take the whole activation and all-gather "
              "y). Run with --gpus 1.", file=sys.stderr)
        return 2

    batched = None
    default_run = (args.config == 3 and args.batch is None and args.x_dtype is None and not args.separate
                   and not args.eager_pass and args.layout == "auto")
    if args.batched == "on" or (args.batched == "auto" and default_run):
        batched = batched_lines(args)  # child runs first: this process has not touched the GPU yet

    import numpy as np
    import torch

    from block_quantized_weight_qmv_amd import qmv
    from synth import CONFIGS, gen_weights, gen_x, weight_seed, x_seed

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layout = _layout(args)
    plan = workload_plan(args.config, args.batch, args.separate, layout, args.x_dtype)
    cfg, fmt, x_dtype, batch = plan["cfg"], plan["fmt"], plan["x_dtype"], plan["batch"]
    mats, names, groups = plan["mats"], plan["names"], plan["groups"]
    gbytes, gflops, kname, by_kernel, dom = (plan["gbytes"], plan["gflops"], plan["kname"],
                                             plan["by_kernel"], plan["dom"])
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[x_dtype]

    # -- inputs: synthesize, pack on the host with the library packer, upload ---
    fields_list, packed_dev, xs, xs_dev, ys = [], [], [], [], []
    leader = {m: g[0] for g in groups for m in g}
    for i, (name, rows, cols) in enumerate(mats):
        f = gen_weights(fmt, rows, cols, weight_seed(args.config, i))
        fields_list.append(f)
        packed_dev.append(torch.from_numpy(qmv.pack_fields(fmt, f, rows, cols)).to(dev))
        if leader[i] == i:
            x = gen_x(batch, cols, x_dtype, x_seed(args.config, i))
            xt = torch.from_numpy(x.view(np.int16) if x_dtype == "bf16" else x).to(dev)
            xs.append(x)
            xs_dev.append(xt.view(tdt) if x_dtype == "bf16" else xt)
        else:  # same activation as the group's first matrix
            xs.append(xs[leader[i]])
            xs_dev.append(xs_dev[leader[i]])
        ys.append(torch.empty(batch, rows, dtype=torch.float32, device=dev))
    step_w_bytes = sum(plan["wbytes"])
    step_bytes = sum(gbytes)
    copies = max(1, int(np.ceil(args.rotate_gib * 2 ** 30 / step_w_bytes)))
    descs = []  # descs[c][m]
    keep = []
    for c in range(copies):
        row = []
        for m, (name, rows, cols) in enumerate(mats):
            t = packed_dev[m] if c == 0 else packed_dev[m].clone()
            d = qmv.qmv_create_weights(fmt, rows, cols, t)
            if layout == "planes":  # repacked once, at load; the planes replace the blocks
                planes = torch.empty(plan["wbytes"][m], dtype=torch.uint8, device=dev)
                d = qmv.qmv_repack_planes(d, planes)
                torch.cuda.synchronize()
                t = planes
            keep.append(t)
            row.append(d)
        descs.append(row)
    if layout == "planes":
        del packed_dev
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    # one workspace for every launch of the step (they run in stream order),
    # sized for the launch that needs the most; allocated before any capture
    ws_bytes = max(qmv.qmv_workspace_size(fmt, x_dtype, batch,
                                          [(descs[0][m], xs_dev[m], ys[m]) for m in g])
                   for g in groups)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def launch(c, g, sptr):
        qmv.qmv_gemv_multi_ws(fmt, x_dtype, batch, [(descs[c][m], xs_dev[m], ys[m]) for m in g],
                              ws, ws_bytes, sptr)

    # dominant kernel (plan["dom"]): the instantiation with the most algorithmic
    # bytes per step

    for s in range(args.warmup):
        for g in groups:
            launch(s % copies, g, sp)
    torch.cuda.synchronize()
    if args.eager_pass:
        for s in range(args.steps):
            for g in groups:
                launch((args.warmup + s) % copies, g, sp)
        torch.cuda.synchronize()
        print(json.dumps({"eager_pass": cfg["name"], "steps": args.steps, "warmup": args.warmup,
                          "launches": ["+".join(names[m] for m in g) for g in groups],
                          "kernels": kname}), flush=True)
        return 0

    # -- timed regions: HIP-graph replays ------------------------------------------
    # Launching from Python costs more than these kernels run, so every timed
    # region is captured once as a graph and replayed; events on the replay stream
    # bracket the replay.  (1) K whole steps -> ms_per_step.  (2) per kernel
    # instantiation, the same K steps restricted to that kernel's launches, so the
    # rotation over weight copies and the launch order are unchanged -> its average
    # launch duration (the duration plus the small gap between graph nodes).
    cap = torch.cuda.Stream(dev)
    spread = []   # (min, median, max) ms of each timed region's replays

    def timed_graph(gis, fn=None):
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            for s in range(args.steps):
                c = (args.warmup + s) % copies
                if fn is not None:
                    fn(c, cap.cuda_stream)
                for gi in gis:
                    launch(c, groups[gi], cap.cuda_stream)
        g.replay()                    # untimed: first-touch costs
        torch.cuda.synchronize()
        # untimed replays for --settle-ms: the first timed region otherwise runs
        # before the clocks settle under load (a single-launch step measured
        # 92 us in the first graph and 80 us in the next, same kernel)
        t_end = time.perf_counter() + args.settle_ms * 1e-3
        while time.perf_counter() < t_end:
            g.replay()
            torch.cuda.synchronize()
        # median of --replays timed replays, each bracketed by events on the
        # replay stream (the current stream) and a synchronize on both sides
        times = []
        for _ in range(args.replays):
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0.record(stream)
            g.replay()
            t1.record(stream)
            torch.cuda.synchronize()
            times.append(t0.elapsed_time(t1))
        times.sort()
        spread.append((times[0], times[len(times) // 2], times[-1]))
        return times[len(times) // 2]

    total_ms = timed_graph(list(range(len(groups))))
    ms_per_step = total_ms / args.steps
    step_spread = [round(v / args.steps, 5) for v in spread[-1]]
    kern = {}
    for k, gis in by_kernel.items():
        el = timed_graph(gis)
        kern[k] = {"launches": ["+".join(names[m] for m in groups[gi]) for gi in gis],
                   "launches_per_step": len(gis),
                   "avg_launch_us": round(el * 1e3 / (args.steps * len(gis)), 3),
                   "avg_launch_us_min_max": [round(spread[-1][0] * 1e3 / (args.steps * len(gis)), 3),
                                             round(spread[-1][2] * 1e3 / (args.steps * len(gis)), 3)],
                   "bytes_per_launch": sum(gbytes[gi] for gi in gis) / len(gis)}
        kern[k]["GBps"] = round(kern[k]["bytes_per_launch"] / (kern[k]["avg_launch_us"] * 1e-6) / 1e9, 1)
    if not args.separate or len(groups) > 1:
        per_launch = {}
        for gi, g in enumerate(groups):
            el = timed_graph([gi])
            us = el * 1e3 / args.steps
            per_launch["+".join(names[m] for m in g)] = {
                "us": round(us, 3), "GBps": round(gbytes[gi] / (us * 1e-6) / 1e9, 1),
                "us_min_max": [round(spread[-1][0] * 1e3 / args.steps, 3),
                               round(spread[-1][2] * 1e3 / args.steps, 3)]}
    else:
        per_launch = None
    # The SwiGLU epilogue: gate and up as one launch writing silu(g) * u
    # (qmv_gemv_swiglu), against the unfused gate+up launch above (decode
    # steps, one activation row).
    fused = None
    if "gate" in names and "up" in names and not args.separate and batch == 1:
        mg, mu = names.index("gate"), names.index("up")
        _, grows, gcols = mats[mg]
        if gcols <= (2048 if fmt == "q8_0" else 4096):
            hbuf = torch.empty(batch, grows, dtype=torch.float32, device=dev)

            def swiglu_launch(c, sptr):
                qmv.qmv_gemv_swiglu(fmt, descs[c][mg], descs[c][mu], xs_dev[mg], x_dtype, hbuf,
                                    grows, gcols, batch, sptr)
            el = timed_graph([], swiglu_launch)
            us = el * 1e3 / args.steps
            gb = gbytes[[i for i, g in enumerate(groups) if mg in g][0]]
            fused = {"launch": "gate+up -> silu(gate) * up", "us": round(us, 3),
                     "GBps": round((gb - batch * grows * 4) / (us * 1e-6) / 1e9, 1),
                     "us_min_max": [round(spread[-1][0] * 1e3 / args.steps, 3),
                                    round(spread[-1][2] * 1e3 / args.steps, 3)],
                     "unfused_gate_up_us": (per_launch or {}).get("gate+up", {}).get("us")}
    dom_avg_us = kern[dom]["avg_launch_us"]
    dom_bytes_per_launch = kern[dom]["bytes_per_launch"]
    dom_flops_per_launch = sum(gflops[gi] for gi in by_kernel[dom]) / len(by_kernel[dom])
    dom_bound = plan["bound"][by_kernel[dom][0]]
    if dom_bound == "mfma":
        achieved, peak, unit = dom_flops_per_launch / (dom_avg_us * 1e-6) / 1e12, PEAK_TFLOPS_BF16, "TFLOP/s"
    else:
        achieved, peak, unit = dom_bytes_per_launch / (dom_avg_us * 1e-6) / 1e9, PEAK_GBPS, "GB/s"
    detail = kern

    # -- HBM read ceiling on this GPU (nontemporal 128-bit streaming read of 2 GiB) ------
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

    workload = plan["workload"]
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    rec = {
        "metric": "achieved HBM GB/s (% of peak) and µs per GEMV, batch-1 7B-shaped Q4_K",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_min_median_max": step_spread,
        "timed_replays": args.replays,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "fp32", "f16": "fp16", "bf16": "bf16"}[x_dtype],
        "data": "synthetic",
        "config": {"workload": workload, "format": fmt, "layout": layout, "batch": batch, "x_dtype": x_dtype,
                   "matrices": {n: f"{r}x{c}" for n, r, c in mats},
                   "launches": ["+".join(names[m] for m in g) for g in groups],
                   "bytes_per_step": int(step_bytes), "weight_copies": copies},
        "pct_of_peak": round(100 * value / PEAK_GBPS, 1),
        "us_per_gemv": round(ms_per_step * 1e3 / len(mats), 3),
        "per_kernel": detail,
        "per_launch": per_launch,
        "read_ceiling_GBps": round(read_ceiling, 1),
        "pct_of_read_ceiling": round(100 * value / read_ceiling, 1),
        "roofline": {"bound": dom_bound, "achieved": round(achieved, 1), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(dom, workload),
                     "kernel": dom, "avg_launch_us": round(dom_avg_us, 3),
                     "launches_per_step": len(by_kernel[dom]),
                     "timing": "median of the HIP-event times of "
                               f"{args.replays} graph replays of the K steps restricted to "
                               "this kernel's launches, on the replay stream, after "
                               f"{args.settle_ms:g} ms of untimed replays",
                     "bytes_per_launch": round(dom_bytes_per_launch, 1),
                     "flops_per_launch": round(dom_flops_per_launch, 1)},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(mats, fmt, x_dtype, fields_list, xs, args.cpu_sample_rows)
    if fused is not None:
        rec["swiglu_fused"] = fused
    if batched is not None:
        rec["batched"] = batched
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
