"""bench.py's host-side bookkeeping (CPU only).

* The kernel instantiation bench.py names for each workload (the key of its
  per-kernel timings and of the committed counter figures) must exist in the
  built library -- it mirrors the launcher's routing, and this catches drift.
* Algorithmic bytes per launch = packed weights + each activation once + y,
  with packed sizes from the library; flops = 2 batch rows cols.
* More than one GPU is refused with an explanation.
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_quantized_weight_qmv_amd import qmv  # noqa: E402
from synth import CONFIGS  # noqa: E402

CASES = [(c, b) for c, cfg in CONFIGS.items() for b in cfg["batch"]] + [(5, 3), (5, 17), (5, 33), (5, 65)]


def _library_kernels():
    if shutil.which("nm") is None or not os.path.exists(qmv.LIB_PATH):
        pytest.skip("nm or the built library is not available")
    out = subprocess.run(["nm", "-C", qmv.LIB_PATH], capture_output=True, text=True, check=True).stdout
    names = set()
    # this nm leaves the _Float16 instantiations mangled
    f16 = re.compile(r"_ZN3qmv11gemv_kernelINS_\d+(\w+?)EDF16_Li(\d+)ELi(\d+)ELi(\d+)ELb([01])EEEvNS_10GemvLaunchE")
    f16_rows = re.compile(r"_ZN3qmv16gemv_rows_kernelINS_\d+(\w+?)EDF16_Li(\d+)ELi(\d+)ELi(\d+)ELi(\d+)EEEvNS_10GemvLaunchEi")
    f16_split = re.compile(r"_ZN3qmv22gemv_rows_split_kernelINS_\d+(\w+?)EDF16_Li(\d+)ELi(\d+)ELi(\d+)EEEvNS_10GemvLaunchEi")
    f16_lx = re.compile(r"_ZN3qmv14gemv_lx_kernelINS_\d+(\w+?)EDF16_Li(\d+)ELi(\d+)ELi(\d+)EEEvNS_10GemvLxArgsE")
    f16_pair = re.compile(r"_ZN3qmv16gemv_pair_kernelINS_\d+(\w+?)EDF16_Li(\d+)EEEvNS_10GemvLaunchE")
    for line in out.splitlines():
        m = f16.search(line)
        if m:
            sx = "true" if m.group(5) == "1" else "false"
            names.add(f"qmv::gemv_kernel<qmv::{m.group(1)}, _Float16, {m.group(2)}, {m.group(3)}, {m.group(4)}, {sx}>")
            continue
        m = f16_split.search(line)
        if m:
            names.add(f"qmv::gemv_rows_split_kernel<qmv::{m.group(1)}, _Float16, {m.group(2)}, {m.group(3)}, "
                      f"{m.group(4)}>")
            continue
        m = f16_lx.search(line)
        if m:
            names.add(f"qmv::gemv_lx_kernel<qmv::{m.group(1)}, _Float16, {m.group(2)}, {m.group(3)}, {m.group(4)}>")
            continue
        m = f16_pair.search(line)
        if m:
            names.add(f"qmv::gemv_pair_kernel<qmv::{m.group(1)}, _Float16, {m.group(2)}>")
            continue
        m = f16_rows.search(line)
        if m:
            names.add(f"qmv::gemv_rows_kernel<qmv::{m.group(1)}, _Float16, {m.group(2)}, {m.group(3)}, "
                      f"{m.group(4)}, {m.group(5)}>")
            continue
        if ("qmv::gemv_kernel<" in line or "qmv::gemv_rows_kernel<" in line or "qmv::gemv_rows_split_kernel<" in line
                or "qmv::gemv_lx_kernel<" in line or "qmv::gemv_pair_kernel<" in line
                or "qmv::gemm_q4_k_bf16_" in line or "qmv::gemm_q4_k_stream<" in line
                or "qmv::gemm_q4_k_tile<" in line or "qmv::gemm_q4_k_ksplit<" in line
                or "qmv::act_rows_f16<" in line or "qmv::gemm_q4_k_dqreg<" in line or "qmv::dqreg_sum" in line):
            sym = line.split(" ", 2)[2]
            sym = sym[5:] if sym.startswith("void ") else sym
            names.add(sym.split("(")[0])
    return names


def _layouts(config, batch):
    """The layout bench.py uses by default, and the canonical blocks."""
    return sorted({bench.default_layout(config, batch), "blocks"})


@pytest.mark.parametrize("config,batch", CASES)
def test_named_kernel_exists_in_library(config, batch):
    names = _library_kernels()
    for layout in _layouts(config, batch):
        plan = bench.workload_plan(config, batch, separate=False, layout=layout)
        for k in plan["kname"]:
            assert k in names, (k, sorted(n for n in names if k.split("<")[0] in n))


def test_default_layout():
    assert bench.default_layout(3, None) == "planes"
    assert bench.default_layout(5, 1) == "planes"
    assert bench.default_layout(5, 4) == "planes"       # multi-row GEMV
    assert bench.default_layout(5, 16) == "blocks"      # matrix cores: blocks stream faster
    assert bench.default_layout(4, None) == "planes"
    assert bench.default_layout(6, None) == "planes"
    for c in (1, 2):
        assert bench.default_layout(c, None) == "blocks"


@pytest.mark.parametrize("config,batch", CASES)
def test_algorithmic_bytes_and_flops(config, batch):
    for layout in _layouts(config, batch):
        _check_bytes_and_flops(config, batch, layout)


def _check_bytes_and_flops(config, batch, layout):
    plan = bench.workload_plan(config, batch, separate=False, layout=layout)
    size = qmv.qmv_planes_size if layout == "planes" else qmv.qmv_packed_size
    xb = {"f32": 4, "f16": 2, "bf16": 2}[plan["x_dtype"]]
    mats = plan["mats"]
    for gi, g in enumerate(plan["groups"]):
        w = sum(size(plan["fmt"], mats[m][1], mats[m][2]) for m in g)
        y = sum(batch * mats[m][1] * 4 for m in g)
        x = batch * mats[g[0]][2] * xb           # one activation per launch
        assert all(mats[m][2] == mats[g[0]][2] for m in g)
        assert plan["gbytes"][gi] == w + x + y
        assert plan["gflops"][gi] == sum(2.0 * batch * mats[m][1] * mats[m][2] for m in g)
    assert plan["dom"] in plan["kname"]


def test_decode_groups_share_activations():
    assert bench.decode_groups(["q", "k", "v", "o", "gate", "up", "down"]) == [[0, 1, 2], [3], [4, 5], [6]]
    assert bench.decode_groups(["gate", "up", "down"]) == [[0, 1], [2]]
    assert bench.decode_groups(["w"]) == [[0]]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "single GPU" in r.stderr


@pytest.mark.parametrize("config,batch,x_dtype", [(2, 4, None), (2, 3, "bf16"), (4, 4, "bf16"), (4, 2, "f16"),
                                                  (3, 2, "f16"), (5, 4, "f16"), (1, 4, "f16"),
                                                  (1, 2, "bf16"), (3, 2, None), (4, 4, None), (5, 3, "f32")])
def test_small_batch_overrides_name_library_kernels(config, batch, x_dtype):
    # --batch on any configuration and --x-dtype: the multi-row GEMV for the
    # formats that have one, named as the library exports it
    names = _library_kernels()
    layout = bench.default_layout(config, batch, x_dtype)
    plan = bench.workload_plan(config, batch, separate=False, layout=layout, x_dtype=x_dtype)
    assert plan["x_dtype"] == (x_dtype or CONFIGS[config]["x_dtype"])
    for k, g in zip(plan["kname"], plan["groups"]):
        assert k in names, k
    multi = [k for k in plan["kname"] if "gemv_rows_kernel" in k or "gemv_rows_split_kernel" in k]
    assert multi, plan["kname"]


@pytest.mark.parametrize("config,batch,x_dtype", [(2, 2, None), (6, 2, "bf16"), (6, 4, "f16"), (3, 2, "f16"),
                                                  (2, 8, "bf16")])
def test_split_k_small_batches_name_the_split_kernel(config, batch, x_dtype):
    # the down projections (several waves along K) take the K-split form
    names = _library_kernels()
    layout = bench.default_layout(config, batch, x_dtype)
    plan = bench.workload_plan(config, batch, separate=False, layout=layout, x_dtype=x_dtype)
    split = [k for k in plan["kname"] if "gemv_rows_split_kernel" in k]
    assert split and all(k in names for k in split), plan["kname"]


@pytest.mark.parametrize("batch,kernel", [(5, "qmv::gemm_q4_k_stream<false, true>"),
                                          (16, "qmv::gemm_q4_k_stream<false, true>"),
                                          (17, "qmv::gemm_q4_k_tile<1, 1, 2, 5, false, true>"),
                                          (64, "qmv::gemm_q4_k_tile<1, 2, 2, 5, false, true>"),
                                          (65, "qmv::gemm_q4_k_dqreg<"),
                                          (128, "qmv::gemm_q4_k_dqreg<"),
                                          (512, "qmv::gemm_q4_k_dqreg<")])
def test_q4_k_f16_batches_name_the_f16_matrix_core_kernels(batch, kernel):
    # Q4_K x fp16 from 5 rows: the matrix cores with fp16 operands (from 65
    # rows the register-dequantized kernels, in the form the plan picks)
    names = _library_kernels()
    layout = bench.default_layout(5, batch, "f16")
    assert layout == "blocks"
    plan = bench.workload_plan(5, batch, separate=False, layout=layout, x_dtype="f16")
    assert len(plan["kname"]) == 1 and plan["kname"][0].startswith(kernel)
    assert all(d[2] in names for d in plan["dispatches"]), plan["dispatches"]


@pytest.mark.parametrize("config,batch,kernel", [(3, 8, "qmv::gemm_q4_k_ksplit<1, 1, false, true>"),
                                                 (3, 16, "qmv::gemm_q4_k_ksplit<1, 1, false, true>")])
def test_q4_k_f16_wide_batches_name_the_f16_ksplit_kernel(config, batch, kernel):
    # the 7B layer's down projection (K = 18944) at 5-16 fp16 rows: the K-split
    # matrix-core kernel with fp16 operands
    names = _library_kernels()
    plan = bench.workload_plan(config, batch, separate=False, layout="blocks", x_dtype="f16")
    assert plan["kname"][-1] == kernel and kernel in names


@pytest.mark.parametrize("x_dtype,batch", [("bf16", 8), ("f16", 16)])
def test_small_multi_matrix_batches_name_the_rows_kernel(x_dtype, batch):
    # the 7B layer's q+k+v (4608 rows in three matrices) at 5-16 rows: one
    # multi-row launch; o (one matrix) stays on the matrix cores
    names = _library_kernels()
    plan = bench.workload_plan(3, batch, separate=False, layout="planes", x_dtype=x_dtype)
    qkv, o = plan["kname"][0], plan["kname"][1]
    assert qkv.startswith("qmv::gemv_rows_kernel<") and qkv in names, qkv
    assert o.startswith("qmv::gemm_q4_k_"), o


@pytest.mark.parametrize("rows,cols,batch", [(18944, 3584, 512), (3584, 18944, 512), (3584, 3584, 512),
                                             (512, 3584, 512), (18944, 3584, 128), (3584, 18944, 64),
                                             (300, 768, 400), (4100, 512, 1000), (30001, 256, 500)])
def test_dqreg_plan_is_well_formed(rows, cols, batch):
    # the launcher's model (mirrored here for naming): a built form, slices
    # that cover K with at least one block each
    t, nbt, splits, bps = bench.dqreg_plan(rows, cols, batch)
    nb = cols // 256
    assert 1 <= t <= 5 and nbt in (4, 8) and 1 <= splits <= 8
    assert (splits - 1) * bps < nb <= splits * bps
    assert splits == -(-nb // bps)


@pytest.mark.parametrize("mats,batch,run", [([(18944, 3584)], 64, 0), ([(3584, 18944)], 64, 1),
                                           ([(18944, 3584)], 128, 1), ([(300, 768)], 400, 1),
                                           ([(255, 3584)], 512, 0), ([(3584, 18944)], 17, 1),
                                           ([(3584, 18944)], 16, 0), ([(3584, 8192)], 64, 1),
                                           ([(3584, 7936)], 64, 0), ([(18944, 3584)] * 2, 32, 2),
                                           ([(3584, 3584), (512, 3584), (512, 3584)], 64, 3),
                                           ([(3584, 3584), (255, 3584), (512, 3584)], 64, 0),
                                           ([(3584, 3584), (255, 3584), (512, 3584)], 128, 1),
                                           ([(3584, 3584)] * 5, 256, 4), ([(3584, 3584), (3584, 1024)], 64, 0),
                                           ([(18944, 3584)], 65, 1), ([(3584, 3584), (3584, 1024)], 96, 1)])
def test_dq_run(mats, batch, run):
    # runs of up to four matrices of one width from 17 rows, a lone matrix
    # from 65 rows (from 17 against 8192 columns and more), matrices of 256
    # rows and more
    assert bench.dq_run(mats, batch, "blocks") == run
