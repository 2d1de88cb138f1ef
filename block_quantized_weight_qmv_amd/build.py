"""Build libqmv.so in-tree with hipcc for gfx950 (no JIT, no torch extension).

Usage: python -m block_quantized_weight_qmv_amd.build [-v]
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqmv.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
# Device code: gfx950 only; packed-fp32 VALU forms are disabled (the host pass
# warns that it does not know the feature, which is harmless).
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

HIP_SOURCES = ["api.cpp", "gemv_q8_0.hip", "gemv_q4_k.hip", "gemv_q5_k.hip", "gemv_q6_k.hip",
               "gemv_int4_g128.hip", "gemm_q4_k_mfma.hip", "gemm_q4_k_dqreg.hip", "dequant.hip", "repack.hip", "probe.hip"]
CXX_SOURCES = ["packer.cpp"]
# Per-source device flags.  The matrix-core kernels scale each product in
# VALU right away; in accumulation registers every result would need a
# v_accvgpr_read first, so their results are kept in ordinary VGPRs.
SOURCE_FLAGS = {"gemm_q4_k_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link libqmv.so; returns the library path."""
    os.makedirs(OBJDIR, exist_ok=True)
    cmds, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(OBJDIR, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmds.append([HIPCC] + COMMON + DEVICE + SOURCE_FLAGS.get(src, []) + lang +
                    ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(OBJDIR, src + ".o")
        cmds.append(["g++"] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    jobs = jobs or min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
