"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

api.cpp (validation, routing, status text) and packer.cpp (the block packers)
are rebuilt with host-side ASan + UBSan instrumentation (device code is not
instrumented; -Xarch_host keeps the sanitizers off the gfx950 pass) and
linked with the ordinary objects of the kernel sources.  The ABI and packer
suites then run in a child process against that build, with the sanitizer
runtime preloaded and every report fatal."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from block_quantized_weight_qmv_amd import build as B  # noqa: E402

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_and_packer_suites_under_asan_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None or not os.path.exists(B.HIPCC):
        pytest.skip("no clang ASan runtime or hipcc in this image")
    kernel_objs = [os.path.join(B.OBJDIR, s + ".o") for s in B.HIP_SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in kernel_objs):
        B.build()
    objs = []
    for src in ("api.cpp", "packer.cpp"):
        obj = str(tmp_path / (src + ".o"))
        B._run([B.HIPCC, "-O1", "-g", "-fPIC", "-std=c++17", f"-I{B.INCLUDE}", f"-I{B.CSRC}"] + B.DEVICE
               + SAN + ["-x", "hip", "-c", os.path.join(B.CSRC, src), "-o", obj], False)
        objs.append(obj)
    lib = str(tmp_path / "libqmv_asan.so")
    B._run([B.HIPCC, "-shared", "-fPIC", f"--offload-arch={B.ARCH}"] + SAN + ["-shared-libasan", "-o", lib]
           + objs + kernel_objs, False)
    env = dict(os.environ, QMV_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
    # the child really runs the instrumented build
    probe = ("from block_quantized_weight_qmv_amd import qmv; qmv.lib(); "
             "m = open('/proc/self/maps').read(); "
             f"assert {lib!r} in m and 'libclang_rt.asan' in m, 'sanitized library not mapped'")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "tests/test_packer.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout
