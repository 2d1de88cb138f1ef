"""The C ABI without a GPU: library loads, exports what include/qmv.h declares,
and every validation error is raised before any HIP call."""
import os
import re

import numpy as np
import pytest

from block_quantized_weight_qmv_amd import qmv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmv.h")

FAKE = 0x7F0000000000  # a 16-byte aligned address; never dereferenced by these tests


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmv_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = qmv.lib()
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(qmv.EXPORTED) == names


def test_block_and_packed_sizes():
    assert [qmv.qmv_block_size(f) for f in ("q8_0", "q4_k", "q6_k", "int4_g128", "q5_k")] == [32, 256, 256, 128, 256]
    assert qmv.qmv_block_size(0) == 0 and qmv.qmv_block_size(6) == 0
    assert qmv.qmv_packed_size("q8_0", 1536, 1536) == 2_506_752
    assert qmv.qmv_packed_size("q4_k", 18944, 3584) == 38_191_104
    assert qmv.qmv_packed_size("q6_k", 152064, 3584) == 447_068_160
    assert qmv.qmv_packed_size("int4_g128", 3584, 18944) == 35_008_512
    assert qmv.qmv_packed_size("q5_k", 3584, 18944) == 46_678_016
    for bad in [(0, 256), (1, 0), (1, 255), (-1, 256)]:
        assert qmv.qmv_packed_size("q4_k", *bad) == 0


def _desc(fmt="q4_k", rows=8, cols=512, ptr=FAKE):
    return qmv.qmv_create_weights(fmt, rows, cols, ptr, qmv.qmv_packed_size(fmt, rows, cols))


def _expect(status, fn, *args):
    with pytest.raises(qmv.QmvError) as e:
        fn(*args)
    assert e.value.status == status, str(e.value)
    assert qmv.qmv_last_error() != ""


def test_create_weights_errors():
    n = qmv.qmv_packed_size("q4_k", 8, 512)
    _expect(-1, qmv.qmv_create_weights, "q4_k", 8, 512, None, n)
    _expect(-2, qmv.qmv_create_weights, 9, 8, 512, FAKE, n)
    _expect(-3, qmv.qmv_create_weights, "q4_k", 8, 500, FAKE, n)
    _expect(-3, qmv.qmv_create_weights, "q4_k", 0, 512, FAKE, n)
    _expect(-5, qmv.qmv_create_weights, "q4_k", 8, 512, FAKE, n + 1)
    _expect(-4, qmv.qmv_create_weights, "q4_k", 8, 512, FAKE + 2, n)
    w = _desc("int4_g128", 4, 256)
    assert w.scales_offset == 4 * 256 // 2 and w.fmt == 4 and w.nbytes == 4 * 128 + 4 * 2 * 2
    assert _desc().scales_offset == 0


def test_gemv_validation_errors():
    w = _desc()
    g = qmv.qmv_gemv
    _expect(-1, g, "q4_k", w, None, "f32", FAKE, 8, 512, 1)
    _expect(-1, g, "q4_k", w, FAKE, "f32", None, 8, 512, 1)
    _expect(-2, g, "q6_k", w, FAKE, "f32", FAKE, 8, 512, 1)     # fmt disagrees
    _expect(-2, g, "q4_k", w, FAKE, "f32", FAKE, 9, 512, 1)     # rows disagree
    _expect(-2, g, "q4_k", w, FAKE, "f32", FAKE, 8, 256, 1)     # cols disagree
    _expect(-3, g, "q4_k", w, FAKE, "f32", FAKE, 8, 512, 0)     # batch < 1
    _expect(-6, g, "q4_k", w, FAKE, 7, FAKE, 8, 512, 1)         # dtype
    _expect(-4, g, "q4_k", w, FAKE + 4, "f32", FAKE, 8, 512, 1)
    _expect(-4, g, "q4_k", w, FAKE, "f32", FAKE + 8, 8, 512, 1)
    _expect(-6, g, "q4_k", w, FAKE, "f32", FAKE, 8, 512, 70000)  # batch above the limit
    big = _desc("q4_k", 1, 256 * 300)
    _expect(-6, g, "q4_k", big, FAKE, "f32", FAKE, 1, 256 * 300, 1)
    # a tampered descriptor is caught
    bad = _desc()
    bad.nbytes += 144
    _expect(-5, g, "q4_k", bad, FAKE, "f32", FAKE, 8, 512, 1)
    bad = _desc()
    bad.data = None
    _expect(-1, g, "q4_k", bad, FAKE, "f32", FAKE, 8, 512, 1)
    bad = _desc("int4_g128", 4, 256)
    bad.scales_offset = 0
    _expect(-2, g, "int4_g128", bad, FAKE, "f32", FAKE, 4, 256, 1)


def test_gemv_multi_validation_errors():
    a, b = _desc(), _desc("q4_k", 16, 512)
    m = qmv.qmv_gemv_multi
    Y2 = FAKE + 4096
    _expect(-3, m, "q4_k", "f32", 1, [])                                   # no items
    _expect(-6, m, "q4_k", "f32", 1, [(a, FAKE, FAKE + 64 * i) for i in range(17)])
    _expect(-2, m, "q6_k", "f32", 1, [(a, FAKE, FAKE)])                    # format differs
    _expect(-2, m, 9, "f32", 1, [(a, FAKE, FAKE)])
    _expect(-3, m, "q4_k", "f32", 1, [(a, FAKE, FAKE), (b, FAKE, FAKE + 16)])  # y overlap
    _expect(-4, m, "q4_k", "f32", 1, [(a, FAKE, FAKE), (b, FAKE + 2, Y2)])
    _expect(-1, m, "q4_k", "f32", 1, [(a, FAKE, FAKE), (b, None, Y2)])
    _expect(-6, m, "q4_k", 3, 1, [(a, FAKE, FAKE)])
    _expect(-3, m, "q4_k", "f32", 0, [(a, FAKE, FAKE)])
    bad = _desc()
    bad.nbytes = 1
    _expect(-5, m, "q4_k", "f32", 1, [(a, FAKE, FAKE), (bad, FAKE, Y2)])


def test_workspace_size_and_caller_workspace_errors():
    """qmv_workspace_size needs no GPU; qmv_gemv_multi_ws refuses a missing,
    misaligned or too small workspace before any HIP call."""
    gate = _desc("q4_k", 18944, 3584)
    down = _desc("q4_k", 3584, 18944)
    small = _desc("q4_k", 64, 3584)
    Y2 = FAKE + (1 << 30)
    size = qmv.qmv_workspace_size
    n = size("q4_k", "bf16", 512, [(gate, FAKE, FAKE)])
    assert n >= 512 * 3584 * 2 + 512 * 4 and n % 256 == 0                # fp16 rows + row scales
    # K in slices: the partial outputs too
    assert size("q4_k", "bf16", 512, [(down, FAKE, FAKE)]) >= 512 * 18944 * 2 + 2 * 512 * 3584 * 4
    assert size("q4_k", "f16", 512, [(gate, FAKE, FAKE)]) > 0
    assert size("q4_k", "bf16", 32, [(down, FAKE, FAKE)]) > 0        # long K: from 17 rows
    assert size("q4_k", "bf16", 32, [(gate, FAKE, FAKE)]) == 0       # a lone matrix: from 65 rows
    assert size("q4_k", "bf16", 32, [(gate, FAKE, FAKE), (gate, FAKE, Y2)]) > 0  # a run: from 17
    assert size("q4_k", "bf16", 512, [(small, FAKE, FAKE)]) == 0     # fewer than 256 weight rows
    assert size("q4_k", "f32", 512, [(gate, FAKE, FAKE)]) == 0
    assert size("q4_k", "bf16", 1, [(gate, FAKE, FAKE)]) == 0
    assert size("q6_k", "bf16", 512, [(_desc("q6_k", 18944, 3584), FAKE, FAKE)]) == 0
    _expect(-3, size, "q4_k", "bf16", 0, [(gate, FAKE, FAKE)])
    _expect(-1, size, "q4_k", "bf16", 512, [(gate, None, FAKE)])
    m = qmv.qmv_gemv_multi_ws
    items = [(gate, FAKE, FAKE)]
    _expect(-1, m, "q4_k", "bf16", 512, items, None, n)
    _expect(-4, m, "q4_k", "bf16", 512, items, FAKE + 16, n)
    _expect(-5, m, "q4_k", "bf16", 512, items, FAKE, n - 1)
    _expect(-5, m, "q4_k", "bf16", 512, items, FAKE, 0)
    # the fixed scratch of the allocation-free call holds 64 MiB
    _expect(-5, qmv.qmv_gemv_noalloc, "q4_k", down, FAKE, "bf16", FAKE, 3584, 18944, 2048)


def test_swiglu_validation_errors():
    g, u = _desc("q4_k", 8, 512), _desc("q4_k", 8, 512)
    f = qmv.qmv_gemv_swiglu
    H = FAKE + 4096
    _expect(-2, f, "q6_k", g, u, FAKE, "f32", H, 8, 512, 1)                 # fmt disagrees
    _expect(-2, f, "q4_k", g, _desc("q4_k", 9, 512), FAKE, "f32", H, 8, 512, 1)
    _expect(-2, f, "q4_k", g, u, FAKE, "f32", H, 8, 256, 1)
    pl = qmv.qmv_create_weights_planes("q4_k", 8, 512, FAKE, qmv.qmv_planes_size("q4_k", 8, 512))
    _expect(-6, f, "q4_k", g, pl, FAKE, "f32", H, 8, 512, 1)                # layouts differ
    _expect(-1, f, "q4_k", g, u, None, "f32", H, 8, 512, 1)
    _expect(-4, f, "q4_k", g, u, FAKE, "f32", H + 4, 8, 512, 1)
    _expect(-3, f, "q4_k", g, u, FAKE, "f32", H, 8, 512, 0)
    _expect(-6, f, "q4_k", g, u, FAKE, 7, H, 8, 512, 1)
    _expect(-3, f, "q4_k", g, u, FAKE, "f32", FAKE + 16, 8, 512, 1)          # h overlaps x
    w17 = _desc("q4_k", 8, 17 * 256)                                         # past one wave's K slice
    _expect(-6, f, "q4_k", w17, w17, FAKE, "f32", FAKE + (1 << 20), 8, 17 * 256, 1)
    q8 = _desc("q8_0", 8, 2080)
    _expect(-6, f, "q8_0", q8, q8, FAKE, "f32", FAKE + (1 << 20), 8, 2080, 1)
    bad = _desc()
    bad.nbytes += 144
    _expect(-5, f, "q4_k", g, bad, FAKE, "f32", H, 8, 512, 1)


def test_dequant_and_probe_validation_errors():
    w = _desc()
    _expect(-1, qmv.qmv_dequant, w, None, "f32")
    _expect(-6, qmv.qmv_dequant, w, FAKE, 5)
    _expect(-4, qmv.qmv_dequant, w, FAKE + 2, "f32")
    _expect(-5, qmv.qmv_probe_read, FAKE, 17, FAKE)
    _expect(-4, qmv.qmv_probe_copy, FAKE + 1, FAKE, 16)
    _expect(-1, qmv.qmv_probe_copy, None, FAKE, 16)
    assert qmv.qmv_probe_read_outputs(1 << 30) >= 1


def test_status_strings():
    for s in range(-8, 1):
        assert qmv.qmv_status_string(s) not in ("", "unknown status")
    assert qmv.qmv_status_string(-99) == "unknown status"


def test_hip_error_surfaces_without_a_gpu():
    """A valid call on a machine with no GPU fails inside HIP -> QMV_ERR_HIP."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this test would launch with fake pointers")
    w = _desc()
    _expect(-8, qmv.qmv_gemv, "q4_k", w, FAKE, "f32", FAKE, 8, 512, 1)


def test_single_hip_runtime_mapped():
    import torch  # noqa: F401
    qmv.lib()
    maps = {line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line}
    assert len(maps) == 1, maps


def test_planes_sizes_and_repack_validation_errors():
    """Plane layout: sizes, and every refusal of qmv_repack_planes, of a plane
    descriptor that does not match its shape, and of mixed or matrix-core
    launches -- all before any HIP call."""
    n_blocks = 8 * 2
    a = (16 * n_blocks + 255) // 256 * 256
    assert qmv.qmv_planes_size("q4_k", 8, 512) == 5 * a + 64 * n_blocks
    assert qmv.qmv_planes_size("q4_k", 18944, 3584) == 38_191_104  # 16 N is a multiple of 256 there
    assert qmv.qmv_planes_size("q6_k", 8, 512) == 13 * a + 2 * n_blocks
    assert qmv.qmv_planes_size("q6_k", 152064, 3584) == 447_068_160  # no padding at the lm-head shape
    assert qmv.qmv_planes_size("q5_k", 8, 512) == 7 * a + 64 * n_blocks
    assert qmv.qmv_planes_size("q5_k", 3584, 18944) == 46_678_016  # no padding at the down shape
    for f in ("q8_0", "int4_g128"):
        assert qmv.qmv_planes_size(f, 8, 512) == 0
    assert qmv.qmv_planes_size("q4_k", 8, 500) == 0
    src = _desc()
    need = qmv.qmv_planes_size("q4_k", 8, 512)
    dst = FAKE + (1 << 20)
    r = qmv.qmv_repack_planes
    _expect(-1, r, src, None, need)
    _expect(-5, r, src, dst, need - 1)
    _expect(-4, r, src, dst + 8, need)
    _expect(-3, r, src, FAKE + 64, need)                    # overlaps the source
    _expect(-6, r, _desc("q8_0", 8, 512), dst, need)        # no plane layout for Q8_0
    bad = _desc()
    bad.nbytes += 1
    _expect(-5, r, bad, dst, need)
    # a plane descriptor, filled by hand as a caller restoring saved planes would
    p = _desc()
    p.layout, p.nbytes, p.scales_offset = 1, need, a
    _expect(-6, r, p, dst, need)                            # already planes
    g = qmv.qmv_gemv
    tampered = _desc()
    tampered.layout, tampered.nbytes, tampered.scales_offset = 1, need, 0
    _expect(-2, g, "q4_k", tampered, FAKE, "f32", FAKE, 8, 512, 1)  # wrong plane offset
    tampered.scales_offset, tampered.nbytes = a, need + 16
    _expect(-5, g, "q4_k", tampered, FAKE, "f32", FAKE, 8, 512, 1)
    tampered.nbytes, tampered.layout = need, 7
    _expect(-2, g, "q4_k", tampered, FAKE, "f32", FAKE, 8, 512, 1)  # unknown layout
    q8 = _desc("q8_0", 8, 512)
    q8.layout = 1
    _expect(-6, g, "q8_0", q8, FAKE, "f32", FAKE, 8, 512, 1)
    _expect(-6, qmv.qmv_gemv_multi, "q4_k", "f32", 1, [(src, FAKE, FAKE), (p, FAKE, FAKE + 4096)])
    assert _desc().layout == 0


def test_create_weights_planes():
    """Wrapping kept plane bytes: the descriptor equals what qmv_repack_planes
    would return, and every refusal comes before any HIP call."""
    c = qmv.qmv_create_weights_planes
    for fmt in ("q4_k", "q5_k", "q6_k"):
        n = qmv.qmv_planes_size(fmt, 8, 512)
        w = c(fmt, 8, 512, FAKE, n)
        a = (16 * 16 + 255) // 256 * 256
        assert (w.fmt, w.layout, w.rows, w.cols, w.nbytes, w.scales_offset) == (qmv.FMT[fmt], 1, 8, 512, n, a)
    n = qmv.qmv_planes_size("q4_k", 8, 512)
    _expect(-1, c, "q4_k", 8, 512, None, n)
    _expect(-2, c, 9, 8, 512, FAKE, n)
    _expect(-6, c, "q8_0", 8, 512, FAKE, n)
    _expect(-3, c, "q4_k", 8, 500, FAKE, n)
    _expect(-5, c, "q4_k", 8, 512, FAKE, n - 16)
    _expect(-4, c, "q4_k", 8, 512, FAKE + 8, n)


def test_header_is_plain_c_and_links():
    """include/qmv.h compiles as C99 with every warning on, and a C program
    that calls entry points which need no GPU links against libqmv.so and
    runs: the boundary is a plain C ABI."""
    import shutil
    import subprocess
    import tempfile
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = r'''
#include <stdio.h>
#include "qmv.h"
int main(void) {
  qmv_weights w;
  uint64_t n = qmv_packed_size(QMV_Q4_K, 8, 512), ws = 1;
  qmv_gemv_item it;
  if (n != 8 * 2 * 144) return 1;
  if (qmv_create_weights(QMV_Q4_K, 8, 512, (const void*)(uintptr_t)0x7F0000000000ull, n, &w) != QMV_OK) return 2;
  it.W = &w; it.x = (const void*)(uintptr_t)0x7F0000100000ull; it.y = (float*)(uintptr_t)0x7F0000200000ull;
  if (qmv_workspace_size(QMV_Q4_K, QMV_BF16, 1, &it, 1, &ws) != QMV_OK || ws != 0) return 3;
  if (qmv_gemv_swiglu(QMV_Q4_K, &w, &w, 0, QMV_F32, it.y, 8, 512, 1, 0) != QMV_ERR_NULL) return 4;
  printf("%s\n", qmv_status_string(QMV_ERR_SIZE));
  return 0;
}
'''
    lib = qmv.lib()._name
    if "asan" in os.path.basename(lib):
        pytest.skip("the sanitizer build of the library runs the other ABI tests; this one links the regular build")
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                        c, lib, "-Wl,-rpath," + os.path.dirname(lib), "-o", exe], check=True)
        r = subprocess.run([exe], capture_output=True, text=True)
        assert r.returncode == 0, (r.returncode, r.stderr)
        assert r.stdout.strip() != ""
