"""Python binding of libqmv.so: the C ABI of include/qmv.h, one function per entry point.

Argument marshalling only.  Device buffers are torch tensors (or raw integer
device pointers); every computation runs in the library's HIP kernels.  If the
library is not built, the first call raises: there is no fallback path.

torch is imported before the library is loaded so that libqmv.so binds to the
HIP runtime torch already mapped (both use the soname libamdhip64.so.7), which
makes torch's hipStream_t values valid inside the library.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# QMV_LIBRARY names another build of the same library (the sanitizer build of
# the CPU test suite); by default the in-tree libqmv.so.
LIB_PATH = os.environ.get("QMV_LIBRARY") or os.path.join(PKG_DIR, "libqmv.so")

FMT = {"q8_0": 1, "q4_k": 2, "q6_k": 3, "int4_g128": 4, "q5_k": 5}
DTYPE = {"f32": 0, "f16": 1, "bf16": 2}
LAYOUT = {"blocks": 0, "planes": 1}

QMV_OK = 0
STATUS = {0: "QMV_OK", -1: "QMV_ERR_NULL", -2: "QMV_ERR_FORMAT", -3: "QMV_ERR_SHAPE",
          -4: "QMV_ERR_ALIGN", -5: "QMV_ERR_SIZE", -6: "QMV_ERR_UNSUPPORTED",
          -7: "QMV_ERR_RANGE", -8: "QMV_ERR_HIP"}


class QmvError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


class QmvWeights(ctypes.Structure):
    """Mirror of struct qmv_weights."""
    _fields_ = [("fmt", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("data", ctypes.c_void_p), ("nbytes", ctypes.c_uint64),
                ("scales_offset", ctypes.c_uint64)]


class QmvGemvItem(ctypes.Structure):
    """Mirror of struct qmv_gemv_item."""
    _fields_ = [("W", ctypes.POINTER(QmvWeights)), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p)]


_lib = None

_i32, _i64, _u64, _p = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
_SIGS = {
    "qmv_block_size": (_i32, [_i32]),
    "qmv_packed_size": (_u64, [_i32, _i64, _i64]),
    "qmv_pack_q8_0": (_i32, [_p, _p, _i64, _i64, _p, _u64]),
    "qmv_pack_q4_k": (_i32, [_p, _p, _p, _p, _p, _i64, _i64, _p, _u64]),
    "qmv_pack_q5_k": (_i32, [_p, _p, _p, _p, _p, _i64, _i64, _p, _u64]),
    "qmv_pack_q6_k": (_i32, [_p, _p, _p, _i64, _i64, _p, _u64]),
    "qmv_pack_int4_g128": (_i32, [_p, _p, _i64, _i64, _p, _u64]),
    "qmv_create_weights": (_i32, [_i32, _i64, _i64, _p, _u64, ctypes.POINTER(QmvWeights)]),
    "qmv_planes_size": (_u64, [_i32, _i64, _i64]),
    "qmv_create_weights_planes": (_i32, [_i32, _i64, _i64, _p, _u64, ctypes.POINTER(QmvWeights)]),
    "qmv_repack_planes": (_i32, [ctypes.POINTER(QmvWeights), _p, _u64, ctypes.POINTER(QmvWeights), _p]),
    "qmv_gemv": (_i32, [_i32, ctypes.POINTER(QmvWeights), _p, _i32, _p, _i64, _i64, _i64, _p]),
    "qmv_gemv_noalloc": (_i32, [_i32, ctypes.POINTER(QmvWeights), _p, _i32, _p, _i64, _i64, _i64, _p]),
    "qmv_gemv_multi": (_i32, [_i32, _i32, _i64, ctypes.POINTER(QmvGemvItem), _i32, _p]),
    "qmv_workspace_size": (_i32, [_i32, _i32, _i64, ctypes.POINTER(QmvGemvItem), _i32,
                                  ctypes.POINTER(_u64)]),
    "qmv_gemv_multi_ws": (_i32, [_i32, _i32, _i64, ctypes.POINTER(QmvGemvItem), _i32, _p, _u64, _p]),
    "qmv_gemv_swiglu": (_i32, [_i32, ctypes.POINTER(QmvWeights), ctypes.POINTER(QmvWeights), _p, _i32, _p,
                               _i64, _i64, _i64, _p]),
    "qmv_dequant": (_i32, [ctypes.POINTER(QmvWeights), _p, _i32, _p]),
    "qmv_probe_read_outputs": (_i64, [_u64]),
    "qmv_probe_read": (_i32, [_p, _u64, _p, _p]),
    "qmv_probe_copy": (_i32, [_p, _p, _u64, _p]),
    "qmv_status_string": (ctypes.c_char_p, [_i32]),
    "qmv_last_error": (ctypes.c_char_p, []),
}
EXPORTED = tuple(_SIGS)


def lib() -> ctypes.CDLL:
    """Load libqmv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_quantized_weight_qmv_amd.build`")
        try:
            import torch  # noqa: F401  (maps torch's HIP runtime first)
        except ImportError:
            pass
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int) -> None:
    if status != QMV_OK:
        raise QmvError(status, (lib().qmv_last_error() or b"").decode())


def _ptr(a):
    """Device or host address of a torch tensor, numpy array, int or None."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    return a.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    for t in tensors:
        if hasattr(t, "is_cuda") and t.is_cuda:
            import torch
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


# Tensor dtypes accepted for each activation / output dtype code (bf16 may
# also arrive as its 16-bit patterns).
_TORCH_OK = {0: ("float32",), 1: ("float16",), 2: ("bfloat16", "int16", "uint16")}
_ELEM = {0: 4, 1: 2, 2: 2}


def _check_dev(t, what: str, dtype_code: int | None, min_elems: int) -> None:
    """Refuse a device buffer the kernels could not use safely.

    The C ABI sees raw pointers only, so this is the one layer that can check
    a torch tensor before the kernels read or write through it: it must live
    on the GPU, be contiguous, have the element type of ``dtype_code`` (None:
    any) and hold at least ``min_elems`` elements of that type.  Integer
    addresses are passed through unchecked (the caller vouches for them)."""
    if t is None or isinstance(t, int):
        return
    if isinstance(t, np.ndarray):
        raise QmvError(-6, f"{what}: a host numpy array; device memory (a GPU tensor) is required")
    if not getattr(t, "is_cuda", False):
        raise QmvError(-6, f"{what}: tensor is not on a GPU")
    if not t.is_contiguous():
        raise QmvError(-6, f"{what}: tensor is not contiguous")
    if dtype_code is not None:
        name = str(t.dtype).replace("torch.", "")
        if name not in _TORCH_OK[dtype_code]:
            raise QmvError(-2, f"{what}: tensor dtype {name}, expected one of {_TORCH_OK[dtype_code]}")
        have = t.numel() * t.element_size() // _ELEM[dtype_code]
    else:
        have = t.numel() * t.element_size()
    if have < min_elems:
        raise QmvError(-5, f"{what}: holds {have} elements, needs {min_elems}")


def _fmt(fmt) -> int:
    return FMT[fmt] if isinstance(fmt, str) else int(fmt)


def _dtype(dt) -> int:
    if isinstance(dt, str):
        return DTYPE[dt]
    if isinstance(dt, int):
        return dt
    import torch
    return {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}[dt]


# -- entry points -------------------------------------------------------------
def qmv_block_size(fmt) -> int:
    return lib().qmv_block_size(_fmt(fmt))


def qmv_packed_size(fmt, rows: int, cols: int) -> int:
    return lib().qmv_packed_size(_fmt(fmt), rows, cols)


def _pack_out(fmt, rows, cols):
    n = qmv_packed_size(fmt, rows, cols)
    if n == 0:
        raise QmvError(-3, f"bad shape {rows}x{cols} for {fmt}")
    return np.empty(n, np.uint8)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def qmv_pack_q8_0(d_bits, q, rows: int, cols: int) -> np.ndarray:
    d, qq, out = _c(d_bits, np.uint16), _c(q, np.int8), _pack_out("q8_0", rows, cols)
    _check(lib().qmv_pack_q8_0(_ptr(d), _ptr(qq), rows, cols, _ptr(out), out.size))
    return out


def qmv_pack_q4_k(d_bits, dmin_bits, sc6, m6, q4, rows: int, cols: int) -> np.ndarray:
    d, dm = _c(d_bits, np.uint16), _c(dmin_bits, np.uint16)
    sc, m, q = _c(sc6, np.uint8), _c(m6, np.uint8), _c(q4, np.uint8)
    out = _pack_out("q4_k", rows, cols)
    _check(lib().qmv_pack_q4_k(_ptr(d), _ptr(dm), _ptr(sc), _ptr(m), _ptr(q), rows, cols,
                               _ptr(out), out.size))
    return out


def qmv_pack_q5_k(d_bits, dmin_bits, sc6, m6, q5, rows: int, cols: int) -> np.ndarray:
    d, dm = _c(d_bits, np.uint16), _c(dmin_bits, np.uint16)
    sc, m, q = _c(sc6, np.uint8), _c(m6, np.uint8), _c(q5, np.uint8)
    out = _pack_out("q5_k", rows, cols)
    _check(lib().qmv_pack_q5_k(_ptr(d), _ptr(dm), _ptr(sc), _ptr(m), _ptr(q), rows, cols,
                               _ptr(out), out.size))
    return out


def qmv_pack_q6_k(d_bits, sc8, q6, rows: int, cols: int) -> np.ndarray:
    d, sc, q = _c(d_bits, np.uint16), _c(sc8, np.int8), _c(q6, np.uint8)
    out = _pack_out("q6_k", rows, cols)
    _check(lib().qmv_pack_q6_k(_ptr(d), _ptr(sc), _ptr(q), rows, cols, _ptr(out), out.size))
    return out


def qmv_pack_int4_g128(s_bits, q, rows: int, cols: int) -> np.ndarray:
    s, qq, out = _c(s_bits, np.uint16), _c(q, np.int8), _pack_out("int4_g128", rows, cols)
    _check(lib().qmv_pack_int4_g128(_ptr(s), _ptr(qq), rows, cols, _ptr(out), out.size))
    return out


def pack_fields(fmt: str, fields: dict, rows: int, cols: int) -> np.ndarray:
    """Call the packer of `fmt` with the field arrays named as in synth/."""
    if fmt == "q8_0":
        return qmv_pack_q8_0(fields["d_bits"], fields["q"], rows, cols)
    if fmt == "q4_k":
        return qmv_pack_q4_k(fields["d_bits"], fields["dmin_bits"], fields["sc"], fields["m"],
                             fields["u"], rows, cols)
    if fmt == "q5_k":
        return qmv_pack_q5_k(fields["d_bits"], fields["dmin_bits"], fields["sc"], fields["m"],
                             fields["u"], rows, cols)
    if fmt == "q6_k":
        return qmv_pack_q6_k(fields["d_bits"], fields["sc"], fields["q"], rows, cols)
    if fmt == "int4_g128":
        return qmv_pack_int4_g128(fields["s_bits"], fields["q"], rows, cols)
    raise ValueError(fmt)


def qmv_create_weights(fmt, rows: int, cols: int, dev_packed, nbytes: int | None = None) -> QmvWeights:
    """Descriptor for packed bytes already in device memory (a uint8 tensor or a pointer)."""
    if nbytes is None:
        nbytes = dev_packed.numel() * dev_packed.element_size()
    _check_dev(dev_packed, "packed weights", None, nbytes)
    w = QmvWeights()
    _check(lib().qmv_create_weights(_fmt(fmt), rows, cols, _ptr(dev_packed), nbytes, ctypes.byref(w)))
    # The descriptor holds a raw pointer: keep the tensor alive with it, or the
    # caching allocator may hand its memory back to the driver (empty_cache(),
    # which graph capture calls) while launches still read it.
    w.owner = None if isinstance(dev_packed, int) else dev_packed
    return w


def qmv_planes_size(fmt, rows: int, cols: int) -> int:
    return lib().qmv_planes_size(_fmt(fmt), rows, cols)


def qmv_create_weights_planes(fmt, rows: int, cols: int, dev_planes, nbytes: int | None = None) -> QmvWeights:
    """Descriptor for plane-layout bytes already in device memory (a uint8 tensor or a pointer)."""
    if nbytes is None:
        nbytes = dev_planes.numel() * dev_planes.element_size()
    _check_dev(dev_planes, "plane weights", None, nbytes)
    w = QmvWeights()
    _check(lib().qmv_create_weights_planes(_fmt(fmt), rows, cols, _ptr(dev_planes), nbytes, ctypes.byref(w)))
    w.owner = None if isinstance(dev_planes, int) else dev_planes
    return w


def qmv_repack_planes(src: QmvWeights, dst, dst_bytes: int | None = None, stream=None) -> QmvWeights:
    """Enqueue the repack of canonical Q4_K blocks into the plane layout at dst
    (a uint8 device tensor or a pointer); returns the planes descriptor."""
    if dst_bytes is None:
        dst_bytes = dst.numel() * dst.element_size()
    _check_dev(dst, "dst", None, dst_bytes)
    w = QmvWeights()
    _check(lib().qmv_repack_planes(ctypes.byref(src), _ptr(dst), dst_bytes, ctypes.byref(w),
                                   _stream(stream, dst)))
    w.owner = None if isinstance(dst, int) else dst
    return w


def qmv_gemv(fmt, W: QmvWeights, x, x_dtype, y, rows: int, cols: int, batch: int,
             stream=None) -> None:
    xd = _dtype(x_dtype)
    _check_dev(x, "x", xd, batch * cols)
    _check_dev(y, "y", 0, batch * rows)
    _check(lib().qmv_gemv(_fmt(fmt), ctypes.byref(W), _ptr(x), _dtype(x_dtype), _ptr(y),
                          rows, cols, batch, _stream(stream, x, y)))


def qmv_gemv_noalloc(fmt, W: QmvWeights, x, x_dtype, y, rows: int, cols: int, batch: int,
                     stream=None) -> None:
    xd = _dtype(x_dtype)
    _check_dev(x, "x", xd, batch * cols)
    _check_dev(y, "y", 0, batch * rows)
    _check(lib().qmv_gemv_noalloc(_fmt(fmt), ctypes.byref(W), _ptr(x), _dtype(x_dtype), _ptr(y),
                                  rows, cols, batch, _stream(stream, x, y)))


def _items(x_dtype, batch: int, items, check: bool = True):
    arr = (QmvGemvItem * max(1, len(items)))()
    xd = _dtype(x_dtype)
    for i, (W, x, y) in enumerate(items):
        if check:
            _check_dev(x, f"item {i} x", xd, batch * W.cols)
            _check_dev(y, f"item {i} y", 0, batch * W.rows)
        arr[i].W = ctypes.pointer(W)
        arr[i].x = _ptr(x)
        arr[i].y = _ptr(y)
    return arr


def qmv_gemv_multi(fmt, x_dtype, batch: int, items, stream=None) -> None:
    """items: sequence of (QmvWeights, x, y) triples; one launch for all of them."""
    arr = _items(x_dtype, batch, items)
    tensors = [t for _, x, y in items for t in (x, y)]
    _check(lib().qmv_gemv_multi(_fmt(fmt), _dtype(x_dtype), batch, arr, len(items),
                                _stream(stream, *tensors)))


def qmv_workspace_size(fmt, x_dtype, batch: int, items) -> int:
    """Bytes of workspace qmv_gemv_multi_ws needs for these items (0: none)."""
    arr = _items(x_dtype, batch, items, check=False)
    n = _u64(0)
    _check(lib().qmv_workspace_size(_fmt(fmt), _dtype(x_dtype), batch, arr, len(items),
                                    ctypes.byref(n)))
    return int(n.value)


def qmv_gemv_multi_ws(fmt, x_dtype, batch: int, items, workspace, workspace_bytes: int,
                      stream=None) -> None:
    """qmv_gemv_multi with a caller-owned device workspace (None: no workspace)."""
    arr = _items(x_dtype, batch, items)
    tensors = [t for _, x, y in items for t in (x, y)]
    if workspace is not None:
        _check_dev(workspace, "workspace", None, workspace_bytes)
        tensors.append(workspace)
    _check(lib().qmv_gemv_multi_ws(_fmt(fmt), _dtype(x_dtype), batch, arr, len(items),
                                   _ptr(workspace) if workspace is not None else None,
                                   workspace_bytes, _stream(stream, *tensors)))


def qmv_gemv_swiglu(fmt, Wg: QmvWeights, Wu: QmvWeights, x, x_dtype, h, rows: int, cols: int, batch: int,
                    stream=None) -> None:
    """h = silu(Wg x) * (Wu x) in one launch (h: [batch][rows] fp32)."""
    xd = _dtype(x_dtype)
    _check_dev(x, "x", xd, batch * cols)
    _check_dev(h, "h", 0, batch * rows)
    _check(lib().qmv_gemv_swiglu(_fmt(fmt), ctypes.byref(Wg), ctypes.byref(Wu), _ptr(x), xd, _ptr(h),
                                 rows, cols, batch, _stream(stream, x, h)))


def qmv_dequant(W: QmvWeights, out, out_dtype, stream=None) -> None:
    od = _dtype(out_dtype)
    _check_dev(out, "out", od, W.rows * W.cols)
    _check(lib().qmv_dequant(ctypes.byref(W), _ptr(out), _dtype(out_dtype), _stream(stream, out)))


def qmv_probe_read_outputs(nbytes: int) -> int:
    return lib().qmv_probe_read_outputs(nbytes)


def qmv_probe_read(src, nbytes: int, out, stream=None) -> None:
    _check_dev(src, "src", None, nbytes)
    _check_dev(out, "out", 0, qmv_probe_read_outputs(nbytes))
    _check(lib().qmv_probe_read(_ptr(src), nbytes, _ptr(out), _stream(stream, src, out)))


def qmv_probe_copy(src, dst, nbytes: int, stream=None) -> None:
    _check_dev(src, "src", None, nbytes)
    _check_dev(dst, "dst", None, nbytes)
    _check(lib().qmv_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream, src, dst)))


def qmv_status_string(status: int) -> str:
    return lib().qmv_status_string(status).decode()


def qmv_last_error() -> str:
    return (lib().qmv_last_error() or b"").decode()
