"""Helpers for the GPU parity tests: upload packed weights, run the library."""
import numpy as np
import torch

import oracle
from block_quantized_weight_qmv_amd import qmv
from synth import gen_weights, gen_x

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def to_dev_x(x_np, x_dtype):
    if x_dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x_np)).to(DEV)
    if x_dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(x_np)).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).to(DEV).view(torch.bfloat16)


class Weights:
    """Fields from synth, packed by the library packer and uploaded; oracle bytes packed separately."""

    def __init__(self, fmt, rows, cols, seed=None, fields=None):
        self.fmt, self.rows, self.cols = fmt, rows, cols
        self.fields = fields if fields is not None else gen_weights(fmt, rows, cols, seed)
        packed = qmv.pack_fields(fmt, self.fields, rows, cols)
        self.dev = torch.from_numpy(packed).to(DEV)
        self.desc = qmv.qmv_create_weights(fmt, rows, cols, self.dev)

    def oracle_bytes(self, row_ids=None):
        """Oracle-packed bytes of all rows, or of the listed rows as a standalone tensor."""
        f = self.fields
        if row_ids is None:
            return oracle.pack(self.fmt, f, self.rows, self.cols)
        ids = np.asarray(row_ids)
        sub = {k: v[ids] for k, v in f.items()}
        return oracle.pack(self.fmt, sub, len(ids), self.cols)

    def gemv(self, x_dev, x_dtype, batch, y=None, stream=None, ws=True):
        """y = W x through qmv_gemv_multi_ws with a workspace of the size the
        library asks for (the register-dequantized kernels where the launch
        takes them), or through plain qmv_gemv (ws=False)."""
        if y is None:
            y = torch.empty(batch, self.rows, dtype=torch.float32, device=DEV)
        if not ws:
            qmv.qmv_gemv(self.fmt, self.desc, x_dev, x_dtype, y, self.rows, self.cols, batch, stream)
            return y
        self._ws = gemv_ws(self.fmt, [(self.desc, x_dev, y)], x_dtype, batch, stream)
        return y


def gemv_ws(fmt, items, x_dtype, batch, stream=None):
    """qmv_gemv_multi_ws over `items` with a fresh workspace of the size the
    library asks for; returns the workspace, which the caller holds until the
    launch has run (a graph capture keeps it in the graph's own pool)."""
    n = qmv.qmv_workspace_size(fmt, x_dtype, batch, items)
    buf = torch.empty(n, dtype=torch.uint8, device=DEV) if n else None
    qmv.qmv_gemv_multi_ws(fmt, x_dtype, batch, items, buf, n, stream)
    if buf is not None and isinstance(stream, torch.cuda.Stream) and stream != torch.cuda.current_stream():
        buf.record_stream(stream)  # not reused before the launch on `stream` has run
    return buf


def oracle_y(w: Weights, x_np, x_dtype, row_ids=None):
    if row_ids is None:
        return oracle.gemv64(w.fmt, w.oracle_bytes(), w.rows, w.cols, x_np, x_dtype)
    return oracle.gemv64(w.fmt, w.oracle_bytes(row_ids), len(row_ids), w.cols, x_np, x_dtype)
