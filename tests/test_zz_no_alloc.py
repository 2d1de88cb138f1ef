"""qmv_gemv_noalloc: a variant of qmv_gemv_multi_ws (one item) for callers
that cannot allocate, whose register-dequantized kernels take the library's
fixed scratch in place of a caller workspace.  Through the C ABI it must
return what qmv_gemv_multi_ws returns with a workspace of the size
qmv_workspace_size names, bit for bit (the same kernels run; only the
workspace differs), on two calls in a row (the second smaller, reusing the
fixed scratch the first left full), under graph capture on a stream that
never ran a call before, and refuse a call whose workspace exceeds the fixed
scratch with QMV_ERR_SIZE."""
import pytest
import torch

from block_quantized_weight_qmv_amd import qmv
from gpu_util import DEV, Weights, gemv_ws, say, to_dev_x
from synth import gen_x

pytestmark = pytest.mark.gpu


def _both(w, x, x_dtype, batch):
    ya = torch.full((batch, w.rows), 7.0, dtype=torch.float32, device=DEV)
    yb = torch.full((batch, w.rows), -7.0, dtype=torch.float32, device=DEV)
    buf = gemv_ws(w.fmt, [(w.desc, x, ya)], x_dtype, batch)
    qmv.qmv_gemv_noalloc(w.fmt, w.desc, x, x_dtype, yb, w.rows, w.cols, batch)
    torch.cuda.synchronize()
    del buf
    return ya, yb


@pytest.mark.parametrize("x_dtype", ["bf16", "f16"])
def test_noalloc_matches_gemv_two_calls(x_dtype):
    # the 7B FFN down matrix (K in slices: converted activations and partial
    # outputs in the scratch), then a smaller, ragged batch against the gate
    # matrix's shape class
    for rows, cols, batch, seed in [(3584, 18944, 512, 1), (4100, 14 * 256, 130, 2)]:
        say(f"noalloc {x_dtype} q4_k {rows}x{cols} batch {batch}")
        w = Weights("q4_k", rows, cols, seed=2500 + seed)
        x = to_dev_x(gen_x(batch, cols, x_dtype, seed=250 + seed), x_dtype)
        ya, yb = _both(w, x, x_dtype, batch)
        assert torch.equal(ya, yb)
        assert torch.isfinite(ya).all()
        del w
        torch.cuda.empty_cache()


def test_noalloc_other_paths_and_size_limit():
    # paths without a workspace (batch 1 and 16) give plain qmv_gemv's
    # result; 64 rows against this long-K matrix take the register kernels;
    # a workspace above the fixed scratch is refused before any launch
    w = Weights("q4_k", 3584, 18944, seed=2600)
    for batch, x_dtype in [(1, "f32"), (16, "bf16"), (64, "bf16")]:
        say(f"noalloc {x_dtype} batch {batch}")
        x = to_dev_x(gen_x(batch, w.cols, x_dtype, seed=260 + batch), x_dtype)
        ya, yb = _both(w, x, x_dtype, batch)
        assert torch.equal(ya, yb)
        registers = qmv.qmv_workspace_size(w.fmt, x_dtype, batch, [(w.desc, x, ya)]) > 0
        assert registers == (batch == 64)
        if not registers:
            assert torch.equal(ya, w.gemv(x, x_dtype, batch, ws=False))
    batch = 2048  # 2048 x 18944 fp16 activations alone exceed 64 MiB
    x = to_dev_x(gen_x(batch, w.cols, "bf16", seed=269), "bf16")
    y = torch.full((batch, w.rows), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(qmv.QmvError, match="QMV_ERR_SIZE"):
        qmv.qmv_gemv_noalloc(w.fmt, w.desc, x, "bf16", y, w.rows, w.cols, batch)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())  # nothing ran


def test_noalloc_under_capture_on_a_fresh_stream():
    # no call ever ran on this stream and no workspace comes with the call
    rows, cols, batch = 3584, 14 * 256, 256
    w = Weights("q4_k", rows, cols, seed=2700)
    x = to_dev_x(gen_x(batch, cols, "bf16", seed=270), "bf16")
    y0 = w.gemv(x, "bf16", batch)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    yg = torch.zeros(batch, rows, dtype=torch.float32, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            qmv.qmv_gemv_noalloc(w.fmt, w.desc, x, "bf16", yg, rows, cols, batch, stream=s)
    for _ in range(3):
        yg.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y0)
