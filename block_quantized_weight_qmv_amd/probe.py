"""HBM probes of libqmv (qmv_probe_read / qmv_probe_copy) from the command line.

    python -m block_quantized_weight_qmv_amd.probe read --mib 2048 --iters 10
    python -m block_quantized_weight_qmv_amd.probe copy --mib 256 --iters 5

`read` streams a buffer with 128-bit loads (the practical read ceiling the
GEMV kernels are compared with); `copy` moves a buffer of known size, which
calibrates hardware byte counters (a copy of N bytes reads N and writes N).
Launches are eager, one per iteration, on the current stream.
"""
from __future__ import annotations

import argparse
import json


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("mode", choices=["read", "copy"])
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--iters", type=int, default=10)
    args = ap.parse_args()

    import torch

    from block_quantized_weight_qmv_amd import qmv

    nb = args.mib * 2 ** 20
    dev = torch.device("cuda:0")
    src = torch.empty(nb, dtype=torch.uint8, device=dev)
    src.fill_(1)
    if args.mode == "read":
        out = torch.empty(qmv.qmv_probe_read_outputs(nb), dtype=torch.float32, device=dev)
        run = lambda: qmv.qmv_probe_read(src, nb, out)  # noqa: E731
    else:
        dst = torch.empty(nb, dtype=torch.uint8, device=dev)
        run = lambda: qmv.qmv_probe_copy(src, dst, nb)  # noqa: E731
    run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.iters):
        run()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / args.iters
    moved = nb * (1 if args.mode == "read" else 2)
    print(json.dumps({"probe": args.mode, "bytes": nb, "launches": args.iters + 1,
                      "us_per_launch": round(us, 2), "GBps": round(moved / us / 1e3, 1)}), flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
