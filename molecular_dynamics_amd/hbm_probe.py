"""Attainable HBM bandwidth of plain streaming kernels on this GPU, for context beside
the published 8 TB/s peak: a device-to-device copy (read + write), a fill (write only)
and a sum (read only), each over a buffer far larger than the caches, timed with HIP
events on the current stream (median of repeated launches).

    python -m molecular_dynamics_amd.hbm_probe [--gib 4] [--reps 10]

Prints one JSON line with GB/s (1e9 bytes per second) per pattern.
"""
import argparse
import json
import statistics
import sys


def timed(fn, reps):
    import torch
    fn()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        out.append(a.elapsed_time(b) * 1e-3)
    return statistics.median(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gib", type=float, default=4.0, help="buffer size in GiB")
    ap.add_argument("--reps", type=int, default=10)
    a = ap.parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("hbm_probe: needs a GPU")
    n = int(a.gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    nbytes = 4 * n
    res = {"buffer_bytes": nbytes, "device": torch.cuda.get_device_name(0)}
    t = timed(lambda: dst.copy_(src), a.reps)
    res["copy_GBps"] = round(2 * nbytes / t * 1e-9, 1)
    t = timed(lambda: dst.fill_(1.0), a.reps)
    res["fill_GBps"] = round(nbytes / t * 1e-9, 1)
    t = timed(lambda: src.sum(), a.reps)
    res["sum_GBps"] = round(nbytes / t * 1e-9, 1)
    res["peak_GBps"] = 8000.0
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
