"""Plain device-to-device copy of a known size, for calibrating HBM traffic
counters (FETCH_SIZE / WRITE_SIZE per dispatch) against bytes that are known
exactly.

    python kv_cache_vector_05_amd/copy_probe.py [--mib 1024] [--reps 3]

Each repetition copies --mib MiB from one device buffer into another
(one read and one write of that many bytes).
"""
from __future__ import annotations

import argparse
import sys


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        print("copy_probe needs a GPU", file=sys.stderr)
        return 1
    n = args.mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    # event-timed read-and-write (copy), write-only (fill) and read-only (sum)
    # rates, for context next to the kernels' algorithmic rates
    nbytes = n * 4
    for label, fn, moved in (("copy", lambda: dst.copy_(src), 2 * nbytes),
                             ("fill", lambda: dst.fill_(2.0), nbytes),
                             ("sum", lambda: src.sum(), nbytes)):
        fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(args.reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / args.reps
        print(f"{label}: {moved / ms / 1e6:.0f} GB/s ({ms * 1e3:.0f} us per {moved / 2**20:.0f} MiB)", flush=True)
    print(f"copied {args.mib} MiB x {args.reps}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
