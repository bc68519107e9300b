"""Reference copy for calibrating HBM traffic counters.

    python -m decode_megakernel_cooperative_amd.copy_probe [--mib 1024] [--reps 3]

Runs `reps` device-to-device copies of exactly `mib` MiB on cuda:0 (one copy kernel each). Under
`rocprofv3 --pmc FETCH_SIZE` (then, in a run of its own, `--pmc WRITE_SIZE`) the per-dispatch
counter of these copies, set against the known byte count, gives the scale factor that turns the
same counter read on the decode kernel into HBM bytes.
"""
from __future__ import annotations

import argparse
import sys


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    import torch
    assert torch.cuda.is_available(), "the copy probe needs a GPU"
    n = args.mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {args.reps} x {n} bytes", file=sys.stderr, flush=True)
    return 0


if __name__ == "__main__":
    _rc = main()
    if _rc:
        sys.exit(_rc)
