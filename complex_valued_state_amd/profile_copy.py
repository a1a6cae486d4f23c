"""A plain device-to-device copy of known size, for calibrating HBM byte counters.

    rocprofv3 --pmc FETCH_SIZE -- python3 -m complex_valued_state_amd.profile_copy

Copies a 1 GiB float32 buffer into another 1 GiB buffer REPS times.  Each copy
kernel reads exactly 1 GiB and writes exactly 1 GiB from/to HBM (the buffers are
4x larger than the on-package caches), so the FETCH_SIZE / WRITE_SIZE values a
counter run reports for it give the factor between the counters' units and real
bytes on this machine.
"""
import sys

BYTES = 1 << 30
REPS = 3


def main() -> int:
    import torch
    assert torch.cuda.is_available()
    src = torch.ones(BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(REPS):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {BYTES} bytes x {REPS}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
