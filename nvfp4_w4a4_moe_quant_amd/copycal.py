"""Calibration workload for HBM byte counters: a plain device-to-device copy of
a known size, so that a FETCH_SIZE / WRITE_SIZE counter pass over it gives the
factor between what the counters report and the bytes actually moved.

    python -m nvfp4_w4a4_moe_quant_amd.copycal [MiB]

Runs dst = src + 1 three times, each one elementwise kernel dispatch that
reads MiB mebibytes and writes MiB mebibytes.  The buffers are larger than
the last-level caches, so every byte goes to HBM.
"""
import sys

import torch


def main(mib: int = 1024) -> None:
    dev = torch.device("cuda:0")
    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.add(src, 1, out=dst)
    torch.cuda.synchronize()
    assert int(dst[-1].item()) == n
    print(f"copied {mib} MiB x3", flush=True)


if __name__ == "__main__":
    main(int(sys.argv[1]) if len(sys.argv) > 1 else 1024)
