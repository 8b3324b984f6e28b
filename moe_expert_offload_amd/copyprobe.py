"""Plain device copy of a known size, for calibrating HBM traffic counters.

    python -m moe_expert_offload_amd.copyprobe [MiB]

Copies a MiB-sized buffer (default 1024) device to device three times.  Run it
under rocprofv3 --pmc FETCH_SIZE (or WRITE_SIZE): each copy moves exactly that
many bytes each way, so the counter's reading per dispatch divided into the
buffer size is the factor that turns the counter into bytes.
"""
import sys

import torch


def main():
    mib = int(sys.argv[1]) if len(sys.argv) > 1 else 1024
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB three times", flush=True)


if __name__ == "__main__":
    main()
