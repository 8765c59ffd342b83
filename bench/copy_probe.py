"""Plain device-to-device copy of a known size, used to calibrate the HBM byte counters
(FETCH_SIZE, WRITE_SIZE) that rocprofv3 reports for the attention kernels: the counters
read for this copy, divided by the bytes it must move, give the scale factor.

    python bench/copy_probe.py [MiB]
"""

import sys

import torch


def main():
    mib = int(sys.argv[1]) if len(sys.argv) > 1 else 512
    n = mib * (1 << 20) // 4
    x = torch.arange(n, device="cuda", dtype=torch.float32)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    assert torch.equal(x[-4:], y[-4:])
    print(f"copied {mib} MiB three times", flush=True)


if __name__ == "__main__":
    main()
