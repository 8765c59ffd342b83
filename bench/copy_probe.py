"""Plain device-to-device copies of a known size, used to calibrate the HBM byte counters
(FETCH_SIZE, WRITE_SIZE) that rocprofv3 reports for the attention kernels: the counters
read for a copy, divided by the bytes it must move, give the scale factor.

Two copies run, three times each: the runtime's own buffer copy (`copy_`), and an
elementwise kernel (`x + 0` into `y`) whose lanes load and store 16 contiguous bytes each,
the access width of the attention kernels' tile loads. The elementwise copy calibrates;
the buffer copy checks that the factor does not depend on the copying kernel.

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
    y.zero_()
    for _ in range(3):
        torch.add(x, 0.0, out=y)
    torch.cuda.synchronize()
    assert torch.equal(x[-4:], y[-4:])
    print(f"copied {mib} MiB three times by each of two kernels", flush=True)


if __name__ == "__main__":
    main()
