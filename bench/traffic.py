"""HBM traffic per kernel launch from rocprofv3 counter passes.

Inputs are the counter_collection CSVs of four `rocprofv3 --pmc` runs: FETCH_SIZE and
WRITE_SIZE (KiB per dispatch) over the benchmark, and the same two counters over
`copy_probe` (a copy of known size). The copy gives the factor between counter bytes and
bytes moved; the benchmark's kernels are scaled by it and averaged per launch. The result
is written as JSON next to the kernel source hash that bench.py checks.

    python bench/traffic.py BENCH_FETCH.csv BENCH_WRITE.csv \
        COPY_FETCH.csv COPY_WRITE.csv COPY_MIB OUT_DIR
"""

import csv
import collections
import hashlib
import json
import os
import sys

KERNELS = {  # library timing name -> kernel template name (rocprofv3 may or may not demangle)
    "exattn_fwd_kernel": "fwd_kernel",
    "exattn_bwd_dkdv_kernel": "bwd_kv_kernel",
    "exattn_bwd_dq_kernel": "bwd_dq_kernel",
    "exattn_bwd_delta_kernel": "delta_kernel",
    "exattn_fwd_fp8_kernel": "fwd_fp8_kernel",
}


def matches(kernel_name, template):
    """True when `kernel_name` (demangled or Itanium-mangled) is an instance of exattn::`template`."""
    return (f"exattn::{template}<" in kernel_name
            or f"N6exattn{len(template)}{template}I" in kernel_name
            or f"ZN6exattn{len(template)}{template}I" in kernel_name)


def source_hash():
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    csrc = os.path.join(root, "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def per_kernel(path, counter):
    """Mean counter value (KiB) per dispatch, by kernel-name substring."""
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        vals[r["Dispatch_Id"]][counter] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for d, v in vals.items():
        out[names[d]].append(v[counter])
    return {k: sum(v) / len(v) for k, v in out.items()}


def main():
    bf, bw, cf, cw, mib, out_dir = sys.argv[1:7]
    copy_bytes = int(mib) * (1 << 20)
    cfetch = max(per_kernel(cf, "FETCH_SIZE").values()) * 1024
    cwrite = max(per_kernel(cw, "WRITE_SIZE").values()) * 1024
    fscale, wscale = copy_bytes / cfetch, copy_bytes / cwrite
    fetch, write = per_kernel(bf, "FETCH_SIZE"), per_kernel(bw, "WRITE_SIZE")
    shash = source_hash()
    for name, sub in KERNELS.items():
        fk = [v for k, v in fetch.items() if matches(k, sub)]
        wk = [v for k, v in write.items() if matches(k, sub)]
        if not fk or not wk:
            continue
        rec = {
            "kernel": name,
            "workload": "B=2 S=8192 H=32 Hkv=32 D=128 non-causal "
                        + ("e4m3" if name == "exattn_fwd_fp8_kernel" else "bf16"),
            "fetch_bytes_per_launch": sum(fk) / len(fk) * 1024 * fscale,
            "write_bytes_per_launch": sum(wk) / len(wk) * 1024 * wscale,
            "copy_calibration": {"bytes": copy_bytes, "fetch_factor": fscale, "write_factor": wscale},
            "source_hash": shash,
        }
        rec["hbm_bytes_per_launch"] = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
        path = os.path.join(out_dir, f"{name}_b2_s8192_h32_d128_pmc.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(path, json.dumps(rec))


if __name__ == "__main__":
    main()
