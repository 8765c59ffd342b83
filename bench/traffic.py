"""HBM traffic per kernel launch from rocprofv3 counter passes.

Inputs are the counter_collection CSVs of four `rocprofv3 --pmc` runs: FETCH_SIZE and
WRITE_SIZE (KiB per dispatch) over the benchmark, and the same two counters over
`copy_probe` (copies of known size). The elementwise copy, whose lanes move 16 contiguous
bytes like the attention kernels' tile loads, gives the factor between counter bytes and
bytes moved; the runtime's buffer copy gives a second factor, recorded beside it as a
check. Each benchmark kernel is scaled by it and averaged over its first FIRST dispatches
(the benchmark's warm-up and timed steps, before its side measurements run other
variants). The result is written as JSON next to the kernel source hash that bench.py
checks.

    python bench/traffic.py BENCH_FETCH.csv BENCH_WRITE.csv \
        COPY_FETCH.csv COPY_WRITE.csv COPY_MIB OUT_DIR [FIRST]
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
    "exattn_bwd_dkdv_ds_kernel": "bwd_kv_kernel",      # the instance that also stores dS
    "exattn_bwd_dq_kernel": "bwd_dq_kernel",
    "exattn_bwd_dq_ds_kernel": "bwd_dq_ds_kernel",
    "exattn_bwd_delta_kernel": "delta_kernel",
    "exattn_fwd_fp8_kernel": "fwd_fp8_kernel",
}


def matches(kernel_name, template):
    """True when `kernel_name` (demangled or Itanium-mangled) is an instance of exattn::`template`."""
    return (f"exattn::{template}<" in kernel_name
            or f"N6exattn{len(template)}{template}I" in kernel_name
            or f"ZN6exattn{len(template)}{template}I" in kernel_name)


def stores_ds(kernel_name):
    """True for the dK/dV kernel instance whose last template argument (store dS) is true."""
    return kernel_name.endswith("Lb1EEEvNS_7BwdArgsE") or kernel_name.endswith(", true>(exattn::BwdArgs)")


def kernel_key(kernel_name):
    """The library timing name of a kernel instance name, or None for other kernels."""
    for k, t in KERNELS.items():
        if matches(kernel_name, t):
            if t == "bwd_kv_kernel":
                return "exattn_bwd_dkdv_ds_kernel" if stores_ds(kernel_name) else "exattn_bwd_dkdv_kernel"
            return k
    return None


def source_hash():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    h = hashlib.sha256()
    csrc = os.path.join(root, "exact_attention_40_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def per_kernel(path, counter, first=None):
    """Mean counter value (KiB) per dispatch over each kernel's first `first` dispatches
    (all when None), by kernel name."""
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        vals[r["Dispatch_Id"]][counter] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for d in sorted(vals, key=int):
        out[names[d]].append(vals[d][counter])
    return {k: sum(v[:first]) / len(v[:first]) for k, v in out.items()}


def copy_factor(path, counter, copy_bytes, kind):
    """Bytes moved per counter byte for the copy kernel of `kind` ("elementwise": the
    16-byte-per-lane add of zero; "runtime": the runtime's buffer copy), over the dispatches
    that move the whole buffer (the probe's result check also runs a tiny runtime copy)."""
    want = "CUDAFunctorOnSelf_add" if kind == "elementwise" else "__amd_rocclr_copyBuffer"
    vals = collections.defaultdict(float)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter and want in r["Kernel_Name"]:
            vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {kind} copy kernel in {path}")
    big = [v for v in vals.values() if v >= max(vals.values()) / 2]
    return copy_bytes / (sum(big) / len(big) * 1024)


def main():
    bf, bw, cf, cw, mib, out_dir = sys.argv[1:7]
    first = int(sys.argv[7]) if len(sys.argv) > 7 else None
    copy_bytes = int(mib) * (1 << 20)
    fscale = copy_factor(cf, "FETCH_SIZE", copy_bytes, "elementwise")
    wscale = copy_factor(cw, "WRITE_SIZE", copy_bytes, "elementwise")
    fscale_rt = copy_factor(cf, "FETCH_SIZE", copy_bytes, "runtime")
    wscale_rt = copy_factor(cw, "WRITE_SIZE", copy_bytes, "runtime")
    fetch, write = per_kernel(bf, "FETCH_SIZE", first), per_kernel(bw, "WRITE_SIZE", first)
    shash = source_hash()
    for name in KERNELS:
        fk = [v for k, v in fetch.items() if kernel_key(k) == name]
        wk = [v for k, v in write.items() if kernel_key(k) == name]
        if not fk or not wk:
            continue
        rec = {
            "kernel": name,
            "workload": "B=2 S=8192 H=32 Hkv=32 D=128 non-causal "
                        + ("e4m3" if name == "exattn_fwd_fp8_kernel" else "bf16"),
            "fetch_bytes_per_launch": sum(fk) / len(fk) * 1024 * fscale,
            "write_bytes_per_launch": sum(wk) / len(wk) * 1024 * wscale,
            "copy_calibration": {"bytes": copy_bytes, "kernel": "elementwise 16 B per lane",
                                 "fetch_factor": fscale, "write_factor": wscale,
                                 "runtime_copy_fetch_factor": fscale_rt,
                                 "runtime_copy_write_factor": wscale_rt},
            "dispatches_averaged": first,
            "source_hash": shash,
        }
        rec["hbm_bytes_per_launch"] = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
        path = os.path.join(out_dir, f"{name}_b2_s8192_h32_d128_pmc.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(path, json.dumps(rec))


if __name__ == "__main__":
    main()
