"""Writes the kernel-duration and HBM-traffic summary for profiles/ from the output of
profile_bench.sh (rocprofv3 kernel stats CSV and the per-kernel traffic JSON files).

    python bench/profile_summary.py PROF_DIR OUT.md [TIMED_STEPS [WARMUP]]
"""

import csv
import json
import os
import re
import sys

from traffic import KERNELS, kernel_key

MIN_BYTES = {  # algorithmic bytes per launch at B=2 S=8192 H=32 D=128 (bf16 tensors 134.2 MB, row vectors 2.1 MB)
    "exattn_fwd_kernel": ("q, k, v read 0.403 GB; out + lse written 0.136 GB", 0.4027, 0.1363),
    "exattn_bwd_dkdv_kernel": ("q, k, v, dout 0.537 GB + lse2, delta 0.004 GB read; dk, dv 0.268 GB written", 0.5411, 0.2684),
    "exattn_bwd_dq_kernel": ("q, k, v, dout 0.537 GB + stats 0.004 GB read; dq 0.134 GB written", 0.5411, 0.1342),
    "exattn_bwd_delta_kernel": ("out, dout 0.268 GB + lse read; delta, lse2 0.004 GB written", 0.2705, 0.0042),
    "exattn_fwd_fp8_kernel": ("e4m3 q, k, v read 0.201 GB; bf16 out + lse written 0.136 GB", 0.2013, 0.1363),
    "exattn_bwd_dkdv_ds_kernel": ("as dK/dV; written: dk, dv 0.268 GB + dS 8.590 GB", 0.5411, 8.8584),
    "exattn_bwd_dq_ds_kernel": ("dS 8.590 GB + k 0.134 GB read; dq 0.134 GB written", 8.7242, 0.1342),
}


def short(name):
    return kernel_key(name) or name


def timed_averages(prof, steps, warmup):
    """Average duration (ms) of each kernel instance over its dispatches warmup .. warmup +
    steps - 1 in issue order: the benchmark's timed steps (the trace also holds the warm-up
    calls and, after the timed steps, the side measurements of other variants)."""
    durs = {}
    for r in csv.DictReader(open(os.path.join(prof, "trace", "bench_kernel_trace.csv"))):
        durs.setdefault(r["Kernel_Name"], []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    out = {}
    for name, d in durs.items():
        sel = [x for _, x in sorted(d)][warmup:warmup + steps]
        if sel:
            out[name] = sum(sel) / len(sel) / 1e6
    return out


def main():
    prof, out = sys.argv[1:3]
    steps = int(sys.argv[3]) if len(sys.argv) > 3 else 20
    warmup = int(sys.argv[4]) if len(sys.argv) > 4 else 5
    rows = list(csv.DictReader(open(os.path.join(prof, "trace", "bench_kernel_stats.csv"))))
    timed = timed_averages(prof, steps, warmup)
    lines = [
        "# Kernel durations and HBM traffic: fwd + bwd step, B=2 S=8192 H=32 Hkv=32 D=128 (non-causal, bf16)",
        "",
        "Kernel trace (rocprofv3 `--kernel-trace --stats`) over the benchmark's warm-up and timed steps.",
        f"\"timed avg\" is the mean over each kernel instance's dispatches {warmup} .. {warmup + steps - 1} (the timed",
        "steps, from the per-dispatch trace; the side measurements of other variants come after",
        "them); it is the figure to compare with bench.py's in-process HIP-event timing.",
        "\"avg\" includes the first (cold) calls.",
        "",
        "Command (from the repository root; `bench/profile_bench.sh` runs all passes):",
        "",
        "```",
        f"rocprofv3 --kernel-trace --stats -d gpurun_out/prof/trace -o bench -f csv -- python3 bench.py --steps {steps} --warmup {warmup} --no-cpu-baseline",
        "```",
        "",
        "| kernel | instance | calls | timed avg ms | avg ms | min ms | max ms | share |",
        "|---|---|---|---|---|---|---|---|",
    ]
    for r in rows:
        t = timed.get(r["Name"])
        lines.append(f"| {short(r['Name'])} | `{r['Name']}` | {r['Calls']} | "
                     f"{'' if t is None else f'{t:.3f}'} | {float(r['AverageNs']) / 1e6:.3f} | "
                     f"{float(r['MinNs']) / 1e6:.3f} | {float(r['MaxNs']) / 1e6:.3f} | {float(r['Percentage']):.1f}% |")
    lines += [
        "",
        "HBM bytes per launch: `rocprofv3 --pmc FETCH_SIZE` and, in a second run, `--pmc WRITE_SIZE` over",
        "`python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline`, each scaled by the same counter over",
        "`python3 bench/copy_probe.py 512` (512 MiB copied three times by each of two kernels), and",
        "averaged over each kernel's first 3 dispatches (the benchmark's warm-up and timed steps).",
    ]
    recs = {}
    for k in KERNELS:
        p = os.path.join(prof, f"{k}_b2_s8192_h32_d128_pmc.json")
        if os.path.exists(p):
            recs[k] = json.load(open(p))
    if recs:
        cal = next(iter(recs.values()))["copy_calibration"]
        lines += [
            f"For the elementwise copy, whose lanes move 16 contiguous bytes like the attention kernels'",
            f"tile loads, FETCH_SIZE reads 1/{cal['fetch_factor']:.3f} of the copied bytes and WRITE_SIZE",
            f"1/{cal['write_factor']:.3f}; these factors scale the table. The runtime's buffer copy reads",
            f"1/{cal.get('runtime_copy_fetch_factor', float('nan')):.3f} and 1/{cal.get('runtime_copy_write_factor', float('nan')):.3f}.",
            "The per-kernel JSON files next to this one hold the numbers with the kernel source hash",
            f"bench.py checks ({next(iter(recs.values()))['source_hash']}).",
            "",
            "| kernel | read GB | written GB | read / minimum | written / minimum | algorithmic minimum |",
            "|---|---|---|---|---|---|",
        ]
        for k, r in recs.items():
            desc, mr, mw = MIN_BYTES[k]
            rd, wr = r["fetch_bytes_per_launch"] / 1e9, r["write_bytes_per_launch"] / 1e9
            lines.append(f"| {k} | {rd:.3f} | {wr:.3f} | {rd / mr:.2f} | {wr / mw:.2f} | {desc} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
