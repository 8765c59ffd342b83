"""Per-kernel clock, MFMA and LDS utilisation from two rocprofv3 counter passes over the
benchmark (written by profile_bench.sh under PROF_DIR/util and PROF_DIR/lds).

Normalisation (MI355X: 8 XCDs, 256 CUs, 4 SIMDs per CU):
- GRBM_GUI_ACTIVE is summed over the XCDs, so held clock = GRBM_GUI_ACTIVE / 8 / duration;
- SQ_VALU_MFMA_BUSY_CYCLES is summed over the SIMDs: MFMA busy = it / (4 * CUs) per cycle;
- SQ_LDS_IDX_ACTIVE is summed over the CUs: LDS active = it / CUs per cycle;
- SQ_INSTS_LDS_LOAD_BANDWIDTH counts 64-byte units loaded from LDS.

    python bench/counter_summary.py PROF_DIR OUT.md [CUS]
"""

import collections
import csv
import glob
import os
import sys

from traffic import KERNELS, matches

PEAK_BF16_PER_CU_CLK = 4096.0   # dense bf16 FLOP per CU per clock


def short(name):
    for k, t in KERNELS.items():
        if matches(name, t):
            return k
    return None


def load(pass_dir, last=2):
    """{kernel: {counter: [(value, seconds)]}} over each kernel's last `last` dispatches."""
    files = glob.glob(os.path.join(pass_dir, "*counter_collection.csv"))
    if not files:
        raise SystemExit(f"no counter CSV under {pass_dir}")
    rows = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(files[0])):
        k = short(r["Kernel_Name"])
        if k is None:
            continue
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        rows[k][r["Counter_Name"]].append((int(r["Dispatch_Id"]), float(r["Counter_Value"]), dur))
    out = {}
    for k, d in rows.items():
        out[k] = {c: [(v, t) for _, v, t in sorted(x)[-last:]] for c, x in d.items()}
    return out


def mean(xs):
    return sum(xs) / len(xs) if xs else float("nan")


def main():
    prof, out = sys.argv[1:3]
    cus = int(sys.argv[3]) if len(sys.argv) > 3 else 256
    util = load(os.path.join(prof, "util"))
    lds = load(os.path.join(prof, "lds"))
    lines = [
        "# Clock, MFMA and LDS utilisation per kernel: fwd + bwd step, B=2 S=8192 H=32 Hkv=32 D=128 (non-causal, bf16)",
        "",
        "Two `rocprofv3 --pmc` passes over `python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline`",
        "(from the repository root; `bench/profile_bench.sh` runs them):",
        "",
        "```",
        "rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES -d gpurun_out/prof/util -o bench -f csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline",
        "rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS_LOAD_BANDWIDTH SQ_LDS_BANK_CONFLICT -d gpurun_out/prof/lds -o bench -f csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline",
        "```",
        "",
        f"Averages over each kernel's last two dispatches; {cus} CUs, 8 XCDs. \"held clock\" is",
        "GRBM_GUI_ACTIVE per XCD over the dispatch duration. \"MFMA busy\" is",
        "SQ_VALU_MFMA_BUSY_CYCLES per SIMD over those cycles; for the matrix kernels it equals",
        "the executed MFMA work (32 busy cycles per 32x32x16 MFMA). \"of held-clock peak\" is the",
        "same busy fraction read as a fraction of the dense peak at the held clock",
        f"({cus} CUs x {PEAK_BF16_PER_CU_CLK:.0f} bf16 FLOP/clk x held clock); the nominal peak assumes 2.4 GHz.",
        "Kernel durations under counter collection run longer than in the timed benchmark.",
        "",
        "| kernel | ms (counted run) | held clock GHz | MFMA busy | held-clock peak TFLOP/s | LDS active | LDS read B/clk/CU | LDS bank conflicts |",
        "|---|---|---|---|---|---|---|---|",
    ]
    for k in KERNELS:
        if k not in util:
            continue
        u = util[k]
        g = u["GRBM_GUI_ACTIVE"]
        dur = mean([t for _, t in g])
        cyc = mean([v / 8.0 for v, _ in g])
        clk = mean([v / 8.0 / t for v, t in g]) / 1e9
        mf = mean([v for v, _ in u.get("SQ_VALU_MFMA_BUSY_CYCLES", [])]) / (4 * cus) / cyc
        peak = cus * PEAK_BF16_PER_CU_CLK * clk * 1e9 / 1e12
        la = lb = bc = float("nan")
        if k in lds:
            L = lds[k]
            lcyc = mean([v / 8.0 for v, _ in L["GRBM_GUI_ACTIVE"]])
            la = mean([v for v, _ in L.get("SQ_LDS_IDX_ACTIVE", [])]) / cus / lcyc
            lb = mean([v for v, _ in L.get("SQ_INSTS_LDS_LOAD_BANDWIDTH", [])]) * 64 / cus / lcyc
            bc = mean([v for v, _ in L.get("SQ_LDS_BANK_CONFLICT", [])])
        mf_s = f"{100 * mf:.1f}%" if mf > 0 else "0"
        lines.append(f"| {k} | {dur * 1e3:.3f} | {clk:.2f} | {mf_s} | {peak:.0f} | "
                     f"{100 * la:.1f}% | {lb:.1f} | {bc:.0f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(open(out).read())


if __name__ == "__main__":
    main()
