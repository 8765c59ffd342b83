"""Per-kernel clock, MFMA, LDS and instruction-mix figures from rocprofv3 counter passes over
the benchmark (written by profile_bench.sh under PROF_DIR/util, PROF_DIR/lds and, when
present, PROF_DIR/mix).

Normalisation (MI355X: 8 XCDs, 256 CUs, 4 SIMDs per CU):
- GRBM_GUI_ACTIVE is summed over the XCDs, so held clock = GRBM_GUI_ACTIVE / 8 / duration;
- SQ_VALU_MFMA_BUSY_CYCLES is summed over the SIMDs: MFMA busy = it / (4 * CUs) per cycle;
- SQ_LDS_IDX_ACTIVE is summed over the CUs: LDS active = it / CUs per cycle;
- SQ_INSTS_LDS_LOAD_BANDWIDTH counts 64-byte units loaded from LDS;
- mix pass: SQ_ACTIVE_INST_VALU and SQ_ACTIVE_INST_SCA over SQ_WAVE_CYCLES are the fractions
  of each wave's cycles spent issuing vector and scalar instructions;
  SQ_VALU_MFMA_COEXEC_CYCLES over SQ_VALU_MFMA_BUSY_CYCLES is the share of MFMA-busy cycles
  with vector instructions executing alongside; SQ_INSTS_VALU and SQ_INSTS_SALU over
  SQ_INSTS_MFMA count instructions per MFMA (all three counted the same way).

    python bench/counter_summary.py PROF_DIR OUT.md [CUS]
"""

import collections
import csv
import glob
import os
import sys

from traffic import KERNELS, kernel_key

PEAK_BF16_PER_CU_CLK = 4096.0   # dense bf16 FLOP per CU per clock


def load(pass_dir, skip=1, take=2):
    """{kernel: {counter: [(value, seconds)]}} over each kernel's dispatches skip .. skip +
    take - 1 in issue order: with --warmup 1 --steps 2, the benchmark's two timed steps
    (its side measurements, which run other variants, come after them)."""
    files = glob.glob(os.path.join(pass_dir, "*counter_collection.csv"))
    if not files:
        raise SystemExit(f"no counter CSV under {pass_dir}")
    rows = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(files[0])):
        k = kernel_key(r["Kernel_Name"])
        if k is None:
            continue
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        rows[k][r["Counter_Name"]].append((int(r["Dispatch_Id"]), float(r["Counter_Value"]), dur))
    out = {}
    for k, d in rows.items():
        out[k] = {c: [(v, t) for _, v, t in sorted(x)[skip:skip + take]] for c, x in d.items()}
    return out


def mean(xs):
    return sum(xs) / len(xs) if xs else float("nan")


def main():
    prof, out = sys.argv[1:3]
    cus = int(sys.argv[3]) if len(sys.argv) > 3 else 256
    util = load(os.path.join(prof, "util"))
    lds = load(os.path.join(prof, "lds"))
    mix = load(os.path.join(prof, "mix")) if os.path.isdir(os.path.join(prof, "mix")) else {}
    lines = [
        "# Clock, MFMA and LDS utilisation per kernel: fwd + bwd step, B=2 S=8192 H=32 Hkv=32 D=128 (non-causal, bf16)",
        "",
        "Three `rocprofv3 --pmc` passes over `python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline`",
        "(from the repository root; `bench/profile_bench.sh` runs them):",
        "",
        "```",
        "rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES -d gpurun_out/prof/util -o bench -f csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline",
        "rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS_LOAD_BANDWIDTH SQ_LDS_BANK_CONFLICT -d gpurun_out/prof/lds -o bench -f csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline",
        "rocprofv3 --pmc SQ_WAVE_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_SCA SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_MFMA -d gpurun_out/prof/mix -o bench -f csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline",
        "```",
        "",
        f"Averages over each kernel's two timed dispatches (after one warm-up call); {cus} CUs, 8",
        "XCDs. The stored-dS kernels (backward variant 3) come from the benchmark's side",
        "measurement, also its first two calls after one warm-up. \"held clock\" is",
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
    if mix:
        lines += [
            "",
            "Instruction mix (mix pass): \"VALU active\" and \"scalar active\" are the fractions of",
            "each wave's cycles spent issuing vector and scalar instructions; \"co-executed\" is the",
            "share of MFMA-busy cycles with vector work running alongside; the last two columns",
            "count vector and scalar instructions per MFMA instruction.",
            "",
            "| kernel | VALU active | scalar active | co-executed / MFMA busy | VALU per MFMA | scalar per MFMA |",
            "|---|---|---|---|---|---|",
        ]
        for k in KERNELS:
            if k not in mix:
                continue
            M = mix[k]
            g = lambda c: mean([v for v, _ in M.get(c, [])])  # noqa: E731
            w, mb, mi = g("SQ_WAVE_CYCLES"), g("SQ_VALU_MFMA_BUSY_CYCLES"), g("SQ_INSTS_MFMA")
            co = f"{100 * g('SQ_VALU_MFMA_COEXEC_CYCLES') / mb:.1f}%" if mb > 0 else "-"
            vp = f"{g('SQ_INSTS_VALU') / mi:.2f}" if mi > 0 else "-"
            sp = f"{g('SQ_INSTS_SALU') / mi:.2f}" if mi > 0 else "-"
            lines.append(f"| {k} | {100 * g('SQ_ACTIVE_INST_VALU') / w:.1f}% | "
                         f"{100 * g('SQ_ACTIVE_INST_SCA') / w:.1f}% | {co} | {vp} | {sp} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(open(out).read())


if __name__ == "__main__":
    main()
