#!/bin/bash
# rocprofv3 passes over bench.py (kernel trace + stats, FETCH_SIZE, WRITE_SIZE, clock / MFMA
# and LDS utilisation counters, instruction mix) and over copy_probe (FETCH_SIZE and
# WRITE_SIZE) for the HBM-traffic calibration. Writes raw output, the per-kernel traffic JSON
# and the two summaries under gpurun_out/prof.
set -o pipefail
export TMPDIR=/tmp
R=${GRAFT_REPO_ROOT:-$(cd "$(dirname "$0")/.." && pwd)}
O=$R/gpurun_out/prof
mkdir -p $O
cd $R
echo "trace" && timeout -k 10 240 rocprofv3 --kernel-trace --stats -d $O/trace -o bench -f csv -- python3 bench.py --steps 20 --warmup 5 --no-cpu-baseline > $O/trace.log 2>&1 || exit 1
echo "fetch" && timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE -d $O/fetch -o bench -f csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline > $O/fetch.log 2>&1 || exit 1
echo "write" && timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE -d $O/write -o bench -f csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline > $O/write.log 2>&1 || exit 1
echo "copy fetch" && timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE -d $O/cfetch -o copy -f csv -- python3 bench/copy_probe.py 512 > $O/cfetch.log 2>&1 || exit 1
echo "copy write" && timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE -d $O/cwrite -o copy -f csv -- python3 bench/copy_probe.py 512 > $O/cwrite.log 2>&1 || exit 1
echo "util" && timeout -s KILL 120 rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES -d $O/util -o bench -f csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline > $O/util.log 2>&1 || exit 1
echo "lds" && timeout -s KILL 120 rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS_LOAD_BANDWIDTH SQ_LDS_BANK_CONFLICT -d $O/lds -o bench -f csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline > $O/lds.log 2>&1 || exit 1
echo "mix" && timeout -s KILL 120 rocprofv3 --pmc SQ_WAVE_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_SCA SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_MFMA -d $O/mix -o bench -f csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline > $O/mix.log 2>&1 || exit 1
python3 bench/traffic.py $(ls $O/fetch/*counter_collection.csv) $(ls $O/write/*counter_collection.csv) $(ls $O/cfetch/*counter_collection.csv) $(ls $O/cwrite/*counter_collection.csv) 512 $O 3
python3 bench/profile_summary.py $O $O/exattn_b2_s8192_h32_d128_kernel_stats.md 20 5
python3 bench/counter_summary.py $O $O/exattn_b2_s8192_h32_d128_counters.md
# the per-kernel JSON files and the summary land in gpurun_out/prof; copy them into profiles/
