"""The counter summary's normalisation on synthetic rocprofv3 counter files with known
answers (no GPU): held clock from GRBM_GUI_ACTIVE summed over 8 XCDs, MFMA busy from
SQ_VALU_MFMA_BUSY_CYCLES summed over 4 SIMDs per CU, LDS activity and read bandwidth per CU.
"""

import csv
import os

import sys

sys.path.insert(0, os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bench"))
import counter_summary  # noqa: E402  (bench/counter_summary.py, a script beside bench.py)
import traffic  # noqa: E402,F401  (bench/traffic.py)

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]
KNAME = "_ZN6exattn13bwd_dq_kernelIDF16bLi128ELb0ELi0ELb0EEEvNS_7BwdArgsE"


def _write(path, counters, cus, clock_hz, dur_s, dispatches=3):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d in range(1, dispatches + 1):
            start = 10**9 * d
            end = start + int(dur_s * 1e9)
            cycles = clock_hz * dur_s
            for name, per_cycle in counters.items():
                if name == "GRBM_GUI_ACTIVE":
                    value = cycles * 8                       # summed over the XCDs
                elif name == "SQ_VALU_MFMA_BUSY_CYCLES":
                    value = per_cycle * cycles * 4 * cus     # summed over the SIMDs
                elif name == "SQ_INSTS_LDS_LOAD_BANDWIDTH":
                    value = per_cycle * cycles * cus / 64    # 64-byte units
                else:
                    value = per_cycle * cycles * cus         # summed over the CUs
                row = {k: 0 for k in FIELDS}
                row.update(Dispatch_Id=d, Kernel_Name=KNAME, Counter_Name=name,
                           Counter_Value=value, Start_Timestamp=start, End_Timestamp=end)
                w.writerow(row)


def test_counter_summary_normalisation(tmp_path, monkeypatch):
    cus, clk, dur = 256, 1.8e9, 2.5e-3
    _write(tmp_path / "util", {"GRBM_GUI_ACTIVE": 1, "SQ_VALU_MFMA_BUSY_CYCLES": 0.625,
                               "SQ_BUSY_CYCLES": 1}, cus, clk, dur)
    _write(tmp_path / "lds", {"GRBM_GUI_ACTIVE": 1, "SQ_LDS_IDX_ACTIVE": 0.375,
                              "SQ_INSTS_LDS_LOAD_BANDWIDTH": 96.0, "SQ_LDS_BANK_CONFLICT": 0},
           cus, clk, dur)
    out = tmp_path / "out.md"
    monkeypatch.setattr("sys.argv", ["x", str(tmp_path), str(out), str(cus)])
    counter_summary.main()
    row = [l for l in out.read_text().splitlines() if l.startswith("| exattn_bwd_dq_kernel")]
    assert len(row) == 1
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    assert cells[1] == "2.500"                 # ms
    assert cells[2] == "1.80"                  # held clock, GHz
    assert cells[3] == "62.5%"                 # MFMA busy
    assert cells[4] == f"{cus * 4096 * 1.8e9 / 1e12:.0f}"   # peak at the held clock
    assert cells[5] == "37.5%"                 # LDS active
    assert cells[6] == "96.0"                  # LDS read bytes per clock per CU


def _write_counts(path, rows, counter):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, (name, kib) in enumerate(rows, 1):
            row = {k: 0 for k in FIELDS}
            row.update(Dispatch_Id=d, Kernel_Name=name, Counter_Name=counter, Counter_Value=kib)
            w.writerow(row)


def test_traffic_scaling_and_dispatch_window(tmp_path, monkeypatch):
    """Known answers for the traffic step: the elementwise copy sets the scale, the runtime
    copy is only recorded, small dispatches do not dilute either factor, and only each
    kernel's first dispatches are averaged."""
    import json
    import traffic

    mib = 64
    copy_kib = mib * 1024
    ew = "void at::native::vectorized_elementwise_kernel<4, at::native::CUDAFunctorOnSelf_add<float>>"
    fill = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>>"
    rt = "__amd_rocclr_copyBuffer"
    # read counter: 1/2 of the bytes for the elementwise copy, 3/8 for the runtime copy; a
    # tiny runtime copy (the probe's result check) and a fill are left out of the factors
    _write_counts(tmp_path / "cf.csv", [(rt, copy_kib * 3 / 8)] * 3 + [(rt, 1.5), (fill, 10)]
                  + [(ew, copy_kib / 2)] * 3, "FETCH_SIZE")
    _write_counts(tmp_path / "cw.csv", [(rt, copy_kib)] * 3 + [(rt, 0.03), (fill, copy_kib)]
                  + [(ew, copy_kib)] * 3, "WRITE_SIZE")
    # delta kernel: three main-loop dispatches, then two with extra writes that must be left out
    _write_counts(tmp_path / "bf.csv", [(KNAME.replace("13bwd_dq_kernel", "12delta_kernel"), 1000)] * 5,
                  "FETCH_SIZE")
    _write_counts(tmp_path / "bw.csv", [(KNAME.replace("13bwd_dq_kernel", "12delta_kernel"), w)
                                        for w in (10, 10, 10, 5000, 5000)], "WRITE_SIZE")
    monkeypatch.setattr("sys.argv", ["x", str(tmp_path / "bf.csv"), str(tmp_path / "bw.csv"),
                                     str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), str(mib),
                                     str(tmp_path), "3"])
    traffic.main()
    rec = json.load(open(tmp_path / "exattn_bwd_delta_kernel_b2_s8192_h32_d128_pmc.json"))
    assert rec["copy_calibration"]["fetch_factor"] == 2.0
    assert abs(rec["copy_calibration"]["runtime_copy_fetch_factor"] - 8 / 3) < 1e-12
    assert rec["copy_calibration"]["runtime_copy_write_factor"] == 1.0
    assert rec["fetch_bytes_per_launch"] == 1000 * 1024 * 2.0
    assert rec["write_bytes_per_launch"] == 10 * 1024


def test_kernel_key_separates_the_ds_storing_instance():
    """The dK/dV kernel that also stores dS (last template argument true) gets its own
    row, in mangled and demangled spellings; other instances keep theirs."""
    import traffic

    m = "_ZN6exattn13bwd_kv_kernelIDF16bLi128ELb0ELi0ELb0ELb{}EEEvNS_7BwdArgsE"
    assert traffic.kernel_key(m.format(0)) == "exattn_bwd_dkdv_kernel"
    assert traffic.kernel_key(m.format(1)) == "exattn_bwd_dkdv_ds_kernel"
    d = "void exattn::bwd_kv_kernel<__bf16, 128, false, 0, false, {}>(exattn::BwdArgs)"
    assert traffic.kernel_key(d.format("false")) == "exattn_bwd_dkdv_kernel"
    assert traffic.kernel_key(d.format("true")) == "exattn_bwd_dkdv_ds_kernel"
    assert traffic.kernel_key("_ZN6exattn16bwd_dq_ds_kernelIDF16bLi128ELb0EEEvNS_7BwdArgsE") == \
        "exattn_bwd_dq_ds_kernel"
    assert traffic.kernel_key(KNAME) == "exattn_bwd_dq_kernel"
    assert traffic.kernel_key("__amd_rocclr_copyBuffer") is None


def test_bench_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    """bench.py reports roofline.traffic from a committed counter record only while the
    record's kernel source hash is the sources' hash (the same hash the traffic step
    writes); a stale or missing record gives null."""
    import json
    import bench

    assert bench.kernel_source_hash() == traffic.source_hash()
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    name = "exattn_bwd_dkdv_kernel"
    assert bench.measured_traffic(name) is None                       # no record
    path = tmp_path / f"{name}_b2_s8192_h32_d128_pmc.json"
    path.write_text(json.dumps({"source_hash": bench.kernel_source_hash(),
                                "hbm_bytes_per_launch": 1234.5}))
    assert bench.measured_traffic(name) == 1234.5                     # current record
    path.write_text(json.dumps({"source_hash": "0" * 16, "hbm_bytes_per_launch": 1234.5}))
    assert bench.measured_traffic(name) is None                       # stale record
