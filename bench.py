#!/usr/bin/env python3
"""Throughput of the attention hot path on one MI355X.

One step = one forward (exattn_fwd) and one backward (exattn_bwd: delta, dK/dV kernel, dQ
kernel) over the synthetic workload B=2, S=8192, H=32 (Hkv=32), D=128, non-causal, bf16,
with q, k, v, dout ~ N(0,1) already resident in HBM. The FLOP count is algorithmic: 4*D
per visible (query, key) pair for the forward and 10*D for the backward (five products).
Per kernel: forward 4*D (S, PV); dK/dV kernel 8*D (S, dP, dV, dK); dQ kernel 2*D (the dQ
product; it also recomputes S and dP, 4*D more, which is overhead of the split and not
counted as algorithmic work).

Prints one JSON line. Per-kernel durations come from HIP events the library records
around each of its launches on the launch stream during the timed region.

After the timed steps, and outside them, the fp8 forward (exattn_fwd_fp8, e4m3 inputs with
per-tensor descales) is timed on the same shape and reported under "fp8_forward" against
the dense fp8 MFMA peak; it does not enter `value`.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-fp8]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd & bwd TFLOP/s (bf16, B2 S8192 H32 D128) + % of MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 dense bf16 FLOP/clk x 2.4 GHz (published 2.5 PFLOP/s)
PEAK_FP8_TFLOPS = 5033.2    # 256 CU x 8192 dense fp8 FLOP/clk x 2.4 GHz (published 5.0 PFLOP/s)
PEAK_HBM_GBS = 8000.0
B, S, H, HKV, D = 2, 8192, 32, 32, 128
PROFILE_DIR = os.path.join(ROOT, "profiles")


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_40_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from committed PMC counters, or None when the
    kernel sources changed since they were taken."""
    try:
        with open(os.path.join(PROFILE_DIR, f"{kernel}_b2_s8192_h32_d128_pmc.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def _pin_blas():
    """Worker initialiser: one BLAS thread per worker process, so the core count is exact."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _oracle_unit(seed):
    """One whole (batch, head) unit of the benchmark workload through the float64 oracle,
    forward and backward. Returns (FLOP, seconds)."""
    import numpy as np  # noqa: F401

    import oracle
    from exact_attention_40_amd import workloads

    p = workloads.dense(1, S, S, 1, 1, D, seed=seed)
    q, k, v, do = (t.double().numpy() for t in (p.q, p.k, p.v, p.dout))
    t0 = time.perf_counter()
    oracle.attention_forward(q, k, v)
    oracle.attention_backward(q, k, v, do)
    return 14.0 * D * S * S, time.perf_counter() - t0


def _oracle_long_rows():
    """The long-sequence workload (B1 S61380 H32 D128 causal) as its GPU test samples it:
    64 query rows through the oracle's row forward and row dQ. Returns (pairs, FLOP,
    seconds); the FLOP count is 8*D per visible pair (forward 4*D, dP and dQ 4*D)."""
    import numpy as np

    import oracle
    from exact_attention_40_amd import workloads

    p = workloads.long_causal()
    Sl = p.q.shape[1]
    rng = np.random.default_rng(5001)
    rows = np.array([0, Sl - 1, 127, 128, 61311, 61312] + sorted(rng.choice(Sl, 58, replace=False).tolist()))
    heads = rng.integers(0, 32, size=len(rows))
    scale = p.softmax_scale
    pairs = 0
    t0 = time.perf_counter()
    for h in np.unique(heads):
        rr = rows[heads == h]
        q = p.q[0, :, h].double().numpy()
        k = p.k[0, :, h].double().numpy()
        v = p.v[0, :, h].double().numpy()
        do = p.dout[0, :, h].double().numpy()
        oracle.rows_forward(q[rr], k, v, rr, scale, True)
        oracle.rows_backward_dq(q[rr], k, v, do[rr], rr, scale, True)
        pairs += int(np.sum(rr + 1))
    return pairs, 8.0 * D * pairs, time.perf_counter() - t0


def cpu_baseline(max_units=64, target_seconds=10.0):
    """The float64 oracle on a bounded sample of the benchmark workload, on the host cores:
    one worker process per whole (batch, head) unit (S=8192 keys, forward and backward),
    each worker's BLAS pinned to one thread, as many workers as usable cores (at most 16,
    the host share of one GPU). Units are submitted in rounds of one per worker until about
    `target_seconds` have passed. Also times the long-sequence workload's 64 sampled rows
    and extrapolates, at that sample's rate, to the whole problem (labelled as such)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    import numpy as np

    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    rng = np.random.default_rng(9)
    flops = 0.0
    units = 0
    t0 = time.perf_counter()
    with ProcessPoolExecutor(max_workers=cores, mp_context=mp.get_context("spawn"),
                             initializer=_pin_blas) as ex:
        while units < max_units and time.perf_counter() - t0 < target_seconds:
            n = min(cores, max_units - units)
            for f, _ in ex.map(_oracle_unit, [int(x) for x in rng.integers(1 << 30, size=n)]):
                flops += f
            units += n
        wall = time.perf_counter() - t0
        fut = ex.submit(_oracle_long_rows)
        pairs, lflops, lsec = fut.result()
    full_flops = 14.0 * D * 1883782890 * 32   # long workload: 30.86 + 77.16 TFLOP
    return {"value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{units} whole (batch, head) units of B2 S8192 H32 D128 non-causal, "
                      f"forward + backward in float64, one process per unit on {cores} cores "
                      f"with one BLAS thread each, {wall:.1f} s wall",
            "long_causal_rows": {
                "sample": "B1 S61380 H32 D128 causal: the 64 query rows the GPU test samples, "
                          "row forward and row dQ in float64, one core",
                "seconds": round(lsec, 2), "pairs": pairs,
                "TFLOP/s": round(lflops / lsec / 1e12, 6),
                "extrapolated_full_problem_seconds": round(full_flops / (lflops / lsec), 0),
                "extrapolation": "whole forward + backward (30.86 + 77.16 TFLOP) at the "
                                 "sample's measured per-FLOP rate on one core; not measured"}}


def device_info(dev):
    """CU count and top shader clock as read on this machine, next to the nominal values
    the peaks use (256 CUs, 2.4 GHz). The clock comes from the amdgpu driver's DPM table in
    sysfs (the highest listed level); null when it cannot be read."""
    import glob
    import re

    import torch

    props = torch.cuda.get_device_properties(dev)
    mhz = None
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            levels = [int(m) for m in re.findall(r"(\d+)\s*Mhz", open(path).read(), flags=re.I)]
        except OSError:
            continue
        if levels:
            mhz = max(mhz or 0, max(levels))
    return {"name": props.name, "arch": getattr(props, "gcnArchName", None),
            "cus": props.multi_processor_count, "max_sclk_mhz": mhz,
            "nominal": {"cus": 256, "sclk_mhz": 2400}}


def fp8_forward(api, workloads, dev, flops, steps, warmup):
    """Kernel time of exattn_fwd_fp8 on the same shape (e4m3 q, k, v ~ quantised N(0,1))."""
    import torch

    p = workloads.fp8_dense(B, S, S, H, HKV, D, seed=3002)
    q, k, v = (t.to(dev) for t in (p.q, p.k, p.v))
    run = lambda: api.exattn_fwd_fp8(q, k, v, p.q_descale, p.k_descale, p.v_descale)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    api.timing_enable(True)
    api.timing_read()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    kern = api.timing_read()
    api.timing_enable(False)
    t, c = kern["exattn_fwd_fp8_kernel"]
    ms = t / c
    tf = flops / (ms * 1e-3) / 1e12
    return {"kernel": "exattn_fwd_fp8_kernel", "ms": round(ms, 4), "TFLOP/s": round(tf, 1),
            "peak": PEAK_FP8_TFLOPS, "frac_of_fp8_mfma_peak": round(tf / PEAK_FP8_TFLOPS, 4),
            "dtype": "e4m3 in, fp32 accumulate, bf16 out"}


def side_measurements(api, dev, q, k, v, do, steps, warmup):
    """Outside the timed region: the eager-rescale forward (fwd_variant 1) against the
    default lazy one, and the fused backward (bwd_variant 1), whose dQ-reduce pass is an
    HBM-bound conversion of the fp32 accumulator."""
    import torch

    res = {}
    for name, fv in (("lazy", 0), ("eager", 1)):
        for _ in range(warmup):
            api.exattn_fwd(q, k, v, variant=fv)
        torch.cuda.synchronize()
        api.timing_read()
        for _ in range(steps):
            api.exattn_fwd(q, k, v, variant=fv)
        torch.cuda.synchronize()
        t, c = api.timing_read()["exattn_fwd_kernel"]
        res[name] = t / c
    out, lse = api.exattn_fwd(q, k, v)
    for _ in range(2):
        api.exattn_bwd(q, k, v, out, do, lse, variant=1)
    torch.cuda.synchronize()
    api.timing_read()
    for _ in range(3):
        api.exattn_bwd(q, k, v, out, do, lse, variant=1)
    torch.cuda.synchronize()
    kern = api.timing_read()
    return res, {n: ms / c for n, (ms, c) in kern.items()}


def stored_ds_steps(api, q, k, v, do, steps, warmup):
    """Outside the timed region: whole steps (forward + backward variant 3, whose dK/dV
    kernel stores dS and whose dQ pass is dS K from it) timed like the benchmark's own
    steps, with the per-kernel averages."""
    import torch

    def step():
        out, lse = api.exattn_fwd(q, k, v)
        api.exattn_bwd(q, k, v, out, do, lse, variant=3)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    api.timing_read()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    kern = api.timing_read()
    return t0.elapsed_time(t1) / steps, {n: ms / c for n, (ms, c) in kern.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    # the CPU baseline runs first, before this process touches the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline()

    import torch

    from exact_attention_40_amd import api, workloads

    dev = torch.device("cuda:0")
    p = workloads.dense(B, S, S, H, HKV, D, seed=3001)
    q, k, v, do = (t.to(dev) for t in (p.q, p.k, p.v, p.dout))
    del p
    stream = torch.cuda.current_stream(dev)
    pairs = B * H * S * S
    fwd_flops, bwd_flops = 4.0 * D * pairs, 10.0 * D * pairs

    def step():
        out, lse = api.exattn_fwd(q, k, v)
        dq, dk, dv = api.exattn_bwd(q, k, v, out, do, lse)
        return out, dq

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: whole steps, with per-call and per-kernel HIP events on the stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    api.timing_enable(True)
    api.timing_read()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        out, lse = api.exattn_fwd(q, k, v)
        ev[i][1].record(stream)
        api.exattn_bwd(q, k, v, out, do, lse)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = api.timing_read()
    api.timing_enable(False)

    fwd_ms = sum(a.elapsed_time(b) for a, b, _ in ev) / args.steps
    bwd_ms = sum(b.elapsed_time(c) for _, b, c in ev) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    value = (fwd_flops + bwd_flops) / (ms_per_step * 1e-3) / 1e12
    kavg = {n: ms / cnt for n, (ms, cnt) in kern.items()}

    # algorithmic and executed FLOP per launch of each matrix kernel
    per_kernel = {
        "exattn_fwd_kernel": (4.0 * D * pairs, 4.0 * D * pairs),
        "exattn_bwd_dkdv_kernel": (8.0 * D * pairs, 8.0 * D * pairs),
        "exattn_bwd_dq_kernel": (2.0 * D * pairs, 6.0 * D * pairs),
        "exattn_bwd_fused_kernel": (10.0 * D * pairs, 10.0 * D * pairs),
    }
    kernels = {}
    for name, (alg, exe) in per_kernel.items():
        if name in kavg:
            kernels[name] = {"ms": round(kavg[name], 4),
                             "algorithmic_TFLOP/s": round(alg / (kavg[name] * 1e-3) / 1e12, 1),
                             "executed_TFLOP/s": round(exe / (kavg[name] * 1e-3) / 1e12, 1)}
    dominant = max(kernels, key=lambda n: kavg[n])
    alg = per_kernel[dominant][0]
    achieved = alg / (kavg[dominant] * 1e-3) / 1e12
    traffic = measured_traffic(dominant)
    api.timing_enable(True)
    fwd_var, fused = side_measurements(api, dev, q, k, v, do, min(args.steps, 10), args.warmup)
    sds_ms, sds = stored_ds_steps(api, q, k, v, do, min(args.steps, 10), args.warmup)
    api.timing_enable(False)
    side = {}
    for name, nbytes, src in (
            ("exattn_bwd_delta_kernel", 2 * 2 * B * S * H * D + 4 * B * H * S * 3, kavg),
            ("exattn_bwd_dq_reduce_kernel", 4 * B * S * H * D + 2 * B * S * H * D, fused)):
        if name in src:
            gbs = nbytes / (src[name] * 1e-3) / 1e9
            side[name] = {"ms": round(src[name], 4), "bytes": nbytes, "GB/s": round(gbs, 1),
                          "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 3)}
    side["exattn_bwd_dq_reduce_kernel"]["measured_in"] = (
        "backward variant 1 (fused kernel with fp32 dQ atomics), outside the timed region")
    ds_bytes = B * H * (S // 64) * (S // 128) * 16384
    sds_bwd = sum(t for n, t in sds.items() if n != "exattn_fwd_kernel")
    stored = {"step_ms": round(sds_ms, 4), "TFLOP/s": round((fwd_flops + bwd_flops) / sds_ms / 1e9, 1),
              "fwd_kernel_ms": round(sds.get("exattn_fwd_kernel", float("nan")), 4),
              "bwd_ms": round(sds_bwd, 4),
              "kernels_avg_ms": {n: round(t, 4) for n, t in sds.items()},
              "ds_bytes": ds_bytes,
              "note": ("backward variant 3 (dS stored by the dK/dV kernel, dQ = dS K from it), "
                       "whole steps outside the timed region; not the default")}
    if "exattn_bwd_dq_ds_kernel" in sds:
        gbs = (ds_bytes + 2 * B * S * H * D) / (sds["exattn_bwd_dq_ds_kernel"] * 1e-3) / 1e9
        stored["dq_ds_GB/s"] = round(gbs, 1)
        stored["dq_ds_frac_of_hbm_peak"] = round(gbs / PEAK_HBM_GBS, 3)
    lazy_eager = {"lazy_ms": round(fwd_var["lazy"], 4), "eager_ms": round(fwd_var["eager"], 4),
                  "eager_over_lazy": round(fwd_var["eager"] / fwd_var["lazy"], 4),
                  "fused_backward_kernel_ms": round(fused.get("exattn_bwd_fused_kernel", float("nan")), 4)}

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "exact attention forward + backward, B=2 S=8192 H=32 Hkv=32 D=128, "
                               "non-causal, bf16 in / fp32 accumulate, q,k,v,dout ~ N(0,1)",
                   "batch": B, "seq_len": S, "heads": H, "kv_heads": HKV, "head_dim": D,
                   "causal": False, "parallelism": "single GPU"},
        "frac_of_mfma_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd": {"ms": round(fwd_ms, 4), "TFLOP/s": round(fwd_flops / fwd_ms / 1e9, 1),
                "frac_of_mfma_peak": round(fwd_flops / fwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4)},
        "bwd": {"ms": round(bwd_ms, 4), "TFLOP/s": round(bwd_flops / bwd_ms / 1e9, 1),
                "frac_of_mfma_peak": round(bwd_flops / bwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4)},
        "device": device_info(dev),
        "kernels_avg_ms": {n: round(t, 4) for n, t in kavg.items()},
        "kernels": kernels,
        "side_passes": side,
        "forward_rescale": lazy_eager,
        "stored_ds_backward": stored,
        "roofline": {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "traffic_note": ("estimate: rocprofv3 FETCH_SIZE and WRITE_SIZE per launch, "
                                      "each scaled by the same counter's reading on a plain copy "
                                      "of known size; null once the kernel sources change"),
                     "algorithmic_flops_per_launch": alg},
    }
    if not args.no_fp8:
        rec["fp8_forward"] = fp8_forward(api, workloads, dev, fwd_flops, args.steps, args.warmup)
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
