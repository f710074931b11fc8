"""Benchmark of the batched Newton–Schulz orthogonalization on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--also NAME ...]

One step = one ns_orthogonalize call (normalisation + 5 quintic steps) over
the whole workload, inputs already resident in HBM.  Prints ONE JSON line.

value       effective bf16 TFLOP/s of the primary workload: dense-equivalent
            FLOPs 5 (4 m² n + 2 m³) per slice divided by the measured time
            (the comparison basis of the prime-rl NS microbenchmark table)
roofline    the dominant kernel (the update product) timed with HIP events
            around each of its launches on the launch stream, algorithmic
            FLOPs per launch / mean launch time, against the 2.5 PFLOP/s dense
            bf16 MFMA peak
cpu_baseline the fp64 CPU oracle on a bounded sample of the same workload
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import newton_schulz_07_amd as ns  # noqa: E402
from ns_inputs import WORKLOADS, make_workload  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0
STEPS_NS = 5
# the pages' own number for the 4096² symmetric NS on one H200 (prime-rl
# PR #3873, NS microbenchmark table, QuACK column): context, not the target
PAGES_H200_MS = {"lowrank64_4096x4096": 2.71, "experts128_1536x2048": 25.0, "square_8192x8192": 17.0,
                 "mlp_4096x14336": 7.07, "experts32_7168x2048": 33.0}


def kernel_source_hash():
    """Hash of the kernel sources: counter figures taken from another build
    of the kernels do not describe this one."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "newton_schulz_07_amd", "csrc")
    for name in ("ns_kernels.hip", "ns_layout.h", "ns_plan.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch from profiles/traffic.json (rocprofv3 FETCH_SIZE
    and WRITE_SIZE passes, scaled by a copy kernel of known size), or None when
    the kernels changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    ent = rec.get("kernels", {}).get(f"{workload}/{kernel}")
    if not ent:
        return None
    rd = ent["fetch_kb"] * 1024 * rec["copy_scale_fetch"]
    wr = ent["write_kb"] * 1024 * rec["copy_scale_write"]
    return {"bytes": rd + wr, "fetch_bytes": rd, "write_bytes": wr, "source": "profiles/traffic.json"}


def dense_eq_flops(batch, rows, cols, steps=STEPS_NS):
    m, n = min(rows, cols), max(rows, cols)
    return batch * steps * (4 * m * m * n + 2 * m ** 3)


def algorithmic_flops(batch, rows, cols):
    """Per launch: Gram m(m+1)n (one triangle incl. diagonal), polynomial
    m²(m+1), update 2 m² n."""
    m, n = min(rows, cols), max(rows, cols)
    return {"gram": batch * m * (m + 1) * n, "poly": batch * m * m * (m + 1), "update": batch * 2 * m * m * n}


def time_workload(name, steps, warmup, kernel_mask):
    w = WORKLOADS[name]
    x = make_workload(name)
    if x.dtype != torch.bfloat16:
        x = x.to(torch.bfloat16)
    dev = torch.device("cuda:0")
    xg = x.to(dev)
    out = torch.empty_like(xg)
    for _ in range(warmup):
        ns.orthogonalize(xg, out=out)
    torch.cuda.synchronize()
    ns.ns_timing_reset()
    ns.ns_timing_enable(kernel_mask)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        ns.orthogonalize(xg, out=out)
    stop.record()
    torch.cuda.synchronize()
    ns.ns_timing_enable(0)
    ms = start.elapsed_time(stop) / steps
    kernels = {}
    for kind, kname in ns.KIND_NAMES.items():
        tot, n = ns.ns_timing_query(kind)
        if n:
            kernels[kname] = {"mean_ms": tot / n, "launches": n}
    ns.ns_timing_reset()
    flops = dense_eq_flops(w.batch, w.rows, w.cols)
    eff = flops / (ms * 1e-3) / 1e12
    return {"name": name, "shape": list(w.shape), "ms_per_call": ms, "eff_tflops": eff,
            "pct_dense_bf16_peak": 100.0 * eff / PEAK_BF16_TFLOPS, "kernels": kernels,
            "config": ns.ns_query_last_config(), "x": x, "y": out}


def cpu_baseline(name, y_gpu, budget_s):
    """The fp64 oracle on whole slices of the workload, cycling through them,
    until ~budget_s seconds; each distinct slice is also compared with the GPU
    output."""
    from oracle import newton_schulz_batched  # CPU baseline leg only

    w = WORKLOADS[name]
    x = make_workload(name)
    if name == "iid_256x512":
        x = x.to(torch.bfloat16)
    xs = x.reshape(-1, w.rows, w.cols)
    try:
        from threadpoolctl import threadpool_info
        cores = max(int(i.get("num_threads", 1)) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    ys = y_gpu.reshape(-1, w.rows, w.cols)
    t0 = time.perf_counter()
    done = 0
    errs = []
    while True:
        i = done % xs.shape[0]
        ref = newton_schulz_batched(xs[i:i + 1].double().numpy())[0]
        if done < xs.shape[0]:
            got = ys[i].double().cpu().numpy()
            errs.append(float(np.linalg.norm(got - ref) / np.linalg.norm(ref)))
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = dense_eq_flops(done, w.rows, w.cols)
    distinct = min(done, xs.shape[0])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s (dense-equivalent)", "cores": cores, "kind": "oracle",
            "sample": f"{done} oracle call(s) on {distinct} distinct of the {xs.shape[0]} slice(s) of {name} "
                      f"({w.rows}x{w.cols}), fp64 numpy, {dt:.1f} s",
            "seconds_per_slice": dt / done, "sample_rel_err_gpu_vs_oracle_max": max(errs),
            "sample_rel_err_model_floor": rounding_floor(name, distinct)}


def rounding_floor(name, n):
    """The CPU rounding model's error for the first n slices (any NS whose
    iterate is stored in bf16 lands near it), from tests/golden."""
    path = os.path.join(ROOT, "tests", "golden", "rounding_floor.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        ent = json.load(f)["workloads"].get(name, {})
    vals = [v["diag"] for k, v in ent.items() if int(k) < n]
    return max(vals) if vals else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="lowrank64_4096x4096", choices=list(WORKLOADS))
    ap.add_argument("--also", nargs="*", default=["experts128_1536x2048"])
    ap.add_argument("--kernel-timing", choices=["dominant", "all", "none"], default="dominant")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time, at least (0: skip)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 64 MiB device copy three times (the reference that scales "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE into bytes) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(stacks shard by whole slices across GPUs; see the design notes).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)

    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel(), "reads": src.numel(), "writes": src.numel()}))
        return

    mask = {"dominant": 1 << ns.NS_KIND_UPDATE, "all": 0x1F, "none": 0}[args.kernel_timing]
    main_run = time_workload(args.workload, args.steps, args.warmup, mask)
    extra = [time_workload(n, args.steps, args.warmup, mask) for n in args.also if n != args.workload]

    w = WORKLOADS[args.workload]
    algo = algorithmic_flops(w.batch, w.rows, w.cols)
    roof = None
    upd = main_run["kernels"].get("update")
    if upd:
        achieved = algo["update"] / (upd["mean_ms"] * 1e-3) / 1e12
        tr = measured_traffic(args.workload, "update")
        roof = {"bound": "mfma", "kernel": "gemm_kernel update (X' = C X)", "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": tr["bytes"] if tr else None, "traffic_detail": tr,
                "mean_launch_ms": upd["mean_ms"], "algorithmic_flops_per_launch": algo["update"],
                "kernel_source_hash": kernel_source_hash()}

    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(args.workload, main_run["y"], args.cpu_budget)

    flops = dense_eq_flops(w.batch, w.rows, w.cols)
    pages_ms = PAGES_H200_MS.get(args.workload)
    vs = (main_run["eff_tflops"] / (flops / (pages_ms * 1e-3) / 1e12)) if pages_ms else None

    def summary(r):
        return {k: r[k] for k in ("name", "shape", "ms_per_call", "eff_tflops", "pct_dense_bf16_peak", "kernels")}

    line = {
        "metric": "NS ms/call + effective bf16 TFLOP/s (% MFMA peak) at 4096^2 and 128x1536x2048",
        "value": main_run["eff_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_run["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": vs,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "shape": list(w.shape), "ns_steps": STEPS_NS,
                   "coeffs": list(ns.DEFAULT_COEFFS), "pct_dense_bf16_peak": main_run["pct_dense_bf16_peak"],
                   "kernel_config": main_run["config"]},
        "workloads": [summary(main_run)] + [summary(r) for r in extra],
        "baseline_context": {"hardware": "1x H200", "ms_per_call": pages_ms,
                             "source": "prime-rl PR #3873, NS microbenchmark table (QuACK symmetric GEMM)"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
