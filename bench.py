"""Benchmark of the batched Newton–Schulz orthogonalization on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--also NAME ...]
    python bench.py --all-configs OUT_PREFIX      (every workload; writes OUT_PREFIX.md/.json)

One step = one ns_orthogonalize call (normalisation + 5 quintic steps) over
the whole workload, inputs already resident in HBM.  Prints ONE JSON line.

value       effective bf16 TFLOP/s of the primary workload: dense-equivalent
            FLOPs 5 (4 m² n + 2 m³) per slice divided by the measured time
            (the comparison basis of the prime-rl NS microbenchmark table)
norm_pass   the sum-of-squares pass (HBM-bound): bytes read per launch over
            its mean HIP-event launch time, against 8 TB/s
roofline    the dominant kernel (the update product) timed with HIP events
            in its dispatch packets on the launch stream, in the timed
            region (the third of the five update launches of every timed
            call), algorithmic FLOPs per launch / mean launch time, against
            the 2.5 PFLOP/s dense bf16 MFMA peak and the measured peak
cpu_baseline the fp64 CPU oracle on a bounded sample of the same workload
dense       the same method with dense PyTorch-ROCm bf16 matmuls (hipBLASLt),
            timed on the same inputs: the comparator column of the pages'
            dense-vs-symmetric table (bench only, not a library path)
measured_peak  the bf16 MFMA rate of a register-only loop on this GPU and the
            shader clock it ran at (ns_peak_mfma), with a plain 4096^3
            torch.matmul (hipBLASLt) beside it as a library GEMM reference
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
from ns_inputs import WORKLOADS, gaussian, make_workload  # noqa: E402

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


def call_times(fn, steps):
    """Per-call durations (ms) from HIP events around each call."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def spread(ts):
    q = np.percentile(np.asarray(ts), [10, 50, 90])
    return {"p10_ms": float(q[0]), "median_ms": float(q[1]), "p90_ms": float(q[2])}


def dense_ns(x, steps=STEPS_NS, coeffs=None, eps=1e-7):
    """The same method with dense bf16 matmuls in PyTorch-ROCm (hipBLASLt), as
    in the dense routine the pages compare against: per slice X / (||X||_F +
    eps), transposed if tall, then steps x (A = X Xᵀ, B = b A + c A A,
    X = a X + B X).  A comparator only; the library never runs it."""
    a, b, c = coeffs or ns.DEFAULT_COEFFS
    X = x.reshape(-1, x.shape[-2], x.shape[-1])
    tall = X.shape[-2] > X.shape[-1]
    if tall:
        X = X.transpose(-2, -1).contiguous()
    nrm = torch.linalg.vector_norm(X, dim=(-2, -1), keepdim=True, dtype=torch.float32)
    X = (X.float() / (nrm + eps)).to(x.dtype)
    for _ in range(steps):
        A = torch.matmul(X, X.transpose(-2, -1).contiguous())  # transposed operand made contiguous
        B = b * A + c * torch.matmul(A, A)
        X = a * X + torch.matmul(B, X)
    if tall:
        X = X.transpose(-2, -1).contiguous()
    return X.reshape(x.shape)


def time_dense(xg, steps, warmup):
    for _ in range(warmup):
        y = dense_ns(xg)
    torch.cuda.synchronize()
    ts = call_times(lambda: dense_ns(xg), steps)
    y = dense_ns(xg)
    torch.cuda.synchronize()
    return {"ms_per_call": float(np.mean(ts)), **spread(ts)}, y


def measured_peak(reps=20):
    """Measured bf16 matrix peaks on this GPU: the library's register-only
    MFMA loop (ns_peak_mfma: the rate and shader clock the matrix cores hold
    under full load), and a plain 4096^3 torch.matmul (hipBLASLt) as a
    library GEMM reference."""
    n = 4096
    g = torch.Generator(device="cuda:0").manual_seed(0)
    a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    ts = call_times(lambda: torch.matmul(a, b), reps)
    gemm = 2 * n ** 3 / (float(np.median(ts)) * 1e-3) / 1e12
    ns.ns_peak_mfma("bf16", 1 << 16)  # warm-up
    runs = [ns.ns_peak_mfma("bf16", 1 << 20) for _ in range(3)]
    tf, mhz = max(runs)
    return {"what": "register-only v_mfma_f32_32x32x16_bf16 loop, 2 workgroups of 4 waves per CU (ns_peak_mfma), "
                    "best of 3 runs of ~0.1 s",
            "tflops": tf, "shader_clock_mhz": mhz,
            "gemm_reference": {"what": "torch.matmul bf16 4096x4096x4096 (hipBLASLt)", "tflops": gemm}}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def resident_input(name):
    """The workload's seeded input, on the host and resident in HBM."""
    x = make_workload(name)
    if x.dtype != torch.bfloat16:
        x = x.to(torch.bfloat16)
    return x, x.to(torch.device("cuda:0"))


def time_workload(name, steps, warmup, kernel_mask, inputs=None):
    w = WORKLOADS[name]
    x, xg = inputs if inputs is not None else resident_input(name)
    out = torch.empty_like(xg)
    for _ in range(warmup):
        ns.orthogonalize(xg, out=out)
    torch.cuda.synchronize()
    ns.ns_timing_reset()
    # one timed launch per kernel kind and call (the third of the call's five
    # launches of a step kernel): each timed dispatch releases its events at
    # its end, which delays the next kernel by a few microseconds
    ns.ns_timing_sample(STEPS_NS, STEPS_NS // 2)
    ns.ns_timing_enable(kernel_mask)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        ns.orthogonalize(xg, out=out)
    stop.record()
    torch.cuda.synchronize()
    ns.ns_timing_enable(0)
    ns.ns_timing_sample(1, 0)
    ms = start.elapsed_time(stop) / steps
    per_call = spread(call_times(lambda: ns.orthogonalize(xg, out=out), steps))
    kernels = {}
    for kind, kname in ns.KIND_NAMES.items():
        tot, n = ns.ns_timing_query(kind)
        if n:
            kernels[kname] = {"mean_ms": tot / n, "launches": n}
    ns.ns_timing_reset()
    flops = dense_eq_flops(w.batch, w.rows, w.cols)
    eff = flops / (ms * 1e-3) / 1e12
    return {"name": name, "shape": list(w.shape), "ms_per_call": ms, **per_call, "eff_tflops": eff,
            "pct_dense_bf16_peak": 100.0 * eff / PEAK_BF16_TFLOPS, "kernels": kernels,
            "config": ns.ns_query_last_config(), "x": x, "xg": xg, "y": out}


def sustained(r, seconds):
    """Back-to-back calls on the workload for about `seconds`, after (and
    outside) the timed region: the rate once the shader clock has settled
    under a long load, and GPU activity long enough for an outside utilisation
    sampler to see.  Calls go out in chunks of about 0.2 s, with a host
    synchronisation between chunks."""
    xg, out = r["xg"], r["y"]
    chunk = max(1, int(0.2 / (r["ms_per_call"] * 1e-3)))
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    while True:
        for _ in range(chunk):
            ns.orthogonalize(xg, out=out)
        n += chunk
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / n
    eff = r["eff_tflops"] * r["ms_per_call"] / ms
    return {"name": r["name"], "seconds": time.perf_counter() - t0, "calls": n, "ms_per_call": ms,
            "eff_tflops": eff, "pct_dense_bf16_peak": 100.0 * eff / PEAK_BF16_TFLOPS}


def cpu_baseline(name, y_gpu, budget_s, y_dense=None):
    """The fp64 oracle on whole slices of the workload, cycling through them,
    until ~budget_s seconds; each distinct slice is also compared with the GPU
    output."""
    from oracle import newton_schulz_batched  # CPU baseline leg only

    w = WORKLOADS[name]
    x = make_workload(name)
    if name == "iid_256x512":
        x = x.to(torch.bfloat16)
    xs = x.reshape(-1, w.rows, w.cols)
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max(int(i.get("num_threads", 1)) for i in threadpool_info()) if threadpool_info() else None
    except Exception:  # noqa: BLE001
        blas_threads = None
    ys = y_gpu.reshape(-1, w.rows, w.cols)
    yd = y_dense.reshape(-1, w.rows, w.cols) if y_dense is not None else None
    t0 = time.perf_counter()
    done = 0
    errs, derrs = [], []
    while True:
        i = done % xs.shape[0]
        ref = newton_schulz_batched(xs[i:i + 1].double().numpy())[0]
        if done < xs.shape[0]:
            got = ys[i].double().cpu().numpy()
            errs.append(float(np.linalg.norm(got - ref) / np.linalg.norm(ref)))
            if yd is not None:
                derrs.append(float(np.linalg.norm(yd[i].double().cpu().numpy() - ref) / np.linalg.norm(ref)))
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
            "sample_rel_err_model_floor": rounding_floor(name, distinct),
            "sample_rel_err_dense_vs_oracle_max": max(derrs) if derrs else None, "cpu_model": cpu_model(),
            "blas_threads": blas_threads}


# the pages' H200 microbenchmark (ms per call, dense bf16 / QuACK symmetric)
PAGES_H200_TABLE = {"lowrank64_4096x4096": (3.21, 2.71), "square_8192x8192": (25.5, 17.0),
                    "mlp_4096x14336": (8.74, 7.07), "experts128_1536x2048": (35.9, 25.0),
                    "experts128_2048x768": (12.9, 8.6), "experts32_7168x2048": (49.5, 33.0)}
SAMPLES = {"experts16_1536x2048": [0, 7, 15], "experts128_1536x2048": [0, 63, 127],
           "experts32_7168x2048": [0, 31], "experts128_2048x768": [0, 64, 127]}


def all_configs(prefix, steps, warmup):
    """Every workload: ms/call (and spread) of this library and of the dense
    comparator, effective TFLOP/s against the spec and the measured peak, and
    both outputs' relative error vs the fp64 oracle on sampled slices beside
    the rounding-model floor.  Writes prefix.json and prefix.md."""
    from oracle import newton_schulz  # the error columns only

    peak = measured_peak()
    print(json.dumps({"measured_peak": peak}), flush=True)
    rows = []
    oracle_cache = {}
    runs = [(n, torch.bfloat16) for n in WORKLOADS] + [("iid_256x512", torch.float32)]
    for name, dtype in runs:
        w = WORKLOADS[name]
        x0 = make_workload(name)  # the oracle reads this tensor (the fp32 original for a bf16 run of it)
        x = x0.to(dtype)
        xg = x.to("cuda:0")
        out = torch.empty_like(xg)
        for _ in range(warmup):
            ns.orthogonalize(xg, out=out)
        torch.cuda.synchronize()
        ts = call_times(lambda: ns.orthogonalize(xg, out=out), steps)
        d, yd = time_dense(xg, max(3, steps // 2), 2)
        flops = dense_eq_flops(w.batch, w.rows, w.cols)
        ms = float(np.mean(ts))
        eff = flops / (ms * 1e-3) / 1e12
        xs, ys, yds = (t.reshape(-1, w.rows, w.cols) for t in (x0, out, yd))
        errs, derrs, osec = [], [], []
        for i in SAMPLES.get(name, [0]):
            # the transposed MLP weight reuses its transpose's oracle: NS(Xᵀ) = NS(X)ᵀ
            key = (name.replace("mlp_14336x4096", "mlp_4096x14336"), i)
            t0 = time.perf_counter()
            if key[0] != name and key in oracle_cache:
                ref = oracle_cache[key].T
            else:
                if (name, i) not in oracle_cache:
                    oracle_cache[(name, i)] = newton_schulz(xs[i].double().numpy())
                ref = oracle_cache[(name, i)]
            osec.append(time.perf_counter() - t0)
            for y, e in ((ys, errs), (yds, derrs)):
                g = y[i].double().cpu().numpy()
                e.append(float(np.linalg.norm(g - ref) / np.linalg.norm(ref)))
        peak_spec = PEAK_BF16_TFLOPS if dtype == torch.bfloat16 else PEAK_F32_TFLOPS
        row = {"workload": name, "shape": list(w.shape), "dtype": "bf16" if dtype == torch.bfloat16 else "fp32",
               "ms_per_call": ms, **spread(ts), "eff_tflops": eff, "pct_spec_peak": 100 * eff / peak_spec,
               "pct_measured_peak": 100 * eff / peak["tflops"] if dtype == torch.bfloat16 else None,
               "dense_ms_per_call": d["ms_per_call"], "speedup_vs_dense": d["ms_per_call"] / ms,
               "err_max": max(errs), "err_mean": float(np.mean(errs)), "dense_err_max": max(derrs),
               "model_floor": rounding_floor(name, 10 ** 9) if dtype == torch.bfloat16 else None,
               "sampled_slices": SAMPLES.get(name, [0]), "oracle_s_per_slice": float(np.mean(osec)),
               "pages_h200_dense_quack_ms": PAGES_H200_TABLE.get(name)}
        rows.append(row)
        print(json.dumps(row), flush=True)
        del xg, out, yd
        torch.cuda.empty_cache()
    grows = grouped_rows(steps, warmup)
    orows = odd_shape_rows(steps, warmup)
    host = {"cpu_model": cpu_model(), "cores": len(os.sched_getaffinity(0))}
    with open(prefix + ".json", "w") as f:
        json.dump({"measured_peak": peak, "host": host, "rows": rows, "grouped": grows, "odd_shapes": orows}, f,
                  indent=1)
    lines = ["# ns_orthogonalize on every workload: time, accuracy, the dense comparator, grouped calls, odd sides",
             "", "Command (MI355X, one GPU; `$REPO` is the repository root):", "", "```",
             f"python $REPO/bench.py --all-configs {prefix} --warmup {warmup} --steps {steps}",
             "```", "",
             f"This box: register-only MFMA loop {peak['tflops']:.0f} TFLOP/s at a {peak['shader_clock_mhz']:.0f} MHz "
             f"shader clock; {host['cores']} host cores ({host['cpu_model']}).  Kernel source hash "
             f"`{kernel_source_hash()}`.  Per workload: {warmup} warmup calls, then {steps} calls timed one by one; "
             "errors are relative Frobenius errors against the fp64 oracle on the sampled slices.", "",
             "| workload | dtype | ms/call (p10-p90) | eff. TFLOP/s | % spec peak | % measured peak | dense ms | "
             "speedup vs dense | err max / mean | dense err | model floor | oracle s/slice | H200 dense / QuACK ms |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        pm = f"{r['pct_measured_peak']:.1f}%" if r["pct_measured_peak"] is not None else "-"
        fl = f"{r['model_floor']:.2e}" if r["model_floor"] is not None else "-"
        h2 = "{} / {}".format(*r["pages_h200_dense_quack_ms"]) if r["pages_h200_dense_quack_ms"] else "-"
        lines.append(f"| {r['workload']} | {r['dtype']} | {r['ms_per_call']:.3f} ({r['p10_ms']:.3f}-{r['p90_ms']:.3f}) | "
                     f"{r['eff_tflops']:.0f} | {r['pct_spec_peak']:.1f}% | {pm} | {r['dense_ms_per_call']:.3f} | "
                     f"{r['speedup_vs_dense']:.2f}x | {r['err_max']:.2e} / {r['err_mean']:.2e} | "
                     f"{r['dense_err_max']:.2e} | {fl} | {r['oracle_s_per_slice']:.1f} | {h2} |")
    lines += ["", "Grouped calls (ns_orthogonalize_grouped) vs one ns_orthogonalize call per stack, same inputs "
              "and stream, median of the timed repetitions of the whole set:", "",
              "| set | stacks | ms, one call per stack | ms, one grouped call | speedup | bitwise equal |",
              "|---|---|---|---|---|---|"]
    for r in grows:
        lines.append(f"| {r['set']} | {r['stacks']} | {r['singles_ms']:.3f} | {r['grouped_ms']:.3f} | "
                     f"{r['speedup']:.2f}x | {'yes' if r['bitwise_equal'] else 'NO'} |")
    lines += ["", "Sides not multiples of 8 (the call runs on a zero-padded copy: the pad pass fused with the sum "
              "of squares, and a vectorised copy of the caller's block out) beside the padded shape, bf16, "
              "median ms per call:", "",
              "| shape | ms | padded neighbour | ms | overhead |", "|---|---|---|---|---|"]
    for r in orows:
        lines.append(f"| {r['odd']} | {r['odd_ms']:.3f} | {r['even']} | {r['even_ms']:.3f} | {r['overhead_pct']:+.1f}% |")
    with open(prefix + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


def grouped_rows(steps, warmup):
    """Each grouped set: the median time of one grouped call over all its
    stacks and of one call per stack, and whether the outputs agree bitwise."""
    from ns_inputs import GROUPED_SETS, make_grouped_set
    rows = []
    for name, shapes in GROUPED_SETS.items():
        xs = [x.to("cuda:0") for x in make_grouped_set(name)]
        ya = [torch.empty_like(x) for x in xs]
        yb = [torch.empty_like(x) for x in xs]

        def singles():
            for x, y in zip(xs, ya):
                ns.orthogonalize(x, out=y)

        def grouped():
            ns.orthogonalize_grouped(xs, outs=yb)

        res = {}
        for label, f in (("singles_ms", singles), ("grouped_ms", grouped)):
            for _ in range(warmup):
                f()
            torch.cuda.synchronize()
            res[label] = float(np.median(call_times(f, max(5, steps // 2))))
        torch.cuda.synchronize()
        row = {"set": name, "stacks": "; ".join("x".join(map(str, s)) for s in shapes), **res,
               "speedup": res["singles_ms"] / res["grouped_ms"],
               "bitwise_equal": all(torch.equal(a, b) for a, b in zip(ya, yb))}
        rows.append(row)
        print(json.dumps(row), flush=True)
        del xs, ya, yb
        torch.cuda.empty_cache()
    return rows


ODD_PAIRS = [((16, 1535, 2047), (16, 1536, 2048)), ((1, 4095, 4095), (1, 4096, 4096)),
             ((64, 2047, 767), (64, 2048, 768))]


def odd_shape_rows(steps, warmup):
    """Shapes whose sides are not multiples of 8 (run on zero-padded copies)
    beside their padded neighbour: the median call time of each and the
    overhead of the padded path."""
    rows = []
    for k, (odd, even) in enumerate(ODD_PAIRS):
        res = {}
        for label, shape in (("odd", odd), ("even", even)):
            x = gaussian(shape, 2000 + 2 * k + (label == "even"), torch.bfloat16).to("cuda:0")
            y = torch.empty_like(x)
            for _ in range(warmup):
                ns.orthogonalize(x, out=y)
            torch.cuda.synchronize()
            res[label + "_ms"] = float(np.median(call_times(lambda: ns.orthogonalize(x, out=y), max(5, steps // 2))))
            del x, y
        row = {"odd": "x".join(map(str, odd)), "even": "x".join(map(str, even)), **res,
               "overhead_pct": 100.0 * (res["odd_ms"] / res["even_ms"] - 1.0)}
        rows.append(row)
        print(json.dumps(row), flush=True)
        torch.cuda.empty_cache()
    return rows


def rounding_floor(name, n):
    """The CPU rounding model's error for the first n slices (any NS whose
    iterate is stored in bf16 lands near it), from tests/golden."""
    path = os.path.join(ROOT, "tests", "golden", "rounding_floor.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        ent = json.load(f)["workloads"].get(name, {})
    vals = [v["shipped"] for k, v in ent.items() if int(k) < n]
    return max(vals) if vals else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed calls per workload first: the shader clock ramps up over the first tens of ms")
    ap.add_argument("--workload", default="lowrank64_4096x4096", choices=list(WORKLOADS))
    ap.add_argument("--also", nargs="*", default=["experts128_1536x2048"])
    ap.add_argument("--kernel-timing", choices=["dominant", "all", "none"], default="dominant")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time, at least (0: skip)")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense PyTorch comparator")
    ap.add_argument("--sustain", type=float, default=8.0,
                    help="seconds of back-to-back calls after the timed region, split over the workloads "
                         "(reported under 'sustained'; 0: skip)")
    ap.add_argument("--all-configs", metavar="OUT_PREFIX",
                    help="time and check every workload (this library's and the dense comparator's error vs "
                         "the oracle on sampled slices), write OUT_PREFIX.md and OUT_PREFIX.json, and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 64 MiB device copy three times (the reference that scales "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE into bytes) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
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

    if args.all_configs:
        all_configs(args.all_configs, args.steps, args.warmup)
        return

    # the dominant kernel and the HBM-bound norm pass
    mask = {"dominant": (1 << ns.NS_KIND_UPDATE) | (1 << ns.NS_KIND_SUMSQ), "all": 0x1F,
            "none": 0}[args.kernel_timing]
    # inputs first (host generation leaves the GPU idle), then the MFMA peak
    # probe: its ~0.3 s of full matrix load also brings the shader clock up
    # from idle before the workloads' warmup
    names = [args.workload] + [n for n in args.also if n != args.workload]
    inputs = {n: resident_input(n) for n in names}
    peak = measured_peak()
    main_run = time_workload(args.workload, args.steps, args.warmup, mask, inputs.pop(args.workload))
    extra = [time_workload(n, args.steps, args.warmup, mask, inputs.pop(n)) for n in names[1:]]
    y_dense = None
    for r in [main_run] + extra:
        r["pct_measured_peak"] = 100.0 * r["eff_tflops"] / peak["tflops"]
        r["pct_hipblaslt_gemm"] = 100.0 * r["eff_tflops"] / peak["gemm_reference"]["tflops"]
        if not args.no_dense:
            d, yd = time_dense(r["xg"], max(3, args.steps // 2), 2)
            r["dense"] = {**d, "eff_tflops": r["eff_tflops"] * r["ms_per_call"] / d["ms_per_call"],
                          "speedup_of_this_build": d["ms_per_call"] / r["ms_per_call"]}
            if r is main_run:
                y_dense = yd
            del yd

    runs = [main_run] + extra
    sus = [sustained(r, args.sustain / len(runs)) for r in runs] if args.sustain > 0 else None

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
                "measured_peak": peak["tflops"], "frac_of_measured_peak": achieved / peak["tflops"],
                "mean_launch_ms": upd["mean_ms"], "timed_launches": upd["launches"],
                "timed_launch_sample": "the third update of each timed call (HIP events in the dispatch packet)",
                "algorithmic_flops_per_launch": algo["update"],
                "kernel_source_hash": kernel_source_hash()}

    # the norm pass (sum of squares) reads the input once: HBM-bound
    norm = None
    ss = main_run["kernels"].get("sumsq")
    if ss:
        nbytes = w.batch * w.rows * w.cols * 2
        norm = {"kernel": "sumsq_kernel (per-slice sum of squares)", "bytes_per_launch": nbytes,
                "mean_launch_ms": ss["mean_ms"], "timed_launches": ss["launches"],
                "achieved_GBps": nbytes / (ss["mean_ms"] * 1e-3) / 1e9, "peak_GBps": PEAK_HBM_GBS,
                "frac": nbytes / (ss["mean_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS}

    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(args.workload, main_run["y"], args.cpu_budget, y_dense)

    pages_ms = PAGES_H200_MS.get(args.workload)

    def summary(r):
        keys = ("name", "shape", "ms_per_call", "p10_ms", "median_ms", "p90_ms", "eff_tflops", "pct_dense_bf16_peak",
                "pct_measured_peak", "pct_hipblaslt_gemm", "dense", "kernels")
        return {k: r[k] for k in keys if k in r}

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
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "shape": list(w.shape), "ns_steps": STEPS_NS,
                   "coeffs": list(ns.DEFAULT_COEFFS), "pct_dense_bf16_peak": main_run["pct_dense_bf16_peak"],
                   "kernel_config": main_run["config"]},
        "measured_peak": peak,
        "workloads": [summary(main_run)] + [summary(r) for r in extra],
        "sustained": sus,
        "baseline_context": {"hardware": "1x H200", "ms_per_call": pages_ms,
                             "ratio_of_this_rate": (pages_ms / main_run["ms_per_call"]) if pages_ms else None,
                             "note": "another machine's figure: context only, not the baseline",
                             "source": "prime-rl PR #3873, NS microbenchmark table (QuACK symmetric GEMM)"},
        "roofline": roof,
        "norm_pass": norm,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
