"""The benchmark's command line and its one-line JSON result.

CPU: more than one GPU is refused with a message, before any device is
touched.  GPU: a short run prints one JSON line with the fields the
measurement needs: the metric and unit, the per-step time and the value it
implies, the roofline of the dominant kernel (algorithmic FLOPs over its
timed launches, against the spec and the measured peak), the norm pass's
HBM rate, and the measured peak itself."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=600):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2", timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.gpu
def test_short_run_prints_one_complete_line():
    r = run_bench("--steps", "5", "--warmup", "2", "--also", "--cpu-budget", "0", "--no-dense", "--sustain", "1")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "dtype", "data", "config", "roofline", "measured_peak", "norm_pass", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2 and d["dtype"] == "bf16"
    assert d["config"]["workload"] == "lowrank64_4096x4096"
    m, n = 4096, 4096
    dense_eq = 5 * (4 * m * m * n + 2 * m ** 3)
    assert d["value"] == pytest.approx(dense_eq / (d["ms_per_step"] * 1e-3) / 1e12, rel=1e-6)
    roof = d["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert roof["timed_launches"] == 5  # the third update of each of the 5 timed calls
    assert roof["achieved"] == pytest.approx(2 * m * m * n / (roof["mean_launch_ms"] * 1e-3) / 1e12, rel=1e-6)
    assert 0.0 < roof["frac"] < 1.0 and roof["frac"] == pytest.approx(roof["achieved"] / 2500.0)
    assert 0.0 < roof["frac_of_measured_peak"] < 1.0
    assert d["measured_peak"]["tflops"] > 0 and d["measured_peak"]["shader_clock_mhz"] > 0
    assert d["norm_pass"] is not None and 0.0 < d["norm_pass"]["frac"] < 1.0
    assert d["cpu_baseline"] is None  # --cpu-budget 0
    assert d["vs_baseline"] is None  # the pages' H200 figure is context only
    sus = d["sustained"]  # back-to-back calls after the timed region, outside it
    assert [s["name"] for s in sus] == ["lowrank64_4096x4096"]
    assert sus[0]["seconds"] >= 1.0 and sus[0]["calls"] > 0 and sus[0]["ms_per_call"] > 0
    assert sus[0]["eff_tflops"] == pytest.approx(dense_eq / (sus[0]["ms_per_call"] * 1e-3) / 1e12, rel=1e-6)
