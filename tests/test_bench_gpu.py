"""bench.py end to end on a small workload: one JSON line with the fields the
benchmark contract names, per-kernel durations that add up to the
instrumented step, and a HIP-graph replay of the same step."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.gpu


def test_bench_json_line_small_workload():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "qwen8k", "--steps", "3",
           "--warmup", "1", "--no-cpu-baseline"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.strip().splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "kernels"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["dtype"] == "bf16"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    rf = d["roofline"]
    assert rf["bound"] in ("mfma", "hbm", "alu") and 0 < rf["frac"] < 1
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    # per-kernel durations come from the instrumented pass and must add up to it
    kern = d["kernels"]
    total = sum(k["ms_per_step"] for k in kern.values())
    assert all(k["avg_us"] > 0 for k in kern.values())
    assert abs(total - d["ms_per_step_with_kernel_events"]) < 0.1 * d["ms_per_step_with_kernel_events"]
    # the graph replay of the same step takes about as long as the eager step
    g = d["ms_per_step_hip_graph"]
    assert g is not None and 0.5 * d["ms_per_step"] < g < 1.5 * d["ms_per_step"]
