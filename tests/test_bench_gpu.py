"""bench.py end to end on a small workload: one JSON line with the fields the
benchmark contract names, per-kernel durations that with the host-side hops
between calls add up to the instrumented step, and a HIP-graph replay of the
same step."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.gpu


def test_bench_json_line_small_workload():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "qwen8k", "--steps", "3",
           "--warmup", "1"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=170)
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
    # the per-kernel entries and the host-side hops between calls tile each
    # instrumented step exactly (first event to last event); the hops are GPU idle
    # time that depends on the host, so they are reported apart and not bounded here
    kern = d["kernels"]
    total = sum(k["ms_per_step"] for k in kern.values())
    assert all(k["avg_us"] > 0 for k in kern.values())
    gaps = d["host_gaps"]
    span = d["ms_per_step_with_kernel_events"]
    assert gaps["in_step_ms_per_step"] >= -1e-3 and gaps["between_steps_ms_per_step"] >= -1e-3
    assert abs(total + gaps["in_step_ms_per_step"] - span) < 0.01 * span + 1e-3
    # the oracle leg: CPU baseline and parity of this very workload
    cb, par = d["cpu_baseline"], d["parity"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert par["selection_bit_exact"] and par["compaction_bit_exact"]
    assert par["scores_within_tol"] and par["layer0_out_within_tol"]
    assert 0 <= par["selection_flips_vs_fp64_scores"] <= 1024
    # peak memory against the unpruned path (K = N) at the same N
    mem = d["memory"]
    assert mem["peak_gb_one_layer_unpruned"] > mem["peak_gb_one_layer_pruned"] > 0
    assert mem["kv_cache_gb_27_layers_unpruned"] == pytest.approx(8 * mem["kv_cache_gb_27_layers_pruned"], rel=1e-2)
    # the whole-model prefill against the same model run unpruned
    pf = d["prefill_vs_unpruned"]
    assert pf["layers"] == 28 and pf["gate_layer"] == 1 and pf["n_kept_tokens"] == 1024
    assert pf["pruned_ms"] > 0 and pf["speedup"] > 1 and pf["peak_gb_unpruned"] > pf["peak_gb_pruned"] > 0
    # decode attention over the pruned cache against the full one
    dec = d["decode_vs_unpruned"]
    assert dec["kept_prompt_keys"] == 1024 and dec["prompt_keys_unpruned"] == 8192
    assert dec["pruned_us"] > 0 and dec["speedup"] > 1 and 0 < dec["pruned_frac_hbm"] < 1
    # the gate's gradient path timed at the workload's shapes
    bw = d["backward"]
    assert bw["attn_bwd_us"] > 0 and bw["scorer_bwd_us"] > 0 and 0 < bw["attn_bwd_frac_mfma_peak"] < 1
    assert d["gdn_kept_tokens"]["us"] > 0 and d["gdn_kept_tokens"]["tokens"] == 1024
    # the graph replay of the same step takes about as long as the eager step
    g = d["ms_per_step_hip_graph"]
    assert g is not None and 0.5 * d["ms_per_step"] < g < 1.5 * d["ms_per_step"]
