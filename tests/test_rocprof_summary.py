"""CPU checks of the rocprofv3 summary tool that fills bench.py's roofline traffic."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from learned_token_pruning_post_amd import rocprof_summary as R  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _pmc(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "p_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            # two counter instances per dispatch (summed by the tool)
            for part in (0.25, 0.75):
                w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": name,
                            "Counter_Name": counter, "Counter_Value": value * part})


def test_traffic_scales_by_the_calibration_copy(tmp_path):
    copy = 1 << 20  # bytes
    # the counter reads half of the true bytes for fetches, all of them for writes
    fetch = [("__amd_rocclr_copyBuffer", 4.0), ("__amd_rocclr_copyBuffer", copy / 1024 * 0.5),
             ("void k<2>(P)", 300.0), ("void k<2>(P)", 500.0), ("other", 9.0)]
    write = [("__amd_rocclr_copyBuffer", 8.0), ("__amd_rocclr_copyBuffer", copy / 1024 * 1.0),
             ("void k<2>(P)", 100.0), ("void k<2>(P)", 100.0)]
    _pmc(str(tmp_path / "f"), "FETCH_SIZE", fetch)
    _pmc(str(tmp_path / "w"), "WRITE_SIZE", write)
    res = R.traffic(str(tmp_path / "f"), str(tmp_path / "w"), "k<2>", copy, "gated_attn")
    assert res["fetch_factor"] == pytest.approx(0.5)
    assert res["write_factor"] == pytest.approx(1.0)
    assert res["fetch_kib_per_dispatch"] == pytest.approx(400.0)
    assert res["fetch_bytes"] == round(400.0 * 1024 / 0.5)
    assert res["write_bytes"] == round(100.0 * 1024)
    assert res["traffic_bytes"] == res["fetch_bytes"] + res["write_bytes"]
    assert res["source_sha256"] == R.source_hash("gated_attn")
    assert R.source_hash("gated_attn") != R.source_hash("gate_up_swiglu") != R.source_hash()


def test_traffic_of_a_stage_sums_its_kernels(tmp_path):
    copy = 1 << 20
    fetch = [("__amd_rocclr_copyBuffer", copy / 1024 * 0.5), ("chunk_k<4>", 10.0), ("chunk_k<4>", 30.0),
             ("emit_k<4, true>", 100.0), ("emit_k<4, true>", 100.0)]
    write = [("__amd_rocclr_copyBuffer", copy / 1024 * 1.0), ("chunk_k<4>", 5.0), ("chunk_k<4>", 5.0),
             ("emit_k<4, true>", 50.0), ("emit_k<4, true>", 70.0)]
    _pmc(str(tmp_path / "f"), "FETCH_SIZE", fetch)
    _pmc(str(tmp_path / "w"), "WRITE_SIZE", write)
    res = R.traffic(str(tmp_path / "f"), str(tmp_path / "w"), ["chunk_k", "emit_k"], copy, "select_compact")
    assert res["fetch_kib_per_dispatch"] == pytest.approx(20.0 + 100.0)
    assert res["write_kib_per_dispatch"] == pytest.approx(5.0 + 60.0)
    assert res["fetch_bytes"] == round(120.0 * 1024 / 0.5) and res["write_bytes"] == round(65.0 * 1024)
    assert res["dispatches"] == [[2, 2], [2, 2]] and res["kernel_match"] == "chunk_k+emit_k"


def test_stats_table_orders_by_total(tmp_path):
    p = tmp_path / "run_kernel_stats.csv"
    with open(p, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow(["small", 10, 1000, 100, 1, 90, 110, 1])
        w.writerow(["big", 2, 9000, 4500, 9, 4000, 5000, 1])
    lines = R.stats_table(str(p)).splitlines()
    assert "`big`" in lines[2] and "`small`" in lines[3]
    assert "4.50" in lines[2]


def test_bench_reports_traffic_only_for_unchanged_sources(tmp_path, monkeypatch):
    import bench
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    rec = {"traffic_bytes": 123, "source_sha256": R.source_hash("gate_up_swiglu")}
    with open(tmp_path / "profiles" / "traffic_gate_up_swiglu_w.json", "w") as fh:
        json.dump(rec, fh)
    assert bench.measured_traffic("gate_up_swiglu", "w") == 123
    assert bench.measured_traffic("gated_attn", "w") is None
    # a record taken for one kernel does not stand for another
    with open(tmp_path / "profiles" / "traffic_gated_attn_w.json", "w") as fh:
        json.dump(rec, fh)
    assert bench.measured_traffic("gated_attn", "w") is None
    rec["source_sha256"] = "0" * 64
    with open(tmp_path / "profiles" / "traffic_gate_up_swiglu_w.json", "w") as fh:
        json.dump(rec, fh)
    assert bench.measured_traffic("gate_up_swiglu", "w") is None


def test_mfma_table_joins_counters_and_trace(tmp_path):
    """MOPS x 512 flops per dispatch, busy cycles over GUI_ACTIVE x 1024 SIMDs,
    GUI_ACTIVE per XCD (its per-dispatch sum over the agent's two XCDs here)
    over the traced duration."""
    d = tmp_path / "m"
    os.makedirs(d)
    with open(d / "p_agent_info.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Agent_Type", "Num_Xcc"])
        w.writeheader()
        w.writerow({"Agent_Type": "CPU", "Num_Xcc": 1})
        w.writerow({"Agent_Type": "GPU", "Num_Xcc": 2})
    with open(d / "p_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for disp, name in ((1, "void attn<2, 128>(P)"), (2, "void attn<2, 128>(P)"), (3, "other")):
            for counter, parts in (("SQ_INSTS_VALU_MFMA_MOPS_BF16", (1e6, 1e6)),
                                   ("SQ_VALU_MFMA_BUSY_CYCLES", (102400.0, 102400.0)),
                                   ("GRBM_GUI_ACTIVE", (2000.0, 2000.0))):
                for v in parts:
                    w.writerow({"Correlation_Id": disp, "Dispatch_Id": disp, "Kernel_Name": name,
                                "Counter_Name": counter, "Counter_Value": v})
    with open(d / "p_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for disp in (1, 2, 3):
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": "k", "Start_Timestamp": 1000, "End_Timestamp": 2000})
    (r,) = R.mfma_table(str(d), ["attn<2, 128>"])
    assert r["dispatches"] == 2
    assert r["mfma_gflop_per_dispatch"] == pytest.approx(2e6 * 512 / 1e9)
    assert r["tflops"] == pytest.approx(2e6 * 512 / 1000 / 1e3)
    assert r["mfma_busy_pct"] == pytest.approx(100 * 204800 / (2000 * 1024))
    assert r["clock_ghz"] == pytest.approx(2.0)
