"""Turn rocprofv3 output into the short text summaries kept under profiles/.

    python -m learned_token_pruning_post_amd.rocprof_summary stats STATS_CSV --cmd "..." > out.md
        kernel table (calls, average / total duration) from a --kernel-trace --stats run

    python -m learned_token_pruning_post_amd.rocprof_summary traffic \\
        --fetch FETCH_CSV --write WRITE_CSV --kernel SUBSTR --copy-bytes N --cmd "..." --out PREFIX
        HBM traffic of one kernel from two --pmc runs (FETCH_SIZE, then WRITE_SIZE), each
        scaled by what the same counter reads for the plain device copy of N bytes that
        `bench.py --calib-copy` issues in the same process; writes PREFIX.json (read by
        bench.py) and PREFIX.md

    python -m learned_token_pruning_post_amd.rocprof_summary mfma PMC_DIR --kernel SUBSTR ... --cmd "..."
        matrix-core use per kernel from one --pmc run (with --kernel-trace) of
        SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE (the
        latter summed over the XCDs in rocprofv3's per-dispatch row, so divided by
        their count from agent_info.csv): bf16
        MFMA flops per dispatch (MOPS x 512), flop rate against the 2.5 PFLOP/s dense bf16
        peak, busy fraction of the matrix cores over the kernel's active cycles (busy
        cycles / (GUI_ACTIVE x 1024 SIMDs), rocprofv3's MfmaUtil), and the clock it ran at
        (GUI_ACTIVE / duration)

The JSON carries a hash of the measured kernel's sources (its own .hip file and the shared
device headers); bench.py reports the traffic only while those still hash the same, i.e.
while the counters describe the kernel being timed.
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
COPY_KERNEL = "copyBuffer"  # the HIP runtime's device-to-device copy kernel


# the files that define each stage's kernel: its own source plus the shared device
# helpers (tg_internal.hpp only declares host launchers, so it is not part of a kernel)
_SHARED = ["tg_common.hpp"]
STAGE_SOURCES = {
    "gate_score": ["tg_gemm.hip"] + _SHARED,
    "select_compact": ["tg_select.hip"] + _SHARED,
    "topk_select": ["tg_select.hip"] + _SHARED,
    "compact": ["tg_rowops.hip"] + _SHARED,
    "decode_attn": ["tg_decode.hip"] + _SHARED,
    "rmsnorm_attn": ["tg_rowops.hip"] + _SHARED,
    "rmsnorm_ffn": ["tg_rowops.hip"] + _SHARED,
    "rope_table": ["tg_rowops.hip"] + _SHARED,
    "qkv_rope_kv": ["tg_gemm.hip"] + _SHARED,
    "gated_attn": ["tg_attn.hip"] + _SHARED,
    "o_proj_resid": ["tg_gemm.hip"] + _SHARED,
    "gate_up_swiglu": ["tg_gemm.hip"] + _SHARED,
    "down_proj_resid": ["tg_gemm.hip"] + _SHARED,
}


def source_hash(stage=None) -> str:
    """sha256 over the sources of `stage`'s kernel (every kernel source and the C header
    when `stage` is None or unknown), in a fixed order."""
    if stage in STAGE_SOURCES:
        files = [os.path.join(PKG, "csrc", f) for f in STAGE_SOURCES[stage]]
    else:
        files = sorted(glob.glob(os.path.join(PKG, "csrc", "*"))) + [os.path.join(ROOT, "include", "tokengate.h")]
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _rows(path):
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _find_csv(path, suffix):
    if os.path.isdir(path):
        hits = glob.glob(os.path.join(path, "**", "*" + suffix), recursive=True)
        if not hits:
            raise SystemExit("no *%s under %s" % (suffix, path))
        return hits[0]
    return path


def stats_table(stats_csv: str, top: int = 20) -> str:
    rows = _rows(_find_csv(stats_csv, "kernel_stats.csv"))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    out = ["| kernel | calls | avg us | total us | % |", "|---|---:|---:|---:|---:|"]
    for r in rows[:top]:
        name = r["Name"].replace("|", "\\|")
        if len(name) > 90:
            name = name[:87] + "..."
        out.append("| `%s` | %s | %.2f | %.1f | %.1f |" % (
            name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e3,
            100.0 * float(r["TotalDurationNs"]) / tot))
    return "\n".join(out)


def _per_dispatch(pmc_csv, counter, match, largest=False):
    """Average over dispatches of kernels whose name contains `match` (KiB per dispatch);
    with `largest`, the largest single dispatch instead (the calibration copy among the
    runtime's smaller copies)."""
    per = collections.defaultdict(float)
    names = {}
    for r in _rows(_find_csv(pmc_csv, "counter_collection.csv")):
        if r["Counter_Name"] != counter or match not in r["Kernel_Name"]:
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id") or str(len(per))
        per[key] += float(r["Counter_Value"])  # summed over XCD/SE instances
        names[key] = r["Kernel_Name"]
    if not per:
        raise SystemExit("no %s rows for kernels matching %r" % (counter, match))
    vals = list(per.values())
    if largest:
        return max(vals), 1, sorted(set(names.values()))[0]
    return sum(vals) / len(vals), len(vals), sorted(set(names.values()))[0]


def traffic(fetch_csv, write_csv, kernel, copy_bytes, stage=None):
    """`kernel`: one name substring, or a list of them for a stage made of
    several kernels (their per-dispatch figures are summed: one pass of the
    stage launches each of them once)."""
    kernels = [kernel] if isinstance(kernel, str) else list(kernel)
    f_kib = w_kib = 0.0
    f_n, w_n, names = [], [], []
    for k in kernels:
        fk, fn, name = _per_dispatch(fetch_csv, "FETCH_SIZE", k)
        wk, wn, _ = _per_dispatch(write_csv, "WRITE_SIZE", k)
        f_kib += fk
        w_kib += wk
        f_n.append(fn)
        w_n.append(wn)
        names.append(name)
    name = " + ".join(names)
    kernel = "+".join(kernels)
    cf_kib, _, _ = _per_dispatch(fetch_csv, "FETCH_SIZE", COPY_KERNEL, largest=True)
    cw_kib, _, _ = _per_dispatch(write_csv, "WRITE_SIZE", COPY_KERNEL, largest=True)
    f_factor = cf_kib * 1024.0 / copy_bytes   # counter KiB per true KiB
    w_factor = cw_kib * 1024.0 / copy_bytes
    fetch_b = f_kib * 1024.0 / f_factor
    write_b = w_kib * 1024.0 / w_factor
    return {
        "kernel_match": kernel, "kernel_name": name,
        "dispatches": [f_n[0], w_n[0]] if len(kernels) == 1 else [f_n, w_n],
        "fetch_kib_per_dispatch": round(f_kib, 1), "write_kib_per_dispatch": round(w_kib, 1),
        "copy_bytes": copy_bytes, "copy_fetch_kib": round(cf_kib, 1), "copy_write_kib": round(cw_kib, 1),
        "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4),
        "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
        "traffic_bytes": round(fetch_b + write_b), "source_sha256": source_hash(stage),
    }


SIMD_NUM = 1024            # 256 CUs x 4 SIMDs
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA


def _by_dispatch(rows, counter):
    """{dispatch: value} of one counter summed over its rows (rocprofv3 writes
    one row per dispatch, already summed over the XCDs); names alongside."""
    vals, names = {}, {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        names[key] = r["Kernel_Name"]
    return vals, names


def _num_xcc(pmc_dir):
    """XCDs of the GPU agent (agent_info.csv), whose GRBM_GUI_ACTIVE cycle counts
    the per-dispatch value sums; 8 on MI355X when the file is absent."""
    try:
        for r in _rows(_find_csv(pmc_dir, "agent_info.csv")):
            if r.get("Agent_Type") == "GPU" and int(r.get("Num_Xcc") or 0) > 0:
                return int(r["Num_Xcc"])
    except SystemExit:
        pass
    return 8


def mfma_table(pmc_dir, kernels):
    """Per kernel-name substring: dispatches, average duration (kernel trace of the
    same run), bf16 MFMA flops per dispatch, TFLOP/s and fraction of the bf16 peak,
    MFMA busy % and the clock in GHz."""
    rows = _rows(_find_csv(pmc_dir, "counter_collection.csv"))
    mops, names = _by_dispatch(rows, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    busy, _ = _by_dispatch(rows, "SQ_VALU_MFMA_BUSY_CYCLES")
    gui, _ = _by_dispatch(rows, "GRBM_GUI_ACTIVE")
    xcc = _num_xcc(pmc_dir)
    gui = {d: v / xcc for d, v in gui.items()}  # cycles of one XCD = of the GPU clock
    dur = {}
    for r in _rows(_find_csv(pmc_dir, "kernel_trace.csv")):
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        dur[key] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    out = []
    for k in kernels:
        keys = [d for d, n in names.items() if k in n and d in dur and d in busy and d in gui]
        if not keys:
            raise SystemExit("no dispatches of kernels matching %r with every counter" % k)
        n = len(keys)
        ns = sum(dur[d] for d in keys) / n
        flops = sum(mops[d] for d in keys) * 512.0 / n
        cyc = sum(gui[d] for d in keys) / n
        util = 100.0 * sum(busy[d] for d in keys) / (sum(gui[d] for d in keys) * SIMD_NUM)
        tf = flops / ns / 1e3
        out.append({"kernel_match": k, "kernel_name": names[keys[0]], "dispatches": n,
                    "avg_us": round(ns / 1e3, 2), "mfma_gflop_per_dispatch": round(flops / 1e9, 3),
                    "tflops": round(tf, 1), "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                    "mfma_busy_pct": round(util, 1), "clock_ghz": round(cyc / ns, 3)})
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True, help="the command that produced the csv")
    s.add_argument("--title", default="Kernel durations")
    s.add_argument("--top", type=int, default=20, help="rows of the table (longest total first)")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True, action="append",
                   help="kernel name substring; repeat for a stage made of several kernels")
    t.add_argument("--stage", required=True, help="bench.py stage name of the kernel")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--cmd", required=True, help="the two commands, separated by ' ; '")
    t.add_argument("--out", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("pmc_dir")
    m.add_argument("--kernel", required=True, action="append", help="kernel name substring (repeat)")
    m.add_argument("--label", action="append", help="row label per --kernel (default: the substring)")
    m.add_argument("--cmd", required=True, help="the command that produced the run")
    m.add_argument("--title", default="Matrix-core use")
    a = ap.parse_args(argv)
    if a.cmd_name == "mfma":
        res = mfma_table(a.pmc_dir, a.kernel)
        labels = a.label or a.kernel
        print("# %s\n\nCommand:\n\n```\n%s\n```\n" % (a.title, a.cmd))
        print("| kernel | dispatches | avg us (counters on) | MFMA GFLOP / dispatch | TFLOP/s | of 2.5 PF | MFMA busy % | clock GHz |")
        print("|---|---:|---:|---:|---:|---:|---:|---:|")
        for lab, r in zip(labels, res):
            print("| %s | %d | %.2f | %.3f | %.1f | %.3f | %.1f | %.3f |" % (
                lab, r["dispatches"], r["avg_us"], r["mfma_gflop_per_dispatch"], r["tflops"],
                r["frac_bf16_peak"], r["mfma_busy_pct"], r["clock_ghz"]))
        return
    if a.cmd_name == "stats":
        print("# %s\n\nCommand:\n\n```\n%s\n```\n\n%s" % (a.title, a.cmd, stats_table(a.csv, a.top)))
        return
    res = traffic(a.fetch, a.write, a.kernel if len(a.kernel) > 1 else a.kernel[0], a.copy_bytes, a.stage)
    res["stage"] = a.stage
    res["command"] = a.cmd
    with open(a.out + ".json", "w") as fh:
        json.dump(res, fh, indent=1)
    with open(a.out + ".md", "w") as fh:
        fh.write("# HBM traffic of `%s` (%s)\n\nCommands:\n\n```\n%s\n```\n\n" % (a.stage, res["kernel_name"], a.cmd.replace(" ; ", "\n")))
        fh.write("| counter | kernel KiB/dispatch | copy KiB (of %d B) | factor | bytes/dispatch |\n|---|---:|---:|---:|---:|\n" % a.copy_bytes)
        fh.write("| FETCH_SIZE | %.1f | %.1f | %.4f | %d |\n" % (res["fetch_kib_per_dispatch"], res["copy_fetch_kib"], res["fetch_factor"], res["fetch_bytes"]))
        fh.write("| WRITE_SIZE | %.1f | %.1f | %.4f | %d |\n" % (res["write_kib_per_dispatch"], res["copy_write_kib"], res["write_factor"], res["write_bytes"]))
        fh.write("\nTraffic per dispatch: %.1f MB (source hash %s).\n" % (res["traffic_bytes"] / 1e6, res["source_sha256"][:16]))
    print(json.dumps(res))


if __name__ == "__main__":
    main()
