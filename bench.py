#!/usr/bin/env python3
"""Benchmark of the gated prefill path on one MI355X.

One step = the whole path above layer L's attention on one batch: gate scorer
over all N prompt tokens, Top-K selection with forced keep, compaction, and
the stack of upper layers on the K kept tokens (27 layers at N=32768,
K=4096, Qwen3-1.7B-shaped). Inputs and weights are seeded synthetic tensors
already resident in HBM when timing starts.

Prints ONE JSON line: tokens/s (prompt tokens through the gated path per
second), the gated-attention TFLOPS and its fraction of the bf16 MFMA peak,
the roofline entry of the dominant kernel, per-kernel figures, and the CPU
oracle timed on a bounded sample. `value` comes from the timed region alone
(K steps, no instrumentation); the per-kernel durations come from a second
pass of K steps with a HIP event recorded between every two kernels on the
launch stream (the events cost a few microseconds per kernel, which is why
they stay out of the timed region).
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "gated prefill tokens/s + attn TFLOPS (% MFMA peak) at N=32K,K=4096"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen32k")
    ap.add_argument("--k", type=int, default=None)
    ap.add_argument("--n", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused-norms", action="store_true",
                    help="run the two RMSNorms of each layer as kernels of their own instead of "
                         "fused into the QKV and gate/up GEMMs (norm weights folded at setup)")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="BYTES",
                    help="also run one plain device-to-device copy of BYTES (counter calibration "
                         "for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay pass (ms_per_step_hip_graph)")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time only the whole step (no per-kernel events)")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            self.ev[i] = h
        self.n = n

    def record(self, i, stream):
        assert self.hip.hipEventRecord(self.ev[i], stream) == 0

    def ms(self, a, b):
        f = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(f), self.ev[a], self.ev[b]) == 0
        return f.value

    def sub(self, start: int, count: int):
        """Address of events [start, start+count) as a hipEvent_t* for the C ABI."""
        assert start + count <= self.n
        return ctypes.c_void_p(ctypes.addressof(self.ev) + start * ctypes.sizeof(ctypes.c_void_p))

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(self.ev[i])


CPU_LAYERS = 5  # upper layers the CPU baseline runs (about 10 s of fp64 work at K=4096)


def cpu_baseline(w, dw_host_gate, host_layers):
    """The fp64 oracle timed on the host: scorer + selection + compaction on the
    whole prompt and the first len(host_layers) upper layers (distinct seeded
    weights) on all K kept tokens, the mean layer time scaled to the workload's
    layer count."""
    import numpy as np
    from threadpoolctl import threadpool_info
    import oracle as O
    gi = dw_host_gate
    Ws = [{"wq": L.wq.value, "wk": L.wk.value, "wv": L.wv.value, "wo": L.wo.value,
           "wg": L.wg.value, "wu": L.wu.value, "wd": L.wd.value, "attn_norm": L.attn_norm.value,
           "ffn_norm": L.ffn_norm.value, "t": L.t, "g": L.g} for L in host_layers]
    nl = len(Ws)
    t0 = time.perf_counter()
    s = O.gate_score(gi.h.value, gi.W1.value, gi.b1.value, gi.w2.value, gi.b2.value)
    t1 = time.perf_counter()
    kept, _ = O.topk_select(s, gi.keep_mask, gi.cu_in, gi.cu_kept)
    t2 = time.perf_counter()
    hc, pc, sc = O.compact(gi.h.value, None, s, kept, gi.cu_in, gi.cu_kept)
    t3 = time.perf_counter()
    x = hc
    for W in Ws:
        x = O.upper_layer(x, pc, sc, W, w.dims, gi.cu_kept)["x2"]
    t4 = time.perf_counter()
    t_est = (t3 - t0) + w.layers * (t4 - t3) / nl
    threads = 0
    for p in threadpool_info():
        if p.get("user_api") == "blas":
            threads = max(threads, int(p.get("num_threads", 0)))
    return {
        "value": w.T_in / t_est, "unit": "tokens/s",
        "cores": threads or len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": "fp64 numpy oracle: scorer+select+compact on the full %d-token prompt (%.2f s) "
                  "and %d of %d upper layers on all %d kept tokens (%.2f s), mean layer time x%d"
                  % (w.T_in, t3 - t0, nl, w.layers, w.T, t4 - t3, w.layers),
        "host_cores": len(os.sched_getaffinity(0)),
        "seconds_measured": round(t4 - t0, 2),
    }


def attention_bias_ratio(tg, torch, w, dw, gp, stream, reps=20):
    """The gated attention of the last layer's q/k/v with its gains g, and with g = 0
    (plain causal attention, same shape and kernel), each timed over `reps` calls."""
    L = len(dw.layers)
    dm = dw.dims
    lay = tg.upper_layer_ws_layout(dm, w.T)
    dt = gp.x.dtype
    nq = w.T * dm.Hq * dm.d
    q = gp.ws[lay.q:lay.q + nq * gp.x.element_size()].view(dt).view(w.T, dm.Hq, dm.d)
    k, v = gp.kcache[L - 1], gp.vcache[L - 1]
    t = dw.layers[L - 1].tensors["t"]
    g = dw.layers[L - 1].tensors["g"]
    o = torch.empty_like(q)
    ev = HipEvents(4)
    res = {}
    g0 = torch.zeros_like(g)
    for _ in range(3):  # alternate the two, keep the best of each (clock drift)
        for name, gg in (("bias", g), ("g0", g0)):
            tg.gated_attn_fwd(q, k, v, gp.s_c, t, gg, dw.cu_kept, w.max_k, o=o)
            ev.record(0, stream)
            for _ in range(reps):
                tg.gated_attn_fwd(q, k, v, gp.s_c, t, gg, dw.cu_kept, w.max_k, o=o)
            ev.record(1, stream)
            torch.cuda.synchronize()
            us = ev.ms(0, 1) * 1e3 / reps
            res[name] = min(res.get(name, us), us)
    ev.close()
    return {"us_bias": round(res["bias"], 2), "us_g0": round(res["g0"], 2),
            "ratio": round(res["bias"] / res["g0"], 3)}


def measured_traffic(stage, workload_name):
    """HBM bytes per launch of `stage` from the committed FETCH_SIZE / WRITE_SIZE summary
    (profiles/traffic_<stage>_<workload>.json), or None when there is none or the kernel
    sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (stage, workload_name))
    if not os.path.exists(path):
        return None
    from learned_token_pruning_post_amd.rocprof_summary import source_hash
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != source_hash(stage):
        return None
    return rec["traffic_bytes"]


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: runs on one GPU only (the gated prefill path of one device); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from learned_token_pruning_post_amd import binding as tg
    from learned_token_pruning_post_amd.pipeline import DeviceWorkload, GatedPrefill
    from learned_token_pruning_post_amd.workloads import workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    tg.lib()
    w = workload(args.workload, k=args.k, n=args.n, layers=args.layers)
    dm = w.dims
    print("[bench] generating %s: B=%d N=%s K=%s layers=%d" % (w.name, w.B, w.N[:4], w.K[:4], w.layers),
          file=sys.stderr, flush=True)
    want_cpu = not args.no_cpu_baseline
    dw = DeviceWorkload(w, keep_host=False, norms_folded=not args.unfused_norms)
    gp = GatedPrefill(dw)
    L = len(dw.layers)
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.reset_peak_memory_stats()

    per_step = 4 + L * (tg.LAYER_STAGES + 1)
    use_ev = not args.no_kernel_events
    EV0 = 6  # events 0-1: timed region, 2-3: per-kernel pass, 4-5: graph replays
    ev = HipEvents(EV0 + (per_step * args.steps if use_ev else 0))

    def step(sidx=None):
        if sidx is None:
            gp.run()
            return
        base = EV0 + sidx * per_step
        ev.record(base + 0, stream)
        gp.score()
        ev.record(base + 1, stream)
        gp.select()
        ev.record(base + 2, stream)
        gp.compact()
        ev.record(base + 3, stream)
        for l in range(L):
            tg.upper_layer_fwd(dw.layers[l], dw.dims, gp.x, gp.pos_c, gp.s_c, dw.cu_kept, w.max_k,
                               x_out=gp.x, kcache=gp.kcache[l], vcache=gp.vcache[l], ws=gp.ws,
                               events=ev.sub(base + 4 + l * (tg.LAYER_STAGES + 1), tg.LAYER_STAGES + 1),
                               rope_ready=l > 0, norms_folded=dw.norms_folded,
                               input_ssq=dw.norms_folded and l > 0)

    if args.calib_copy > 0:
        src = torch.empty(args.calib_copy, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print("[bench] warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: exactly `steps` steps, no instrumentation inside.
    print("[bench] timing %d steps" % args.steps, file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_host0 = time.perf_counter()
    ev.record(0, stream)
    for i in range(args.steps):
        step()
    ev.record(1, stream)
    torch.cuda.synchronize()
    t_host1 = time.perf_counter()
    total_ms = ev.ms(0, 1)
    # Second pass of `steps` steps with a HIP event between every kernel (on the
    # launch stream) for the per-kernel durations; the events add a few
    # microseconds per kernel, so this pass does not set `value`.
    ms_instr = None
    if use_ev:
        print("[bench] per-kernel pass, %d steps" % args.steps, file=sys.stderr, flush=True)
        ev.record(2, stream)
        for i in range(args.steps):
            step(i)
        ev.record(3, stream)
        torch.cuda.synchronize()
        ms_instr = ev.ms(2, 3) / args.steps
        attn_bias = attention_bias_ratio(tg, torch, w, dw, gp, stream)
    # The same step captured once into a HIP graph and replayed `steps` times
    # (reported beside `value`; the library makes no allocation, copy or
    # synchronisation inside its calls, so the whole step captures).
    ms_graph = None
    if not args.no_graph:
        print("[bench] HIP graph of one step: capture, %d replays" % args.steps, file=sys.stderr, flush=True)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        ev.record(4, stream)
        for i in range(args.steps):
            graph.replay()
        ev.record(5, stream)
        torch.cuda.synchronize()
        ms_graph = ev.ms(4, 5) / args.steps
        del graph
    ms_per_step = total_ms / args.steps
    tokens_per_s = w.T_in / (ms_per_step / 1e3)
    peak_mem = torch.cuda.max_memory_allocated()

    # ---- per-kernel durations ----
    T, D, Hq, Hkv, d, I, H1 = w.T, dm.D, dm.Hq, dm.Hkv, dm.d, dm.I, dm.H1
    elt = 2 if dm.dtype == "bf16" else 4
    attn_flop = sum(2.0 * d * Hq * k * (k + 1) for k in w.K)
    kflop = {
        "gate_score": 2.0 * w.T_in * D * H1 + 2.0 * w.T_in * H1,
        "qkv_rope_kv": 2.0 * T * D * (Hq + 2 * Hkv) * d,
        "gated_attn": attn_flop,
        "o_proj_resid": 2.0 * T * Hq * d * D,
        "gate_up_swiglu": 2.0 * T * D * 2 * I,
        "down_proj_resid": 2.0 * T * I * D,
    }
    kbytes = {
        "gate_score": w.T_in * D * elt + 4.0 * w.T_in + H1 * D * elt,
        "topk_select": 5.0 * w.T_in + 4.0 * T,
        "compact": 4.0 * T + 2.0 * T * D * elt + 4.0 * T + 8.0 * T,
        "rope_table": 4.0 * T + 4.0 * T * d,
    }
    if not dw.norms_folded:  # fused: stage 1 is x_in's sums of squares (first layer), stage 5 empty
        kbytes["rmsnorm_attn"] = 2.0 * T * D * elt
        kbytes["rmsnorm_ffn"] = 2.0 * T * D * elt
    kern = {}
    if use_ev:
        acc = {}
        for i in range(args.steps):
            base = EV0 + i * per_step
            for name, a in (("gate_score", 0), ("topk_select", 1), ("compact", 2)):
                acc.setdefault(name, []).append(ev.ms(base + a, base + a + 1))
            for l in range(L):
                lb = base + 4 + l * (tg.LAYER_STAGES + 1)
                for j, name in enumerate(tg.LAYER_STAGE_NAMES):
                    # stages that launch nothing in this layer (the RoPE table and,
                    # with fused norms, the sums of squares after the first layer;
                    # the second RMSNorm when fused) only time the events around them
                    empty = (name == "rope_table" and l > 0) or \
                            (dw.norms_folded and (name == "rmsnorm_ffn" or (name == "rmsnorm_attn" and l > 0)))
                    acc.setdefault("empty_stages" if empty else name, []).append(ev.ms(lb + j, lb + j + 1))
        for name, v in acc.items():
            avg_ms = float(np.mean(v))
            per_step_ms = float(np.sum(v)) / args.steps
            e = {"avg_us": round(avg_ms * 1e3, 2), "launches_per_step": len(v) // args.steps,
                 "ms_per_step": round(per_step_ms, 4)}
            if name == "empty_stages":  # event overhead of stages with no kernel
                e = {"avg_us": e["avg_us"], "stages_per_step": e["launches_per_step"],
                     "ms_per_step": e["ms_per_step"]}
            if name in kflop:
                tf = kflop[name] / (avg_ms * 1e-3) / 1e12
                e["tflops"] = round(tf, 1)
                e["frac_mfma_peak"] = round(tf / PEAK_BF16_TFLOPS, 4)
            if name in kbytes:
                gbs = kbytes[name] / (avg_ms * 1e-3) / 1e9
                e["gbs"] = round(gbs, 1)
                e["frac_hbm"] = round(gbs / PEAK_HBM_GBS, 4)
            kern[name] = e
    ev.close()

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dm.dtype,
        "data": "synthetic (seeded; no datasets or trained weights)",
        "config": {
            "workload": "%s: gated prefill, batch %d, N=%s, K=%s, %d unprunable tail tokens/seq, "
                        "%d upper layers, D=%d Hq=%d Hkv=%d d=%d I=%d, scorer %d->%d->1"
                        % (w.name, w.B, "/".join(map(str, w.N[:2])) + ("..." if w.B > 2 else ""),
                           "/".join(map(str, w.K[:2])) + ("..." if w.B > 2 else ""), w.F, L,
                           D, Hq, Hkv, d, I, D, H1),
            "batch": w.B, "n_prompt_tokens": w.T_in, "n_kept_tokens": T, "upper_layers": L,
            "rms_norm": "fused into the QKV and gate/up GEMMs (norm weights folded at setup)"
                        if dw.norms_folded else "separate kernels",
        },
        "host_wall_s_timed": round(t_host1 - t_host0, 3),
        "ms_per_step_with_kernel_events": round(ms_instr, 4) if ms_instr else None,
        "ms_per_step_hip_graph": round(ms_graph, 4) if ms_graph else None,
        "kept_tokens_per_s": round(w.T / (ms_per_step / 1e3), 1),
        "peak_device_mem_gb": round(peak_mem / 1e9, 3),
    }
    if use_ev:
        a = kern["gated_attn"]
        out["attn_tflops"] = a["tflops"]
        out["attn_frac_mfma_peak"] = a["frac_mfma_peak"]
        out["attn_bias_vs_g0"] = attn_bias
        sc_us = kern["topk_select"]["avg_us"] + kern["compact"]["avg_us"]
        sc_bytes = kbytes["topk_select"] + kbytes["compact"]
        out["select_compact"] = {"us": round(sc_us, 2), "bytes": sc_bytes,
                                 "gbs": round(sc_bytes / (sc_us * 1e-6) / 1e9, 1),
                                 "frac_hbm": round(sc_bytes / (sc_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        dom = max((n for n in kern if n != "empty_stages"), key=lambda n: kern[n]["ms_per_step"])
        de = kern[dom]
        traffic = measured_traffic(dom, w.name)
        if dom in kflop:
            out["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": de["tflops"],
                               "peak": PEAK_BF16_TFLOPS if dm.dtype == "bf16" else PEAK_F32_TFLOPS,
                               "unit": "TFLOP/s", "frac": de["frac_mfma_peak"], "traffic": traffic,
                               "work_per_launch": kflop[dom]}
        else:
            out["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": de["gbs"],
                               "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": de["frac_hbm"],
                               "traffic": traffic, "work_per_launch": kbytes[dom]}
        out["kernels"] = kern
    if want_cpu:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        from learned_token_pruning_post_amd.workloads import gate_inputs, layer_weights
        del gp, dw
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(
            w, gate_inputs(w), [layer_weights(w, l) for l in range(min(CPU_LAYERS, w.layers))])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
