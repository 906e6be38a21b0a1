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
    ap.add_argument("--no-memory", action="store_true",
                    help="skip the peak-memory comparison with the unpruned path")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the backward of the gated attention and of the scorer")
    ap.add_argument("--no-gdn", action="store_true",
                    help="skip timing the hybrid variant's Gated DeltaNet mixer")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-attention comparison over the pruned and the full cache")
    ap.add_argument("--no-prefill-time", action="store_true",
                    help="skip the whole-model prefill (all layers from layer 0) against the "
                         "same model run unpruned")
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
MODEL_LAYERS = 28  # decoder layers of Qwen3-1.7B, the model of the prefill-time comparison
GATE_LAYER = 1     # the gate position of the pages' main experiments
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}  # atol, rtol of the parity tests


def gpu_outputs_for_parity(torch, gp, n_layers):
    """One more pass of the path's stages on the GPU, with the outputs the oracle
    is compared against copied to the host: scores, selection, status, the
    compacted rows, positions and scores, x after the first upper layer and
    after `n_layers` of them."""
    gp.score()
    gp.select_compact()
    torch.cuda.synchronize()
    g = {"s": gp.s.cpu().numpy(), "kept": gp.kept.cpu().numpy(), "status": gp.status.cpu().numpy(),
         "x_c": gp.x.clone(), "pos_c": gp.pos_c.cpu().numpy(), "s_c": gp.s_c.cpu().numpy()}
    for l in range(n_layers):
        gp.layer(l)
        if l == 0:
            torch.cuda.synchronize()
            g["x_l0"] = gp.x.float().cpu().numpy()
    torch.cuda.synchronize()
    g["x_last"] = gp.x.float().cpu().numpy()
    g["x_c_bits"] = g["x_c"].cpu().view(torch.int16 if g["x_c"].dtype == torch.bfloat16 else torch.int32).numpy()
    g["x_c"] = g["x_c"].float().cpu().numpy().astype("float64")
    return g


def _excess(got, ref, atol, rtol):
    import numpy as np
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    return float(err.max()) if err.size else 0.0, float((err - (atol + rtol * np.abs(ref))).max()) if err.size else -1.0


def cpu_leg(w, gi, host_layers, g):
    """The fp64 oracle on the host: times scorer + selection + compaction on the
    whole prompt and the first len(host_layers) upper layers (distinct seeded
    weights) on all K kept tokens, the mean layer time scaled to the
    workload's layer count (the CPU baseline); and, with the GPU's outputs `g`
    of the same workload, the parity figures: per-stage maxima (each oracle
    stage fed the GPU's previous-stage output, as in the tests), selection
    flips between the GPU's fp32 scores and the oracle's fp64 ones, and the
    drift of x after len(host_layers) layers (reported, not gated)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    import oracle as O
    Ws = [{"wq": L.wq.value, "wk": L.wk.value, "wv": L.wv.value, "wo": L.wo.value,
           "wg": L.wg.value, "wu": L.wu.value, "wd": L.wd.value, "attn_norm": L.attn_norm.value,
           "ffn_norm": L.ffn_norm.value, "t": L.t, "g": L.g} for L in host_layers]
    nl = len(Ws)
    t0 = time.perf_counter()
    s = O.gate_score(gi.h.value, gi.W1.value, gi.b1.value, gi.w2.value, gi.b2.value)
    t1 = time.perf_counter()
    kept_own, _ = O.topk_select(s, gi.keep_mask, gi.cu_in, gi.cu_kept)
    t2 = time.perf_counter()
    O.compact(gi.h.value, None, s, kept_own, gi.cu_in, gi.cu_kept)
    t3 = time.perf_counter()
    x = g["x_c"]  # the GPU's compacted rows (exact values), so the drift below is the layers' own
    x_l0 = None
    for i, W in enumerate(Ws):
        x = O.upper_layer(x, g["pos_c"], g["s_c"], W, w.dims, gi.cu_kept)["x2"]
        if i == 0:
            x_l0 = x
    t4 = time.perf_counter()
    t_est = (t3 - t0) + w.layers * (t4 - t3) / nl
    threads = 0
    for p in threadpool_info():
        if p.get("user_api") == "blas":
            threads = max(threads, int(p.get("num_threads", 0)))
    base = {
        "value": w.T_in / t_est, "unit": "tokens/s",
        "cores": threads or len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": "fp64 numpy oracle: scorer+select+compact on the full %d-token prompt (%.2f s) "
                  "and %d of %d upper layers on all %d kept tokens (%.2f s), mean layer time x%d"
                  % (w.T_in, t3 - t0, nl, w.layers, w.T, t4 - t3, w.layers),
        "host_cores": len(os.sched_getaffinity(0)),
        "seconds_measured": round(t4 - t0, 2),
    }
    # ---- parity on the benchmarked workload ----
    atol, rtol = TOL[w.dims.dtype]
    s_err, s_exc = _excess(g["s"], s, atol, rtol)
    ref_kept, ref_flags = O.topk_select(g["s"], gi.keep_mask, gi.cu_in, gi.cu_kept)
    sel_exact = bool(np.array_equal(g["kept"], ref_kept.astype(np.int32)) and
                     np.array_equal(g["status"], ref_flags.astype(np.int32)))
    flips = int(np.setdiff1d(g["kept"], kept_own).size)
    hc, pc, sc = O.compact(gi.h.value, None, g["s"], g["kept"].astype(np.int64), gi.cu_in, gi.cu_kept)
    hbits = (np.ascontiguousarray(gi.h.bits[g["kept"]]).view(np.int16) if gi.h.bits is not None
             else np.ascontiguousarray(hc, dtype=np.float32).view(np.int32))
    comp_exact = bool(np.array_equal(g["x_c_bits"], hbits) and np.array_equal(g["pos_c"], pc) and
                      np.array_equal(g["s_c"].view(np.int32), sc.astype(np.float32).view(np.int32)))
    l0_err, l0_exc = _excess(g["x_l0"], x_l0, atol, rtol)
    dr_err, dr_exc = _excess(g["x_last"], x, atol, rtol)
    parity = {
        "tolerance": {"atol": atol, "rtol": rtol},
        "scores_max_abs_err": s_err, "scores_within_tol": s_exc <= 0,
        "selection_bit_exact": sel_exact, "compaction_bit_exact": comp_exact,
        "layer0_out_max_abs_err": l0_err, "layer0_out_within_tol": l0_exc <= 0,
        "selection_flips_vs_fp64_scores": flips,
        "selection_flips_note": "kept tokens chosen from the GPU's fp32 scores that the oracle's fp64 "
                                "scores would not keep (of %d); reported, not gated" % w.T,
        "drift_layers": nl,
        "drift_max_abs_err": dr_err, "drift_max_excess_over_tol": dr_exc,
        "drift_note": "x after %d stacked layers, GPU chain vs oracle chain from the same compacted "
                      "rows (errors compound; reported, not gated)" % nl,
    }
    return base, parity


def memory_vs_unpruned(torch, tg, w):
    """Peak device memory of one pass of the path with one upper layer at the
    workload's budgets and the same path with every token kept (K = N, the
    unpruned layer), each measured from an empty allocator; and the K/V cache
    of 27 upper layers at both budgets from the layer shapes."""
    from learned_token_pruning_post_amd.pipeline import DeviceWorkload, GatedPrefill
    from learned_token_pruning_post_amd.workloads import Workload
    res = {}
    for name, K in (("pruned", w.K), ("unpruned", w.N)):
        wl = Workload(w.name, w.cfg_id, w.N, tuple(K), w.F, w.dims, 1, w.salient)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        dw = DeviceWorkload(wl, n_layers=1, norms_folded=True)
        gp = GatedPrefill(dw)
        gp.run()
        torch.cuda.synchronize()
        res[name] = (torch.cuda.max_memory_allocated() - base) / 1e9
        del gp, dw
    torch.cuda.empty_cache()
    dm = w.dims
    elt = 2 if dm.dtype == "bf16" else 4
    kv = lambda toks: 27 * 2 * toks * dm.Hkv * dm.d * elt / 1e9
    return {"peak_gb_one_layer_pruned": round(res["pruned"], 3),
            "peak_gb_one_layer_unpruned": round(res["unpruned"], 3),
            "peak_ratio_unpruned_over_pruned": round(res["unpruned"] / res["pruned"], 2),
            "kv_cache_gb_27_layers_pruned": round(kv(w.T), 3),
            "kv_cache_gb_27_layers_unpruned": round(kv(w.T_in), 3),
            "note": "same N, scorer + select + compact + one upper layer; unpruned = every token kept "
                    "(K = N); K/V of 27 upper layers from the shapes"}


def prefill_vs_unpruned(torch, tg, dw, reps=3):
    """The whole prefill of a MODEL_LAYERS-layer model with the gate at layer
    GATE_LAYER (layers below it and its attention on all N tokens, its FFN and
    the layers above on the K kept ones; one tg_full_prefill call) against the
    same layers run unpruned (every layer on every token, plain attention; one
    tg_upper_layer_stack_fwd call): GPU time of each with HIP events on the
    launch stream (mean of `reps` after one warmup), and the peak device
    memory each one's buffers and run add to the resident weights. Layers
    beyond the workload's own are generated from the same seeds; the input
    rows are the workload's, standing in for layer 0's input."""
    from learned_token_pruning_post_amd.pipeline import FullPrefill, UnprunedPrefill
    w = dw.w
    if len(dw.layers) < MODEL_LAYERS:
        print("[bench] uploading layers %d..%d for the whole-model prefill"
              % (len(dw.layers), MODEL_LAYERS - 1), file=sys.stderr, flush=True)
        dw.extend_layers(MODEL_LAYERS)
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents(2 * reps)
    res = {}
    makers = (("pruned", lambda: FullPrefill(dw, n_below=GATE_LAYER)),
              ("unpruned", lambda: UnprunedPrefill(dw)))
    for name, make in makers:
        print("[bench] whole-model prefill, %s: 1 warmup + %d timed" % (name, reps),
              file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        run = make()
        run.run()
        torch.cuda.synchronize()
        peak = (torch.cuda.max_memory_allocated() - base) / 1e9
        for i in range(reps):
            ev.record(2 * i, stream)
            run.run()
            ev.record(2 * i + 1, stream)
        torch.cuda.synchronize()
        ms = [ev.ms(2 * i, 2 * i + 1) for i in range(reps)]
        res[name] = (sum(ms) / reps, peak)
        del run
    ev.close()
    torch.cuda.empty_cache()
    (tp, mp), (tu, mu) = res["pruned"], res["unpruned"]
    return {"layers": MODEL_LAYERS, "gate_layer": GATE_LAYER, "n_prompt_tokens": w.T_in, "n_kept_tokens": w.T,
            "pruned_ms": round(tp, 3), "unpruned_ms": round(tu, 3), "speedup": round(tu / tp, 2),
            "pruned_tokens_per_s": round(w.T_in / (tp / 1e3), 1),
            "unpruned_tokens_per_s": round(w.T_in / (tu / 1e3), 1),
            "peak_gb_pruned": round(mp, 3), "peak_gb_unpruned": round(mu, 3),
            "peak_ratio_unpruned_over_pruned": round(mu / mp, 2),
            "note": "GPU time of the decoder layers' prefill (no embedding, LM head or sampling); "
                    "peak = buffers and run on top of the resident weights (K/V of every layer "
                    "included); mean of %d runs after one warmup" % reps}


def backward_timing(torch, tg, w, reps=5):
    """The gate's gradient path at the workload's shapes: the gated attention's
    backward (tg_gated_attn_bwd) over one sequence of the kept-token count,
    next to its forward, and the scorer's backward (tg_gate_score_bwd) over
    the whole prompt. Seeded random operands; HIP events on the launch stream,
    mean of `reps` calls after a warm-up. Algorithmic work: attention backward
    = 2.5x the forward's matmul flops (S recomputed, dP, dV, dK, dQ); scorer
    backward = the three products W1 h, dz W1 and dz^T h (2 T D H1 each)."""
    dm = w.dims
    if dm.dtype != "bf16":
        return None
    gen = torch.Generator(device="cuda").manual_seed(2000 + w.cfg_id)
    rnd = lambda shape, sc=1.0: (sc * torch.randn(shape, generator=gen, device="cuda")).to(torch.bfloat16)
    uni = lambda shape: torch.rand(shape, generator=gen, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents(2)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ev.record(0, stream)
        for _ in range(reps):
            fn()
        ev.record(1, stream)
        torch.cuda.synchronize()
        return ev.ms(0, 1) / reps * 1e3

    K, Hq, Hkv, d = w.K[0], dm.Hq, dm.Hkv, dm.d
    q, k, v, dO = rnd((K, Hq, d)), rnd((K, Hkv, d)), rnd((K, Hkv, d)), rnd((K, Hq, d))
    s_c, t, g = uni(K), 0.8 + 0.4 * uni(Hq), 2.0 * uni(Hq)
    cu = torch.tensor([0, K], dtype=torch.int32, device="cuda")
    o, lse = tg.gated_attn_fwd(q, k, v, s_c, t, g, cu, K, want_lse=True)
    ws = torch.empty(max(tg.lib().tg_gated_attn_bwd_workspace_size(1, K, K, Hq, Hkv, d, 1), 1), dtype=torch.uint8,
                     device="cuda")
    fwd_us = timed(lambda: tg.gated_attn_fwd(q, k, v, s_c, t, g, cu, K, o=o, lse=lse, want_lse=True))
    bwd_us = timed(lambda: tg.gated_attn_bwd(q, k, v, s_c, t, g, cu, K, o, lse, dO, ws=ws))
    attn_flop = 2.0 * d * Hq * K * (K + 1)
    del q, k, v, dO, o, lse, ws
    N, D, H1 = w.N[0], dm.D, dm.H1
    h, W1, b1, w2, b2 = rnd((N, D)), rnd((H1, D), 0.02), rnd((H1,), 0.02), rnd((H1,), 0.02), rnd((1,), 0.02)
    s = tg.gate_score(h, W1, b1, w2, b2)
    ds = torch.randn(N, generator=gen, device="cuda")
    ws = torch.empty(max(tg.lib().tg_gate_score_bwd_workspace_size(N, D, H1, 1), 1), dtype=torch.uint8,
                     device="cuda")
    sc_us = timed(lambda: tg.gate_score_bwd(h, W1, b1, w2, s, ds, ws=ws))
    sc_flop = 3 * 2.0 * N * D * H1
    del h, W1, ws
    ev.close()
    torch.cuda.empty_cache()
    bt = 2.5 * attn_flop / (bwd_us * 1e-6) / 1e12
    st = sc_flop / (sc_us * 1e-6) / 1e12
    return {"attn_bwd_us": round(bwd_us, 1), "attn_fwd_us": round(fwd_us, 1),
            "attn_bwd_over_fwd": round(bwd_us / fwd_us, 2), "attn_bwd_tflops": round(bt, 1),
            "attn_bwd_frac_mfma_peak": round(bt / PEAK_BF16_TFLOPS, 4),
            "scorer_bwd_us": round(sc_us, 1), "scorer_bwd_tflops": round(st, 1),
            "scorer_bwd_frac_mfma_peak": round(st / PEAK_BF16_TFLOPS, 4),
            "shapes": "attention: 1 sequence of %d kept tokens, %d/%d heads x %d; scorer: %d tokens, %d -> %d"
                      % (K, Hq, Hkv, d, N, D, H1),
            "note": "mean of %d calls after a warm-up; attention backward work = 2.5x the forward's" % reps}


def gdn_timing(torch, tg, w, reps=3):
    """The hybrid variant's Gated DeltaNet mixer (tg_gdn_fwd) over one sequence
    of the kept-token count, at the model's head shapes (one head per query
    head, dk = dv = head dim): seeded random operands, HIP events on the launch
    stream. bf16 runs the chunked form (64-token chunks): a parallel prep
    kernel over all chunks and heads, then a scan over the chunks of each
    sequence, head and 32 state rows. Work reported two ways: the token
    recurrence's 6 dk dv flops per token and head, and the matrix-core flops
    the chunked form performs (per chunk and head: K K^T, Q K^T, two halves of
    T times K^ and V, then U, the two output products and the state update)."""
    dm = w.dims
    dt = torch.bfloat16 if dm.dtype == "bf16" else torch.float32
    K, H, d = w.K[0], dm.Hq, dm.d
    gen = torch.Generator(device="cuda").manual_seed(3000 + w.cfg_id)
    rnd = lambda shape: torch.randn(shape, generator=gen, device="cuda").to(dt)
    q, k, v = rnd((K, H, d)), rnd((K, H, d)), rnd((K, H, d))
    al = 0.8 + 0.2 * torch.rand((K, H), generator=gen, device="cuda")
    be = torch.rand((K, H), generator=gen, device="cuda")
    cu = torch.tensor([0, K], dtype=torch.int32, device="cuda")
    o = torch.empty_like(v)
    need = tg.lib().tg_gdn_workspace_size(K, 1, H, d, d, tg.dtype_code(dt))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents(2)
    tg.gdn_fwd(q, k, v, al, be, cu, o=o, ws=ws)
    torch.cuda.synchronize()
    ev.record(0, stream)
    for _ in range(reps):
        tg.gdn_fwd(q, k, v, al, be, cu, o=o, ws=ws)
    ev.record(1, stream)
    torch.cuda.synchronize()
    us = ev.ms(0, 1) / reps * 1e3
    ev.close()
    flop = 6.0 * K * H * d * d
    C = 64
    mfma_flop = ((K + C - 1) // C) * H * (2.0 * C * C * d * 2 + 2 * (2.0 * C * C * d) * 2
                                         + 2.0 * C * d * d * 3 + 2.0 * C * C * d)
    out = {"us": round(us, 1), "tokens": K, "heads": H, "dk": d, "dv": d,
           "recurrence_tflops": round(flop / (us * 1e-6) / 1e12, 3),
           "workspace_mb": round(need / 1e6, 1),
           "note": "one sequence; mean of %d calls after a warm-up" % reps}
    if dt == torch.bfloat16:
        tf = mfma_flop / (us * 1e-6) / 1e12
        out.update({"chunked_mfma_gflop": round(mfma_flop / 1e9, 2), "mfma_tflops": round(tf, 2),
                    "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                    "scan_workgroups": H * (d // 32)})
    return out


DECODE_BATCH = 16  # sequences per decode step
DECODE_GEN = 128   # tokens each has generated so far (segment B of its cache)


def decode_vs_unpruned(torch, tg, w, reps=20):
    """Decode attention of one layer for one step of DECODE_BATCH sequences:
    each has the workload's K kept prompt tokens plus DECODE_GEN generated
    tokens cached (tg_decode_attn_fwd, two cache segments), against the same
    batch with all N prompt tokens cached (no pruning). Seeded random cache
    and queries at the model's head shapes; HIP events on the launch stream
    around `reps` calls after two warm-up calls. Bytes: K and V rows of every
    cached key and kv head, one score per key, q in and o out."""
    dm = w.dims
    dt = torch.bfloat16 if dm.dtype == "bf16" else torch.float32
    elt = 2 if dm.dtype == "bf16" else 4
    B, Hq, Hkv, d, G = DECODE_BATCH, dm.Hq, dm.Hkv, dm.d, DECODE_GEN
    gen = torch.Generator(device="cuda").manual_seed(1000 + w.cfg_id)
    rnd = lambda shape: torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(dt)
    uni = lambda shape: torch.rand(shape, generator=gen, device="cuda", dtype=torch.float32)
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents(2)
    res = {}
    for name, n in (("pruned", w.K[0]), ("unpruned", w.N[0])):
        kA, vA, sA = rnd((B * n, Hkv, d)), rnd((B * n, Hkv, d)), uni(B * n)
        kB, vB, sB = rnd((B, G, Hkv, d)), rnd((B, G, Hkv, d)), uni((B, G))
        q, t, g = rnd((B, Hq, d)), 0.8 + 0.4 * uni(Hq), 2.0 * uni(Hq)
        cuA = torch.arange(0, B * n + 1, n, dtype=torch.int32, device="cuda")
        lenB = torch.full((B,), G, dtype=torch.int32, device="cuda")
        o = torch.empty_like(q)
        status = torch.empty(B, dtype=torch.int32, device="cuda")
        need = tg.lib().tg_decode_attn_workspace_size(B, n + G, Hq, Hkv, d, tg.dtype_code(dt))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        call = lambda: tg.decode_attn_fwd(q, kA, vA, sA, cuA, kB, vB, sB, lenB, t, g, n + G, o=o,
                                          status=status, ws=ws)
        for _ in range(2):
            call()
        torch.cuda.synchronize()
        ev.record(0, stream)
        for _ in range(reps):
            call()
        ev.record(1, stream)
        torch.cuda.synchronize()
        assert not status.any().item(), "decode status flags"
        us = ev.ms(0, 1) / reps * 1e3
        nbytes = 2.0 * B * (n + G) * Hkv * d * elt + 4.0 * B * (n + G) + 2.0 * B * Hq * d * elt
        res[name] = (us, nbytes)
        del kA, vA, sA, kB, vB, sB, q, o, ws
    ev.close()
    torch.cuda.empty_cache()
    (tp, bp), (tu, bu) = res["pruned"], res["unpruned"]
    return {"batch": B, "kept_prompt_keys": w.K[0], "prompt_keys_unpruned": w.N[0], "generated_keys": G,
            "heads": "%d/%d x %d" % (Hq, Hkv, d), "pruned_us": round(tp, 2), "unpruned_us": round(tu, 2),
            "speedup": round(tu / tp, 2), "pruned_bytes": bp,
            "pruned_gbs": round(bp / (tp * 1e-6) / 1e9, 1),
            "pruned_frac_hbm": round(bp / (tp * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "unpruned_gbs": round(bu / (tu * 1e-6) / 1e9, 1),
            "note": "attention of one layer for one decode step; mean of %d calls after two warm-ups" % reps}


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

    per_step = 3 + L * (tg.LAYER_STAGES + 1)
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
        gp.select_compact()
        ev.record(base + 2, stream)
        for l in range(L):
            tg.upper_layer_fwd(dw.layers[l], dw.dims, gp.x, gp.pos_c, gp.s_c, dw.cu_kept, w.max_k,
                               x_out=gp.x, kcache=gp.kcache[l], vcache=gp.vcache[l], ws=gp.ws,
                               events=ev.sub(base + 3 + l * (tg.LAYER_STAGES + 1), tg.LAYER_STAGES + 1),
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
        ms_instr_total = ev.ms(2, 3) / args.steps
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
    step_flop = kflop["gate_score"] + w.layers * sum(
        kflop[n] for n in ("qkv_rope_kv", "gated_attn", "o_proj_resid", "gate_up_swiglu", "down_proj_resid"))
    kbytes = {
        "gate_score": w.T_in * D * elt + 4.0 * w.T_in + H1 * D * elt,
        # selection (scores and mask bytes in, kept indices out) + compaction (rows
        # in and out, positions out, scores gathered in and out; the kept indices
        # are not read back)
        "select_compact": 5.0 * w.T_in + 4.0 * T + 2.0 * T * D * elt + 4.0 * T + 8.0 * T,
        "rope_table": 4.0 * T + 4.0 * T * d,
    }
    if not dw.norms_folded:  # fused: stage 1 is x_in's sums of squares (first layer), stage 5 empty
        kbytes["rmsnorm_attn"] = 2.0 * T * D * elt
        kbytes["rmsnorm_ffn"] = 2.0 * T * D * elt
    kern = {}
    gaps = None
    if use_ev:
        acc = {}
        spans, in_step_gaps = [], []
        last = per_step - 1  # the last layer's closing event
        for i in range(args.steps):
            base = EV0 + i * per_step
            # first event -> last event of the step; the windows no kernel entry
            # covers are host-side hops (compaction end -> first layer, layer ->
            # layer), where the GPU waits for Python to marshal the next call
            span = ev.ms(base, base + last)
            covered = ev.ms(base, base + 2)
            for l in range(L):
                lb = base + 3 + l * (tg.LAYER_STAGES + 1)
                covered += ev.ms(lb, lb + tg.LAYER_STAGES)
            spans.append(span)
            in_step_gaps.append(span - covered)
            for name, a in (("gate_score", 0), ("select_compact", 1)):
                acc.setdefault(name, []).append(ev.ms(base + a, base + a + 1))
            for l in range(L):
                lb = base + 3 + l * (tg.LAYER_STAGES + 1)
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
        ms_instr = float(np.mean(spans))
        gaps = {"in_step_ms_per_step": round(float(np.mean(in_step_gaps)), 4),
                "between_steps_ms_per_step": round(ms_instr_total - ms_instr, 4),
                "note": "GPU idle while the host marshals the next call: compaction end to the "
                        "first layer and between layers inside a step, and from one step's last "
                        "kernel to the next step's first; in no kernel entry"}
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
        # algorithmic flops of one step (scorer on the prompt, every upper layer's
        # projections and gated attention on the kept tokens) over the timed step
        "path_tflops": round(step_flop / (ms_per_step * 1e-3) / 1e12, 1),
        "path_frac_mfma_peak": round(step_flop / (ms_per_step * 1e-3) / 1e12 /
                                     (PEAK_BF16_TFLOPS if dm.dtype == "bf16" else PEAK_F32_TFLOPS), 4),
        "peak_device_mem_gb": round(peak_mem / 1e9, 3),
    }
    if use_ev:
        a = kern["gated_attn"]
        out["attn_tflops"] = a["tflops"]
        out["attn_frac_mfma_peak"] = a["frac_mfma_peak"]
        out["attn_bias_vs_g0"] = attn_bias
        sc_us = kern["select_compact"]["avg_us"]
        sc_bytes = kbytes["select_compact"]
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
        out["host_gaps"] = gaps
    n_cpu_layers = min(CPU_LAYERS, w.layers)
    g_out = gpu_outputs_for_parity(torch, gp, n_cpu_layers) if want_cpu else None
    del gp
    torch.cuda.empty_cache()
    if not args.no_prefill_time:
        out["prefill_vs_unpruned"] = prefill_vs_unpruned(torch, tg, dw)
    del dw
    torch.cuda.empty_cache()
    if not args.no_memory:
        print("[bench] peak memory against the unpruned path (K = N, one layer)", file=sys.stderr, flush=True)
        out["memory"] = memory_vs_unpruned(torch, tg, w)
    if not args.no_backward:
        print("[bench] backward of the gated attention and of the scorer", file=sys.stderr, flush=True)
        out["backward"] = backward_timing(torch, tg, w)
    if not args.no_gdn:
        print("[bench] Gated DeltaNet mixer over the kept tokens", file=sys.stderr, flush=True)
        out["gdn_kept_tokens"] = gdn_timing(torch, tg, w)
    if not args.no_decode:
        print("[bench] decode attention over the pruned and the full cache", file=sys.stderr, flush=True)
        out["decode_vs_unpruned"] = decode_vs_unpruned(torch, tg, w)
    if want_cpu:
        print("[bench] timing the CPU oracle on a bounded sample; parity on this workload",
              file=sys.stderr, flush=True)
        from learned_token_pruning_post_amd.workloads import gate_inputs, layer_weights
        out["cpu_baseline"], out["parity"] = cpu_leg(
            w, gate_inputs(w), [layer_weights(w, l) for l in range(n_cpu_layers)], g_out)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
