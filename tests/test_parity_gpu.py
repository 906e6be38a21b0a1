"""GPU parity: every step of the HIP path against the fp64 CPU oracle.

Per-stage comparison on identical inputs: each oracle stage is fed the GPU's
output of the stage before it. Selection, compaction and positions must match
bit for bit; scores, attention and layer outputs fall within atol 2e-2 /
rtol 1e-2 (bf16 storage, fp32 accumulation) or 1e-4 / 1e-4 (fp32).
Full-size workloads run in the same launch configuration as the benchmark
(the GatedPrefill driver) and compare sampled rows where the oracle cannot do
all of them in seconds.
"""
import numpy as np
import pytest
import torch

import oracle as O
from helpers import TOL, assert_close, bits, f64, layer_dict, sample_rows, say, ws_view
from learned_token_pruning_post_amd import binding as tg
from learned_token_pruning_post_amd.pipeline import DeviceWorkload, GatedPrefill, to_device
from learned_token_pruning_post_amd.workloads import (ModelDims, activations, custom,
                                                      scores_with_ties, workload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    tg.lib()  # raises loudly if the HIP library is missing


def _stage_parity(w, score_rows=None, layer_rows_per_seq=None, seed=0, norms_folded=False):
    dt = w.dims.dtype
    say("workload", w.name, "N", w.N[:3], "K", w.K[:3], "T", w.T, "folded norms" if norms_folded else "")
    dw = DeviceWorkload(w, n_layers=1, keep_host=True, norms_folded=norms_folded)
    gi = dw.host_gate
    gp = GatedPrefill(dw)

    # ---- scorer ----
    gp.score()
    torch.cuda.synchronize()
    s = gp.s.cpu().numpy()
    rows = np.arange(w.T_in) if score_rows is None else \
        np.unique(np.concatenate([np.random.default_rng(seed).choice(w.T_in, score_rows, replace=False),
                                  [0, w.T_in - 1]]))
    ref = O.gate_score(gi.h.value[rows], gi.W1.value, gi.b1.value, gi.w2.value, gi.b2.value)
    e = assert_close(s[rows], ref, dt, "scores")
    say("  scorer max err", e)

    # ---- select + compact: bit exact on the same fp32 scores ----
    ref_kept, flags = O.topk_select(s, gi.keep_mask, gi.cu_in, gi.cu_kept)
    hc_ref, pc_ref, sc_ref = O.compact(gi.h.device_array, None, s, ref_kept, gi.cu_in, gi.cu_kept)

    def check_selected(what):
        torch.cuda.synchronize()
        assert np.array_equal(gp.status.cpu().numpy(), flags.astype(np.int32)), what
        assert np.array_equal(gp.kept.cpu().numpy(), ref_kept.astype(np.int32)), what
        assert np.array_equal(bits(gp.x), np.ascontiguousarray(hc_ref).view(bits(gp.x).dtype)), what
        assert np.array_equal(gp.pos_c.cpu().numpy(), pc_ref.astype(np.int32)), what
        assert np.array_equal(gp.s_c.cpu().numpy().view(np.int32),
                              sc_ref.astype(np.float32).view(np.int32)), what

    for buf in (gp.kept, gp.status, gp.pos_c):
        buf.fill_(-5)
    gp.select()   # the two calls one after the other
    gp.compact()
    check_selected("tg_topk_select + tg_compact")
    for buf in (gp.kept, gp.status, gp.pos_c):
        buf.fill_(-5)
    gp.x.zero_()
    gp.select_compact()  # the fused pass the whole step runs (last: the layer reads its output)
    check_selected("tg_select_compact")
    say("  select + compact bit-exact", len(ref_kept), "(separate calls and fused)")

    # ---- one upper layer, stage by stage ----
    x_in = f64(gp.x)
    pos_c = gp.pos_c.cpu().numpy()
    s_c = gp.s_c.cpu().numpy().astype(np.float64)
    gp.layer(0)
    torch.cuda.synchronize()
    W = layer_dict(dw.host_layers[0])
    dm = w.dims
    lay = tg.upper_layer_ws_layout(dw.dims, w.T)
    tdt = gp.x.dtype
    T = w.T
    q_g = f64(ws_view(gp.ws, lay.q, (T, dm.Hq, dm.d), tdt))
    a_g = f64(ws_view(gp.ws, lay.attn, (T, dm.Hq, dm.d), tdt))
    x1_g = f64(ws_view(gp.ws, lay.x1, (T, dm.D), tdt))
    act_g = f64(ws_view(gp.ws, lay.act, (T, dm.I), tdt))
    k_g, v_g = f64(gp.kcache[0]), f64(gp.vcache[0])
    x2_g = f64(gp.x)
    cu = gi.cu_kept
    lrows = np.arange(T) if layer_rows_per_seq is None else sample_rows(cu, layer_rows_per_seq, seed)
    n1, q_r, k_r, v_r = O.qkv_rope(x_in, pos_c, W, dm, rows=lrows)
    errs = {}
    errs["k"] = assert_close(k_g[lrows], k_r[lrows], dt, "k cache")
    errs["v"] = assert_close(v_g[lrows], v_r[lrows], dt, "v cache")
    errs["q"] = assert_close(q_g[lrows], q_r[lrows], dt, "q")
    o_r, _ = O.gated_attention(q_g, k_g, v_g, s_c, W["t"], W["g"], cu, rows=lrows)
    errs["attn"] = assert_close(a_g[lrows], o_r[lrows], dt, "attention")
    errs["x1"] = assert_close(x1_g[lrows], O.o_proj(x_in[lrows], a_g[lrows], W["wo"]), dt, "x1")
    _, act_r = O.swiglu_act(x1_g[lrows], W, dm.rms_eps)
    errs["act"] = assert_close(act_g[lrows], act_r, dt, "swiglu act")
    errs["x2"] = assert_close(x2_g[lrows], O.down_proj(x1_g[lrows], act_g[lrows], W["wd"]), dt, "x out")
    say("  layer stage max errs", {k: "%.3g" % v for k, v in errs.items()})


def test_stages_tiny_fp32():
    _stage_parity(workload("tiny"))


def test_stages_qwen8k():
    _stage_parity(workload("qwen8k"))


@pytest.mark.parametrize("k", [4096, 512, 2048, 8192])
def test_stages_qwen32k(k):
    _stage_parity(workload("qwen32k", k=k, layers=1), score_rows=8192,
                  layer_rows_per_seq=None if k <= 2048 else 384)


def test_stages_qwen32k_folded_norms():
    """The benchmark's launch configuration: RMSNorms fused into the GEMMs."""
    _stage_parity(workload("qwen32k", k=4096, layers=1), score_rows=8192, layer_rows_per_seq=384,
                  norms_folded=True)


@pytest.mark.parametrize("n", [65536, 131072])
def test_stages_long(n):
    _stage_parity(workload("long", n=n), score_rows=8192, layer_rows_per_seq=384)


def test_stages_multibudget():
    _stage_parity(workload("multibudget"), score_rows=8192, layer_rows_per_seq=96)


@pytest.mark.parametrize("folded", [False, True])
def test_stages_ragged_small_bf16(folded):
    dims = ModelDims(D=256, Hq=4, Hkv=2, d=64, I=512, H1=96, dtype="bf16")
    w = custom(21, N=[300, 1, 77, 1000], K=[150, 1, 77, 333], F=1, dims=dims)
    _stage_parity(w, norms_folded=folded)


@pytest.mark.parametrize("folded", [False, True])
def test_stages_ragged_bf16_k_and_v_head_in_one_pair(folded):
    # Hq + Hkv odd: the QKV epilogue's head pair (2, 3) of the only 256-feature
    # tile holds the k head (rotated) and the v head (not rotated). D = 128
    # also takes the fused norm's scalar path (D/64 = 2 sums per row).
    dims = ModelDims(D=128, Hq=2, Hkv=1, d=64, I=256, H1=64, dtype="bf16")
    w = custom(23, N=[97, 260], K=[40, 130], F=2, dims=dims)
    _stage_parity(w, norms_folded=folded)


@pytest.mark.parametrize("seed", range(6))
def test_stages_random_small_configs(seed):
    """Seeded random shapes within the supported set (bf16): model widths,
    head dims, GQA groups, batch sizes, lengths, budgets and forced tails drawn
    per seed; every stage against the oracle, with and without folded norms."""
    rng = np.random.default_rng(1000 + seed)
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4]))
    Hkv = int(rng.choice([1, 2]))
    D = int(rng.choice([128, 256, 384]))
    I = int(rng.choice([256, 512]))
    H1 = int(rng.choice([64, 128, 256]))
    dims = ModelDims(D=D, Hq=Hkv * G, Hkv=Hkv, d=d, I=I, H1=H1, dtype="bf16")
    B = int(rng.integers(1, 5))
    N = [int(x) for x in rng.integers(16, 700, size=B)]
    F = int(rng.integers(0, 9))
    K = [int(rng.integers(max(F, 1), n + 1)) for n in N]
    w = custom(1100 + seed, N=N, K=K, F=F, dims=dims)
    _stage_parity(w, norms_folded=bool(seed % 2))


def test_stages_ragged_gqa4_fp32_d128():
    dims = ModelDims(D=256, Hq=8, Hkv=2, d=128, I=384, H1=40, dtype="f32")
    w = custom(22, N=[129, 64, 200], K=[65, 64, 3], F=3, dims=dims)
    _stage_parity(w)


def test_layer_stack_reuses_rope_table():
    """Layer 1 of a stack runs on the RoPE table layer 0 left in the workspace
    (TG_LAYER_ROPE_READY): its outputs equal a run that rebuilds the table, and
    its post-RoPE K cache and its output x match the oracle layer fed layer 0's
    GPU output."""
    w = workload("qwen8k", layers=2)
    dw = DeviceWorkload(w, n_layers=2, keep_host=True)
    gp = GatedPrefill(dw)
    gp.score()
    gp.select()
    gp.compact()
    gp.layer(0)
    x_in = gp.x.clone()
    gp.layer(1)
    torch.cuda.synchronize()
    reuse = (gp.x.clone(), gp.kcache[1].clone(), gp.vcache[1].clone())
    fresh_ws = torch.zeros_like(gp.ws)
    x2, k2, v2, _ = tg.upper_layer_fwd(dw.layers[1], dw.dims, x_in, gp.pos_c, gp.s_c, dw.cu_kept,
                                       w.max_k, ws=fresh_ws)
    torch.cuda.synchronize()
    for a, b, name in zip(reuse, (x2, k2, v2), ("x out", "k cache", "v cache")):
        assert torch.equal(a, b), name
    W = layer_dict(dw.host_layers[1])
    rows = sample_rows(dw.host_gate.cu_kept, 256, 1)
    ref = O.upper_layer(f64(x_in), gp.pos_c.cpu().numpy(), f64(gp.s_c), W, w.dims,
                        dw.host_gate.cu_kept, rows=rows)
    e = assert_close(f64(reuse[1])[rows], ref["k"][rows], w.dims.dtype, "layer-1 k cache")
    ex = assert_close(f64(reuse[0])[rows], ref["x2"][rows], w.dims.dtype, "layer-1 x out")
    say("  layer 1 on the reused RoPE table: bit-identical to a rebuilt one; k err %.3g, "
        "x out err %.3g" % (e, ex))


def test_layer_stack_folded_norms_reuses_input_sums():
    """With folded norms, layer 1 reads its input's row sums of squares from the
    workspace, as written by layer 0's down projection (TG_LAYER_INPUT_SSQ): its
    outputs equal a run on a fresh workspace, where a kernel of its own computes
    them, bit for bit; x out and the k cache match the oracle layer fed layer
    0's GPU output."""
    w = workload("qwen8k", layers=2)
    dw = DeviceWorkload(w, n_layers=2, keep_host=True, norms_folded=True)
    gp = GatedPrefill(dw)
    gp.score()
    gp.select()
    gp.compact()
    gp.layer(0)
    x_in = gp.x.clone()
    gp.layer(1)
    torch.cuda.synchronize()
    reuse = (gp.x.clone(), gp.kcache[1].clone(), gp.vcache[1].clone())
    fresh_ws = torch.zeros_like(gp.ws)
    x2, k2, v2, _ = tg.upper_layer_fwd(dw.layers[1], dw.dims, x_in, gp.pos_c, gp.s_c, dw.cu_kept,
                                       w.max_k, ws=fresh_ws, norms_folded=True)
    torch.cuda.synchronize()
    for a, b, name in zip(reuse, (x2, k2, v2), ("x out", "k cache", "v cache")):
        assert torch.equal(a, b), name
    W = layer_dict(dw.host_layers[1])
    rows = sample_rows(dw.host_gate.cu_kept, 256, 1)
    ref = O.upper_layer(f64(x_in), gp.pos_c.cpu().numpy(), f64(gp.s_c), W, w.dims,
                        dw.host_gate.cu_kept, rows=rows)
    e = assert_close(f64(reuse[1])[rows], ref["k"][rows], w.dims.dtype, "layer-1 k cache")
    ex = assert_close(f64(reuse[0])[rows], ref["x2"][rows], w.dims.dtype, "layer-1 x out")
    say("  layer 1 on its input sums from layer 0: bit-identical to a fresh run; k err %.3g, "
        "x out err %.3g" % (e, ex))


def test_native_layer_stack_equals_layer_loop():
    """tg_upper_layer_stack_fwd (one call for all layers, flags set per layer
    inside) gives the same x and K/V caches as calling tg_upper_layer_fwd layer
    by layer, bit for bit, with and without folded norms."""
    dims = ModelDims(D=256, Hq=4, Hkv=2, d=64, I=512, H1=64, dtype="bf16")
    w = custom(93, N=[500, 260], K=[180, 77], F=8, dims=dims, layers=3)
    for folded in (False, True):
        dw = DeviceWorkload(w, n_layers=3, norms_folded=folded)
        gp = GatedPrefill(dw)
        gp.score()
        gp.select()
        gp.compact()
        x0 = gp.x.clone()
        for l in range(3):
            gp.layer(l)
        torch.cuda.synchronize()
        loop = (gp.x.clone(), gp.kcache.clone(), gp.vcache.clone())
        gp.x.copy_(x0)
        gp.kcache.zero_()
        gp.vcache.zero_()
        tg.upper_layer_stack_fwd(dw.layers, dw.dims, gp.x, gp.pos_c, gp.s_c, dw.cu_kept, w.max_k,
                                 gp.kcache, gp.vcache, ws=torch.zeros_like(gp.ws), norms_folded=folded)
        torch.cuda.synchronize()
        for a, r, name in zip((gp.x, gp.kcache, gp.vcache), loop, ("x", "k cache", "v cache")):
            assert torch.equal(a, r), "%s (folded=%s)" % (name, folded)


def test_native_step_equals_staged_calls():
    """tg_gated_prefill (the whole step in one call) gives the same scores,
    selection, status, compacted positions and scores, x and K/V caches as the
    stage-by-stage calls, bit for bit."""
    dims = ModelDims(D=256, Hq=4, Hkv=2, d=64, I=512, H1=64, dtype="bf16")
    w = custom(94, N=[640, 300, 90], K=[200, 150, 90], F=16, dims=dims, layers=2)
    dw = DeviceWorkload(w, n_layers=2, norms_folded=True)
    gp = GatedPrefill(dw)
    gp.score()
    gp.select()
    gp.compact()
    for l in range(2):
        gp.layer(l)
    torch.cuda.synchronize()
    bufs = ("s", "kept", "status", "pos_c", "s_c", "x", "kcache", "vcache")
    staged = {n: getattr(gp, n).clone() for n in bufs}
    for n in bufs:
        getattr(gp, n).zero_()
    gp.run()
    torch.cuda.synchronize()
    for n in bufs:
        assert torch.equal(getattr(gp, n), staged[n]), n


def test_step_replays_from_a_hip_graph():
    """The whole step (scorer, select, compact, 3 fused layers) captured into a
    HIP graph: the library makes no allocation, copy or synchronisation inside
    its calls, so capture works, and every replay (with eager work of the
    program and synchronisations between replays) equals the eager step bit for
    bit."""
    dims = ModelDims(D=256, Hq=4, Hkv=2, d=64, I=512, H1=64, dtype="bf16")
    w = custom(91, N=[700, 333, 64], K=[200, 99, 64], F=16, dims=dims, layers=3)
    dw = DeviceWorkload(w, n_layers=3, norms_folded=True)
    gp = GatedPrefill(dw)
    gp.run()
    torch.cuda.synchronize()
    ref = (gp.x.clone(), gp.kept.clone(), gp.kcache.clone(), gp.vcache.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gp.run()
    for i in range(3):
        gp.x.zero_()
        gp.kcache.zero_()
        junk = torch.randn(1 << 20, device="cuda")  # eager work between replays
        gp.score()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert float(junk.abs().sum()) > 0
        for a, r, name in zip((gp.x, gp.kept, gp.kcache, gp.vcache), ref, ("x", "kept", "k cache", "v cache")):
            assert torch.equal(a, r), "replay %d: %s" % (i, name)


def test_chunked_select_replays_from_a_hip_graph():
    """The chunked selection (max_n above 32768: six kernels, histograms
    cleared by a kernel, no memset) captured once into a HIP graph and replayed
    on new scores, with eager work between replays: every replay equals the
    oracle on the scores of that replay, bit for bit."""
    dev = "cuda"
    N, K = [50000, 20000, 33000], [3000, 19000, 4096]
    T_in, T = sum(N), sum(K)
    cu_in = np.concatenate([[0], np.cumsum(N)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(K)]).astype(np.int32)
    rng = np.random.default_rng(58)
    mask = np.zeros(T_in, np.uint8)
    mask[rng.choice(T_in, 600, replace=False)] = 1
    s_dev = torch.from_numpy(scores_with_ties(58, T_in, 41)).to(dev)
    m_dev = torch.from_numpy(mask).to(dev)
    ci, ck = torch.from_numpy(cu_in).to(dev), torch.from_numpy(cu_k).to(dev)
    max_n = max(N)
    need = tg.lib().tg_topk_select_workspace_size(len(N), T_in, max_n)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    kept = torch.empty(T, dtype=torch.int32, device=dev)
    status = torch.empty(len(N), dtype=torch.int32, device=dev)
    tg.topk_select(s_dev, m_dev, ci, ck, T, max_n, kept=kept, status=status, ws=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tg.topk_select(s_dev, m_dev, ci, ck, T, max_n, kept=kept, status=status, ws=ws)
    for i in range(3):
        s_new = scores_with_ties(59 + i, T_in, 7 + 30 * i)
        s_dev.copy_(torch.from_numpy(s_new))
        kept.fill_(-7)
        junk = torch.randn(1 << 20, device=dev)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert float(junk.abs().sum()) > 0
        ref, flags = O.topk_select(s_new, mask, cu_in, cu_k)
        assert np.array_equal(status.cpu().numpy(), flags.astype(np.int32)), "replay %d" % i
        assert np.array_equal(kept.cpu().numpy(), ref.astype(np.int32)), "replay %d" % i


def test_folded_norm_weights_not_ones():
    """Fold non-unit norm weights into the projections and run the fused layer:
    every stage matches the oracle evaluated with the unfolded weights."""
    dims = ModelDims(D=256, Hq=4, Hkv=2, d=64, I=512, H1=64, dtype="bf16")
    w = custom(24, N=[200, 333], K=[120, 200], F=4, dims=dims)
    dw = DeviceWorkload(w, n_layers=1, keep_host=True)
    gp = GatedPrefill(dw)
    gp.score()
    gp.select()
    gp.compact()
    torch.cuda.synchronize()
    lw = dw.host_layers[0]
    rng = np.random.default_rng(5)
    t = dict(dw.layers[0].tensors)
    norms = {}
    for n in ("attn_norm", "ffn_norm"):
        v = torch.from_numpy(rng.uniform(0.5, 1.5, dims.D).astype(np.float32)).to(torch.bfloat16)
        norms[n] = v.float().numpy().astype(np.float64)
        t[n] = v.cuda()
    for n in ("wq", "wk", "wv", "wg", "wu"):
        t[n] = t[n].clone()
    for n in ("wq", "wk", "wv"):
        tg.fold_norm_weights(t["attn_norm"], t[n])
    for n in ("wg", "wu"):
        tg.fold_norm_weights(t["ffn_norm"], t[n])
    # the fold is W * w rounded to bf16, column by column
    ref_fold = (f64(dw.layers[0].tensors["wq"]) * norms["attn_norm"][None, :]).astype(np.float32)
    assert np.array_equal(bits(t["wq"]), bits(torch.from_numpy(ref_fold).to(torch.bfloat16)))
    x_in = gp.x.clone()
    x_out, k_g, v_g, ws = tg.upper_layer_fwd(tg.UpperLayerWeights(t), dw.dims, x_in, gp.pos_c, gp.s_c,
                                             dw.cu_kept, w.max_k, norms_folded=True)
    torch.cuda.synchronize()
    W = layer_dict(lw)
    W["attn_norm"], W["ffn_norm"] = norms["attn_norm"], norms["ffn_norm"]
    lay = tg.upper_layer_ws_layout(dw.dims, w.T)
    T = w.T
    x_in64 = f64(x_in)
    _, q_r, k_r, v_r = O.qkv_rope(x_in64, gp.pos_c.cpu().numpy(), W, dims)
    assert_close(f64(k_g), k_r, "bf16", "k cache")
    assert_close(f64(v_g), v_r, "bf16", "v cache")
    assert_close(f64(ws_view(ws, lay.q, (T, dims.Hq, dims.d), torch.bfloat16)), q_r, "bf16", "q")
    x1_g = f64(ws_view(ws, lay.x1, (T, dims.D), torch.bfloat16))
    act_g = f64(ws_view(ws, lay.act, (T, dims.I), torch.bfloat16))
    _, act_r = O.swiglu_act(x1_g, W, dims.rms_eps)
    assert_close(act_g, act_r, "bf16", "swiglu act")
    assert_close(f64(x_out), O.down_proj(x1_g, act_g, W["wd"]), "bf16", "x out")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fold_norm_weights_ragged_shapes(dtype):
    """W[r, c] * w[c] rounded once to the dtype, for rows/cols that are not tile multiples."""
    g = torch.Generator().manual_seed(7)
    for rows, cols in [(1, 1), (37, 129), (300, 64)]:
        W = torch.randn(rows, cols, generator=g).to(dtype)
        wn = (torch.rand(cols, generator=g) + 0.5).to(dtype)
        ref = (W.double() * wn.double()[None, :]).float().to(dtype)
        got = tg.fold_norm_weights(wn.cuda(), W.cuda())
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), ref), (rows, cols)


def test_scorer_2048x256_ragged_token_counts():
    """The 2048 -> 256 scorer on batches whose token count is not a multiple
    of its 128-token tiles (a tail tile with 1, 127 and 129 tokens) and on a
    single token, against the oracle on every row."""
    dims = ModelDims(D=2048, Hq=16, Hkv=8, d=128, I=6144, H1=256, dtype="bf16")
    for seed, N in ((24, [1]), (25, [129]), (26, [1000, 383]), (27, [127, 128, 1])):
        w = custom(seed, N=N, K=[1] * len(N), F=0, dims=dims)
        dw = DeviceWorkload(w, n_layers=0, keep_host=True)
        gp = GatedPrefill(dw)
        gp.score()
        torch.cuda.synchronize()
        gi = dw.host_gate
        ref = O.gate_score(gi.h.value, gi.W1.value, gi.b1.value, gi.w2.value, gi.b2.value)
        e = assert_close(gp.s.cpu().numpy(), ref, "bf16", "scores N=%s" % N)
        say("  scorer 2048x256 N=%s max err %.3g" % (N, e))


def test_scorer_wide_hidden_uses_partials():
    dims = ModelDims(D=128, Hq=2, Hkv=1, d=64, I=128, H1=600, dtype="bf16")
    w = custom(23, N=[777], K=[10], F=2, dims=dims)
    dw = DeviceWorkload(w, n_layers=0, keep_host=True)
    gp = GatedPrefill(dw)
    gp.score()
    torch.cuda.synchronize()
    gi = dw.host_gate
    ref = O.gate_score(gi.h.value, gi.W1.value, gi.b1.value, gi.w2.value, gi.b2.value)
    assert_close(gp.s.cpu().numpy(), ref, "bf16", "scores H1=600")


# ---------------------------------------------------------------------------
# selection edge cases
# ---------------------------------------------------------------------------

def _select_case(N, K, mask, s, max_n=None):
    dev = "cuda"
    cu_in = np.concatenate([[0], np.cumsum(N)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(K)]).astype(np.int32)
    st = torch.from_numpy(s.astype(np.float32)).to(dev)
    mt = torch.from_numpy(mask.astype(np.uint8)).to(dev)
    if max_n is None:
        max_n = int(max(N) if len(N) else 0)
    kept, status = tg.topk_select(st, mt, torch.from_numpy(cu_in).to(dev), torch.from_numpy(cu_k).to(dev),
                                  int(cu_k[-1]), max_n)
    torch.cuda.synchronize()
    return kept.cpu().numpy(), status.cpu().numpy()[:len(N)], cu_in, cu_k


def test_select_ties_specials_ragged():
    rng = np.random.default_rng(31)
    N = [1, 7, 1000, 5000, 40000, 3, 2049, 150000]
    K = [1, 3, 100, 5000, 4096, 0, 2049, 1]
    T_in = sum(N)
    s = scores_with_ties(31, T_in, 37)
    special = rng.choice(T_in, 4000, replace=False)
    s[special[:1000]] = np.nan
    s[special[1000:2000]] = -0.0
    s[special[2000:3000]] = 0.0
    s[special[3000:3500]] = np.inf
    s[special[3500:]] = -np.inf
    mask = np.zeros(T_in, np.uint8)
    cu = np.concatenate([[0], np.cumsum(N)])
    for b in range(len(N)):
        nf = min(K[b], max(0, N[b] // 50))
        if nf:
            mask[cu[b] + rng.choice(N[b], nf, replace=False)] = 1
    kept, status, cu_in, cu_k = _select_case(N, K, mask, s)
    ref, flags = O.topk_select(s.astype(np.float32), mask, cu_in, cu_k)
    assert np.array_equal(status, flags.astype(np.int32))
    assert np.array_equal(kept, ref.astype(np.int32))
    # determinism
    kept2, _, _, _ = _select_case(N, K, mask, s)
    assert np.array_equal(kept, kept2)


def test_select_small_batch_ties_specials_ragged():
    """A batch of 8 sequences of at most 32768 tokens: ties, NaN, +-0, +-inf
    and forced tokens mixed in, unaligned sequence starts, one token, an
    empty sequence, budget = length and budget = forced count; bit-exact with
    the oracle, flags included, and the same result on a second call."""
    rng = np.random.default_rng(51)
    N = [1, 7, 1001, 5000, 32768, 0, 2049, 20003]
    K = [1, 3, 100, 5000, 4096, 0, 40, 1]
    T_in = sum(N)
    s = scores_with_ties(51, T_in, 37)
    special = rng.choice(T_in, 4000, replace=False)
    s[special[:1000]] = np.nan
    s[special[1000:2000]] = -0.0
    s[special[2000:3000]] = 0.0
    s[special[3000:3500]] = np.inf
    s[special[3500:]] = -np.inf
    mask = np.zeros(T_in, np.uint8)
    cu = np.concatenate([[0], np.cumsum(N)])
    for b in range(len(N)):
        nf = 40 if b == 6 else min(K[b], max(0, N[b] // 50))   # sequence 6: K = F
        if nf:
            mask[cu[b] + rng.choice(N[b], nf, replace=False)] = 1
    kept, status, cu_in, cu_k = _select_case(N, K, mask, s)
    ref, flags = O.topk_select(s.astype(np.float32), mask, cu_in, cu_k)
    assert np.array_equal(status, flags.astype(np.int32))
    assert np.array_equal(kept, ref.astype(np.int32))
    kept2, _, _, _ = _select_case(N, K, mask, s)
    assert np.array_equal(kept, kept2)


def test_select_one_bin_nan_threshold_and_flags():
    """Every candidate key in one bin (all scores equal: the first indices
    win), the threshold among NaN candidates, and flagged budgets (forced
    count above the budget, budget above the length) next to good
    sequences."""
    N = [32768, 3000, 100, 100, 700]
    K = [4096, 2990, 10, 101, 650]
    T_in = sum(N)
    cu = np.concatenate([[0], np.cumsum(N)])
    s = np.full(T_in, 0.5, np.float32)
    s[cu[1]:cu[2]] = np.linspace(-1, 1, N[1], dtype=np.float32)
    s[cu[1] + np.arange(0, N[1], 100)] = np.nan          # 30 NaN: 20 of them kept
    s[cu[4]:cu[5]] = np.float32(0.25)
    s[cu[4] + 3] = np.float32(0.75)
    mask = np.zeros(T_in, np.uint8)
    mask[cu[2]:cu[2] + 20] = 1                           # 20 forced > K = 10
    mask[cu[4] + 600:cu[5]] = 1
    kept, status, cu_in, cu_k = _select_case(N, K, mask, s)
    ref, flags = O.topk_select(s, mask, cu_in, cu_k)
    assert np.array_equal(status, flags.astype(np.int32))
    assert status[2] & 1 and status[3] & 2
    for b in range(len(N)):
        lo, hi = cu_k[b], cu_k[b + 1]
        if flags[b] & 3:
            assert (kept[lo:hi] == -1).all(), b
        else:
            assert np.array_equal(kept[lo:hi], ref[lo:hi].astype(np.int32)), b


def test_select_all_equal_and_budget_extremes():
    N = [4096, 4096, 4096, 5000]
    K = [100, 4096, 512, 4999]
    s = np.full(sum(N), 0.5, np.float32)
    s[4096 * 3:] = np.linspace(0, 1, 5000, dtype=np.float32)
    mask = np.zeros(sum(N), np.uint8)
    mask[4096 * 2 + 4096 - 512:4096 * 3] = 1   # K = F: exactly the forced tail
    kept, status, cu_in, cu_k = _select_case(N, K, mask, s)
    ref, flags = O.topk_select(s, mask, cu_in, cu_k)
    assert np.array_equal(kept, ref.astype(np.int32)) and not status.any()


def test_select_many_small_random_batches():
    """One batch of 300 short sequences (0 to 80 tokens) with random budgets,
    forced tokens, few distinct values (ties), NaN, -0.0, +-inf and +-0
    mixed in: bit-exact against the oracle, status flags included (budgets
    below the forced count and above the length are flagged)."""
    rng = np.random.default_rng(36)
    nseq = 300
    N = [int(x) for x in rng.integers(0, 81, size=nseq)]
    specials = np.array([np.nan, -0.0, 0.0, np.inf, -np.inf, 1e-30, -1e-30], np.float32)
    s = rng.choice(rng.uniform(-2, 2, 6).astype(np.float32), size=sum(N))
    pick = rng.random(sum(N)) < 0.15
    s[pick] = rng.choice(specials, size=int(pick.sum()))
    mask = (rng.random(sum(N)) < 0.1).astype(np.uint8)
    K = []
    off = 0
    for n in N:
        f = int(mask[off:off + n].sum())
        r = rng.random()
        k = f - 1 if (r < 0.03 and f > 0) else (n + 1 if r < 0.06 else int(rng.integers(min(f, n), n + 1)))
        K.append(max(k, 0))
        off += n
    kept, status, cu_in, cu_k = _select_case(N, K, mask, s)
    ref, flags = O.topk_select(s, mask, cu_in, cu_k)
    assert np.array_equal(status, flags.astype(np.int32))
    ok = (flags & 3) == 0
    for b in range(nseq):
        lo, hi = cu_k[b], cu_k[b + 1]
        if ok[b]:
            assert np.array_equal(kept[lo:hi], ref[lo:hi].astype(np.int32)), b
        else:
            assert (kept[lo:hi] == -1).all(), b
    assert (~ok).any() and ok.sum() > 250


def test_select_and_compact_empty_sequences():
    """Sequences with no tokens (N_b = 0, K_b = 0) between ordinary ones: the
    selection skips them and its other outputs match the oracle; compaction
    of the result is a bit copy."""
    rng = np.random.default_rng(35)
    N = [0, 5, 0, 900, 0]
    K = [0, 5, 0, 77, 0]
    s = rng.random(sum(N)).astype(np.float32)
    mask = np.zeros(sum(N), np.uint8)
    mask[5 + 890:] = 1
    kept, status, cu_in, cu_k = _select_case(N, K, mask, s)
    ref, _ = O.topk_select(s, mask, cu_in, cu_k)
    assert np.array_equal(kept, ref.astype(np.int32)) and not status.any()
    D = 64
    h = activations(35, 1, (sum(N), D), "bf16")
    dev = "cuda"
    hc, pc, sc = tg.compact(to_device(h), None, torch.from_numpy(s).to(dev), torch.from_numpy(kept).to(dev),
                            torch.from_numpy(cu_in).to(dev), torch.from_numpy(cu_k).to(dev))
    torch.cuda.synchronize()
    hr, pr, sr = O.compact(h.device_array, None, s, ref, cu_in, cu_k)
    assert np.array_equal(bits(hc), np.ascontiguousarray(hr).view(bits(hc).dtype))
    assert np.array_equal(pc.cpu().numpy(), pr.astype(np.int32))


def test_layer_ignores_empty_sequences():
    """Empty sequences in the kept-token batch (repeated cu_kept entries) change
    nothing: the layer's outputs equal those of the batch without them, bit for
    bit (every kernel works per token row or per sequence)."""
    dims = ModelDims(D=256, Hq=4, Hkv=2, d=64, I=512, H1=64, dtype="bf16")
    w = custom(92, N=[300, 200], K=[150, 97], F=8, dims=dims)
    dw = DeviceWorkload(w, n_layers=1, norms_folded=True)
    gp = GatedPrefill(dw)
    gp.score()
    gp.select()
    gp.compact()
    torch.cuda.synchronize()
    x0 = gp.x.clone()
    outs = []
    for cu in ([0, 150, 247], [0, 0, 150, 150, 150, 247, 247]):
        cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda")
        x, kc, vc, _ = tg.upper_layer_fwd(dw.layers[0], dw.dims, x0, gp.pos_c, gp.s_c, cu_t, 150,
                                          norms_folded=True)
        torch.cuda.synchronize()
        outs.append((x.clone(), kc.clone(), vc.clone()))
    for a, b, name in zip(outs[0], outs[1], ("x out", "k cache", "v cache")):
        assert torch.equal(a, b), name


def test_select_rounds_ties_across_rounds():
    """Sequences longer than one LDS round (32768 tokens): equal scores whose ties
    straddle rounds, forced tokens in every round, a ragged last round."""
    N = [100003, 32769, 65536, 7]
    K = [50001, 32768, 40000, 7]
    T_in = sum(N)
    s = np.full(T_in, 0.25, np.float32)
    rng = np.random.default_rng(3)
    s[N[0]:N[0] + N[1]] = rng.integers(0, 5, N[1]).astype(np.float32)  # 5 levels, heavy ties
    s[N[0] + N[1]:] = scores_with_ties(4, N[2] + N[3], 11)
    mask = np.zeros(T_in, np.uint8)
    mask[rng.choice(N[0], 300, replace=False)] = 1
    mask[N[0] + rng.choice(N[1], 50, replace=False)] = 1
    kept, status, cu_in, cu_k = _select_case(N, K, mask, s)
    ref, flags = O.topk_select(s, mask, cu_in, cu_k)
    assert np.array_equal(status, flags.astype(np.int32))
    assert np.array_equal(kept, ref.astype(np.int32))


def test_select_chunked_path_budget_extremes_and_short_sequences():
    """The chunked path (max_n above 32768) on every kind of sequence in one
    batch: budget = length, budget = forced count, all scores equal, one key
    above a block of equal ones, lengths on and off 4096-token chunk borders,
    unaligned sequence starts, one token, an empty sequence."""
    rng = np.random.default_rng(41)
    N = [40000, 33001, 36864, 8192, 1, 0, 50003, 4097]
    K = [40000, 300, 1000, 8191, 1, 0, 20000, 4084]
    T_in = sum(N)
    cu = np.concatenate([[0], np.cumsum(N)])
    s = scores_with_ties(41, T_in, 23)
    mask = np.zeros(T_in, np.uint8)
    mask[cu[1] + rng.choice(N[1], 300, replace=False)] = 1  # K = F
    s[cu[2]:cu[3]] = 0.5                                     # all equal
    s[cu[3]:cu[4]] = 0.25
    s[cu[3] + 5000] = 0.75                                   # one key above the block
    mask[cu[6] + rng.choice(N[6], 700, replace=False)] = 1
    s[cu[7]:cu[8]] = np.linspace(-1, 1, N[7], dtype=np.float32)
    s[cu[7] + rng.choice(N[7], 40, replace=False)] = np.nan
    for max_n in (max(N), 1 << 20):
        kept, status, cu_in, cu_k = _select_case(N, K, mask, s, max_n=max_n)
        ref, flags = O.topk_select(s, mask, cu_in, cu_k)
        assert np.array_equal(status, flags.astype(np.int32))
        assert np.array_equal(kept, ref.astype(np.int32))


def test_select_chunked_path_sequence_longer_than_max_n_is_flagged():
    """On the chunked path a sequence longer than max_n would have chunks
    outside the grid: it is flagged with -1 slots, the others are selected."""
    N, K = [50000, 40000, 100], [10, 20, 5]
    s = scores_with_ties(6, sum(N), 9)
    mask = np.zeros(sum(N), np.uint8)
    kept, status, cu_in, cu_k = _select_case(N, K, mask, s, max_n=40000)
    assert status[0] == tg.DEV_LEN_GT_MAX_N and status[1] == 0 and status[2] == 0
    assert (kept[:10] == -1).all()
    ref, _ = O.topk_select(s, mask, cu_in, cu_k)
    assert np.array_equal(kept[10:], ref[10:].astype(np.int32))


def test_select_sequence_longer_than_max_n_is_flagged():
    """The one-round kernel (max_n <= 32768) on a longer sequence: that
    sequence is flagged and its slots are -1; the others are selected."""
    dev = "cuda"
    N, K = [40000, 1000], [10, 20]
    s = scores_with_ties(5, sum(N), 7)
    cu_in = np.concatenate([[0], np.cumsum(N)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(K)]).astype(np.int32)
    kept, status = tg.topk_select(torch.from_numpy(s).to(dev), None, torch.from_numpy(cu_in).to(dev),
                                  torch.from_numpy(cu_k).to(dev), int(cu_k[-1]), 32768)
    torch.cuda.synchronize()
    kept, status = kept.cpu().numpy(), status.cpu().numpy()
    assert status[0] == tg.DEV_LEN_GT_MAX_N and status[1] == 0
    assert (kept[:10] == -1).all()
    ref, _ = O.topk_select(s, np.zeros(sum(N), np.uint8), cu_in, cu_k)
    assert np.array_equal(kept[10:], ref[10:].astype(np.int32))


def test_select_error_flags():
    N = [10, 10, 10]
    K = [3, 11, 4]  # seq 0: 5 forced > 3; seq 1: K > N
    s = np.linspace(0, 1, 30, dtype=np.float32)
    mask = np.zeros(30, np.uint8)
    mask[:5] = 1
    kept, status, _, cu_k = _select_case([10, 10, 10], K, mask, s)
    assert status.tolist() == [1, 2, 0]
    assert (kept[:3] == -1).all() and (kept[3:14] == -1).all()
    ref, _ = O.select_one(s[20:30], mask[20:30].astype(bool), 4)
    assert kept[14:].tolist() == (ref + 20).tolist()


# ---------------------------------------------------------------------------
# compaction with explicit positions, odd row sizes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,D", [("bf16", 6), ("bf16", 2048), ("f32", 100), ("f32", 3)])
def test_compact_positions_and_row_sizes(dtype, D):
    rng = np.random.default_rng(41)
    N = [50, 1, 300]
    K = [10, 1, 299]
    T_in = sum(N)
    h = activations(41, 7, (T_in, D), dtype)
    ht = to_device(h)
    pos = np.concatenate([np.sort(rng.choice(10 ** 6, n, replace=False)) for n in N]).astype(np.int32)
    s = rng.random(T_in).astype(np.float32)
    cu_in = np.concatenate([[0], np.cumsum(N)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(K)]).astype(np.int32)
    ref_kept, _ = O.topk_select(s, None, cu_in, cu_k)
    dev = "cuda"
    kept_t = torch.from_numpy(ref_kept.astype(np.int32)).to(dev)
    hc, pc, sc = tg.compact(ht, torch.from_numpy(pos).to(dev), torch.from_numpy(s).to(dev), kept_t,
                            torch.from_numpy(cu_in).to(dev), torch.from_numpy(cu_k).to(dev))
    torch.cuda.synchronize()
    hr, pr, sr = O.compact(h.device_array, pos, s, ref_kept, cu_in, cu_k)
    assert np.array_equal(bits(hc), np.ascontiguousarray(hr).view(bits(hc).dtype))
    assert np.array_equal(pc.cpu().numpy(), pr.astype(np.int32))
    assert np.array_equal(sc.cpu().numpy(), sr)


# ---------------------------------------------------------------------------
# attention kernels on their own
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,G,d", [("bf16", 1, 64), ("bf16", 2, 64), ("bf16", 4, 64),
                                       ("bf16", 1, 128), ("bf16", 2, 128), ("bf16", 4, 128),
                                       ("f32", 2, 64), ("f32", 2, 128), ("f32", 4, 128)])
def test_attention_varlen(dtype, G, d):
    lens = [1, 31, 64, 65, 200, 129, 0, 3]
    T = sum(lens)
    Hkv = 2
    Hq = Hkv * G
    q = activations(51, 1, (T, Hq, d), dtype)
    k = activations(51, 2, (T, Hkv, d), dtype)
    v = activations(51, 3, (T, Hkv, d), dtype)
    rng = np.random.default_rng(51)
    s_c = rng.random(T).astype(np.float32)
    t = rng.uniform(0.8, 1.2, Hq).astype(np.float32)
    g = rng.uniform(0.0, 2.0, Hq).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    dev = "cuda"
    o, lse = tg.gated_attn_fwd(to_device(q), to_device(k), to_device(v), torch.from_numpy(s_c).to(dev),
                               torch.from_numpy(t).to(dev), torch.from_numpy(g).to(dev),
                               torch.from_numpy(cu).to(dev), max(lens), want_lse=True)
    torch.cuda.synchronize()
    o_r, lse_r = O.gated_attention(q.value, k.value, v.value, s_c, t, g, cu)
    assert_close(f64(o), o_r, dtype, "attention out")
    assert_close(lse.cpu().numpy(), lse_r, dtype, "lse")
    o2, _ = tg.gated_attn_fwd(to_device(q), to_device(k), to_device(v), torch.from_numpy(s_c).to(dev),
                              torch.from_numpy(t).to(dev), torch.from_numpy(g).to(dev),
                              torch.from_numpy(cu).to(dev), max(lens))
    torch.cuda.synchronize()
    assert torch.equal(o, o2)  # deterministic


@pytest.mark.parametrize("G,d", [(1, 128), (4, 64)])
def test_attention_many_short_sequences(G, d):
    """Enough query tiles that workgroups take pairs of them (heavy, light),
    next to the few-tile batches above, where each takes one tile."""
    rng = np.random.default_rng(54)
    lens = [int(x) for x in rng.integers(0, 300, size=90)] + [300, 1]
    T = sum(lens)
    Hkv = 2
    Hq = Hkv * G
    q = activations(54, 1, (T, Hq, d), "bf16")
    k = activations(54, 2, (T, Hkv, d), "bf16")
    v = activations(54, 3, (T, Hkv, d), "bf16")
    s_c = rng.random(T).astype(np.float32)
    t = rng.uniform(0.8, 1.2, Hq).astype(np.float32)
    g = rng.uniform(0.0, 2.0, Hq).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    BQ = 32 * (4 // G)
    assert -(-max(lens) // BQ) * Hkv * len(lens) > 256  # paired tiles
    dev = "cuda"
    o, lse = tg.gated_attn_fwd(to_device(q), to_device(k), to_device(v), torch.from_numpy(s_c).to(dev),
                               torch.from_numpy(t).to(dev), torch.from_numpy(g).to(dev),
                               torch.from_numpy(cu).to(dev), max(lens), want_lse=True)
    torch.cuda.synchronize()
    o_r, lse_r = O.gated_attention(q.value, k.value, v.value, s_c, t, g, cu)
    assert_close(f64(o), o_r, "bf16", "attention out")
    assert_close(lse.cpu().numpy(), lse_r, "bf16", "lse")


@pytest.mark.parametrize("dtype,G,d", [("bf16", 2, 128), ("bf16", 4, 64), ("f32", 2, 64)])
def test_attention_signed_temperature_and_large_gain(dtype, G, d):
    """Negative temperatures (the sign moves into q), a zero temperature (only
    the bias is left: the scale is floored, the bias weight grows to match),
    zero, negative and large gains, against the oracle."""
    lens = [1, 200, 0, 129, 64]
    T, Hkv = sum(lens), 2
    Hq = Hkv * G
    q = activations(56, 1, (T, Hq, d), dtype)
    k = activations(56, 2, (T, Hkv, d), dtype)
    v = activations(56, 3, (T, Hkv, d), dtype)
    rng = np.random.default_rng(56)
    s_c = rng.random(T).astype(np.float32)
    t = np.array([-1.1, 0.0, 0.9, -0.3, 1.0, 0.7, -0.8, 1.2][:Hq], dtype=np.float32)
    g = np.array([0.0, 1.5, 12.0, -2.0, -1.0, 0.0, 0.5, 6.0][:Hq], dtype=np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    dev = "cuda"
    o, lse = tg.gated_attn_fwd(to_device(q), to_device(k), to_device(v), torch.from_numpy(s_c).to(dev),
                               torch.from_numpy(t).to(dev), torch.from_numpy(g).to(dev),
                               torch.from_numpy(cu).to(dev), max(lens), want_lse=True)
    torch.cuda.synchronize()
    o_r, lse_r = O.gated_attention(q.value, k.value, v.value, s_c, t, g, cu)
    assert_close(f64(o), o_r, dtype, "attention out")
    assert_close(lse.cpu().numpy(), lse_r, dtype, "lse")


def test_attention_bias_reduces_to_plain_when_gain_zero():
    """g = 0: the kernel's result must not depend on s_c at all."""
    lens = [300, 257]
    T, Hq, Hkv, d = sum(lens), 4, 2, 128
    q, k, v = (to_device(activations(52, i, (T, H, d), "bf16")) for i, H in ((1, Hq), (2, Hkv), (3, Hkv)))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    t = torch.ones(Hq, device="cuda")
    g = torch.zeros(Hq, device="cuda")
    o1, _ = tg.gated_attn_fwd(q, k, v, torch.rand(T, device="cuda"), t, g, cu, 300)
    o2, _ = tg.gated_attn_fwd(q, k, v, torch.rand(T, device="cuda"), t, g, cu, 300)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_layer_chain_against_oracle_chain(dtype):
    """Four stacked upper layers on the GPU against the oracle's own four-layer
    chain, both started from the same compacted rows, positions and scores
    (compaction is bit-exact): every kept row of the final hidden state and
    of each layer's K cache within four times the one-layer bound. Each
    layer's rounding enters the residual stream and is carried forward, so
    the bound grows with the depth; four layers' worth is the derived limit."""
    L = 4
    dims = ModelDims(D=256, Hq=4, Hkv=2, d=64, I=512, H1=64, dtype=dtype)
    w = custom(31, N=[300, 0, 1, 77, 200], K=[120, 0, 1, 30, 64], F=2, dims=dims, layers=L)
    dw = DeviceWorkload(w, n_layers=L, keep_host=True)
    gp = GatedPrefill(dw)
    gp.score()
    gp.select()
    gp.compact()
    x0 = gp.x.clone()
    for l in range(L):
        gp.layer(l)
    torch.cuda.synchronize()
    pos, sc, cu = gp.pos_c.cpu().numpy(), f64(gp.s_c), dw.host_gate.cu_kept
    x = f64(x0)
    atol, rtol = TOL[dtype]
    worst = 0.0
    for l in range(L):
        r = O.upper_layer(x, pos, sc, layer_dict(dw.host_layers[l]), dims, cu)
        got_k = f64(gp.kcache[l])
        lim = L * (atol + rtol * np.abs(r["k"]))
        assert np.all(np.abs(got_k - r["k"]) <= lim), "layer %d k cache" % l
        x = r["x2"]
    err = np.abs(f64(gp.x) - x)
    lim = L * (atol + rtol * np.abs(x))
    bad = err > lim
    assert not bad.any(), "final x: %d/%d outside %d x the one-layer bound, worst %.3g" % (
        int(bad.sum()), bad.size, L, float(err.max()))
    worst = float(err.max())
    say("  %d-layer chain (%s): final x max err %.3g (one-layer atol %g)" % (L, dtype, worst, atol))
