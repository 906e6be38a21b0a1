"""GPU parity of the three-stage prefill (Tencent Cloud TokenGate article,
early token filtering; farwalk.ai summary, the method): the layers below the
gate and the gate layer's attention on every token with plain attention, the
scorer on that post-attention residual, selection with compaction, the gate
layer's FFN and the gated layers above on the kept tokens.

Three kinds of check:
* every stage, run as its own C-ABI call, against the fp64 oracle fed the GPU's
  output of the stage before it (selection, compaction and positions bit for
  bit; the rest within atol 2e-2 / rtol 1e-2 for bf16, 1e-4 / 1e-4 for fp32);
* the one native call (tg_full_prefill) bit-identical to those staged calls;
* a budget K = N with t = 1, g = 0 above the gate equal to the same model run
  unpruned (every layer on every token).
"""
import numpy as np
import pytest
import torch

import oracle as O
from helpers import assert_close, bits, f64, layer_dict, sample_rows, say
from learned_token_pruning_post_amd import binding as tg
from learned_token_pruning_post_amd.pipeline import (DeviceWorkload, FullPrefill, UnprunedPrefill,
                                                     plain_attention_layer)
from learned_token_pruning_post_amd.workloads import ModelDims, custom, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    tg.lib()  # raises loudly if the HIP library is missing


def _staged(fp: FullPrefill):
    """Each stage of the three-stage prefill as its own C-ABI call, out of
    place, keeping every intermediate."""
    dw = fp.dw
    w = dw.w
    dm = w.dims
    dev = dw.device
    nf = dw.norms_folded
    ws = torch.empty_like(fp.ws)
    zero_s = torch.zeros(w.T_in, dtype=torch.float32, device=dev)
    st = {}
    x = dw.h.clone()
    for l, L in enumerate(fp.below):
        st["below_in%d" % l] = x
        x, k, v, _ = tg.upper_layer_fwd(plain_attention_layer(L, dm.Hq, dev), dw.dims, x, fp.pos, zero_s,
                                        dw.cu_in, w.max_n, ws=ws, rope_ready=l > 0, norms_folded=nf,
                                        input_ssq=nf and l > 0)
        st["below_k%d" % l], st["below_v%d" % l] = k, v
    st["gate_in"] = x
    nb = fp.n_below > 0
    x1, k, v, _ = tg.upper_layer_fwd(plain_attention_layer(fp.gate_layer, dm.Hq, dev), dw.dims, x, fp.pos,
                                     zero_s, dw.cu_in, w.max_n, ws=ws, rope_ready=nb, norms_folded=nf,
                                     input_ssq=nf and nb, attn_only=True)
    st.update(x1=x1, gate_k=k, gate_v=v)
    s = tg.gate_score(x1, dw.W1, dw.b1, dw.w2, dw.b2, ws=ws)
    kept, status, xc, pos_c, s_c = tg.select_compact(s, dw.keep_mask, dw.cu_in, dw.cu_kept, w.T, w.max_n,
                                                     x1, pos=fp.pos, ws=ws)
    st.update(s=s, kept=kept, status=status, xc=xc, pos_c=pos_c, s_c=s_c)
    if w.T == 0:
        torch.cuda.synchronize()
        return st
    x, _, _, _ = tg.upper_layer_fwd(fp.gate_layer, dw.dims, xc, pos_c, s_c, dw.cu_kept, w.max_k, ws=ws,
                                    norms_folded=nf, ffn_only=True)
    st["x_gate"] = x
    for l, L in enumerate(fp.above):
        st["above_in%d" % l] = x
        x, k, v, _ = tg.upper_layer_fwd(L, dw.dims, x, pos_c, s_c, dw.cu_kept, w.max_k, ws=ws,
                                        rope_ready=l > 0, norms_folded=nf, input_ssq=nf and l > 0)
        st["above_k%d" % l], st["above_v%d" % l] = k, v
    st["x"] = x
    torch.cuda.synchronize()
    return st


def _plain_dict(lw, Hq: int) -> dict:
    W = layer_dict(lw)
    W["t"], W["g"] = np.ones(Hq), np.zeros(Hq)
    return W


def _check_stages(fp: FullPrefill, st, rows_per_seq=None, seed=0):
    dw = fp.dw
    w = dw.w
    dm = w.dims
    dt = dm.dtype
    gi = dw.host_gate
    cu_in, cu_kept = gi.cu_in, gi.cu_kept
    pos = O.local_positions(cu_in)
    assert np.array_equal(fp.pos.cpu().numpy(), pos.astype(np.int32))
    rows = None if rows_per_seq is None else sample_rows(cu_in, rows_per_seq, seed)
    sel = slice(None) if rows is None else rows
    zero_s = np.zeros(w.T_in)
    errs = {}

    def layer_ref(x_in, p, s, W, cu, r):
        return O.upper_layer(f64(x_in), p, s, W, dm, cu, rows=r)

    # layers below the gate: K/V of every token, the layer's output
    for l in range(fp.n_below):
        r = layer_ref(st["below_in%d" % l], pos, zero_s, _plain_dict(dw.host_layers[l], dm.Hq), cu_in, rows)
        nxt = st["below_in%d" % (l + 1)] if l + 1 < fp.n_below else st["gate_in"]
        errs["below%d k" % l] = assert_close(f64(st["below_k%d" % l]), r["k"], dt, "below %d k" % l)
        errs["below%d v" % l] = assert_close(f64(st["below_v%d" % l]), r["v"], dt, "below %d v" % l)
        errs["below%d x" % l] = assert_close(f64(nxt)[sel], r["x2"][sel], dt, "below %d out" % l)
    # the gate layer's attention half on every token
    Wg = layer_dict(dw.host_layers[fp.n_below])
    if rows is None:
        a = O.attention_half(f64(st["gate_in"]), pos, zero_s, Wg, dm, cu_in, t=np.ones(dm.Hq),
                             g=np.zeros(dm.Hq))
    else:
        a = layer_ref(st["gate_in"], pos, zero_s, _plain_dict(dw.host_layers[fp.n_below], dm.Hq), cu_in, rows)
    errs["gate k"] = assert_close(f64(st["gate_k"]), a["k"], dt, "gate layer k")
    errs["gate v"] = assert_close(f64(st["gate_v"]), a["v"], dt, "gate layer v")
    errs["x1"] = assert_close(f64(st["x1"])[sel], a["x1"][sel], dt, "post-attention residual")
    # the scorer on that residual (every row), selection and compaction on the GPU's scores
    x1 = f64(st["x1"])
    s = st["s"].cpu().numpy()
    errs["score"] = assert_close(s, O.gate_score(x1, gi.W1.value, gi.b1.value, gi.w2.value, gi.b2.value),
                                 dt, "scores")
    ref_kept, flags = O.topk_select(s, gi.keep_mask, cu_in, cu_kept)
    assert np.array_equal(st["status"].cpu().numpy()[:w.B], flags.astype(np.int32))
    assert np.array_equal(st["kept"].cpu().numpy(), ref_kept.astype(np.int32))
    xc_r, pc_r, sc_r = O.compact(bits(st["x1"]), pos, s, ref_kept, cu_in, cu_kept)
    assert np.array_equal(bits(st["xc"]), np.ascontiguousarray(xc_r))
    assert np.array_equal(st["pos_c"].cpu().numpy(), pc_r.astype(np.int32))
    assert np.array_equal(st["s_c"].cpu().numpy().view(np.int32), sc_r.astype(np.float32).view(np.int32))
    if w.T == 0:
        say("  three-stage stage errors", {k: "%.3g" % v for k, v in errs.items()})
        return
    # the gate layer's FFN half on the kept rows, then the gated layers above
    krows = None if rows_per_seq is None else sample_rows(cu_kept, rows_per_seq, seed + 1)
    ksel = slice(None) if krows is None else krows
    xc = f64(st["xc"])
    errs["ffn"] = assert_close(f64(st["x_gate"])[ksel], O.ffn_half(xc[ksel], Wg, dm), dt, "gate layer FFN")
    pos_c = st["pos_c"].cpu().numpy()
    s_c = st["s_c"].cpu().numpy().astype(np.float64)
    for l in range(len(fp.above)):
        W = layer_dict(dw.host_layers[fp.n_below + 1 + l])
        r = layer_ref(st["above_in%d" % l], pos_c, s_c, W, cu_kept, krows)
        nxt = st["above_in%d" % (l + 1)] if l + 1 < len(fp.above) else st["x"]
        errs["above%d k" % l] = assert_close(f64(st["above_k%d" % l]), r["k"], dt, "above %d k" % l)
        errs["above%d x" % l] = assert_close(f64(nxt)[ksel], r["x2"][ksel], dt, "above %d out" % l)
    say("  three-stage stage errors", {k: "%.3g" % v for k, v in errs.items()})


def _small(dtype: str, folded: bool, n_below: int, N=(500, 0, 1, 260), K=(150, 0, 1, 77), layers=4):
    dims = ModelDims(D=256, Hq=4, Hkv=2, d=64, I=512, H1=64, dtype=dtype)
    w = custom(95 + n_below, N=list(N), K=list(K), F=8, dims=dims, layers=layers)
    dw = DeviceWorkload(w, keep_host=True, norms_folded=folded)
    return FullPrefill(dw, n_below=n_below)


SMALL_CASES = [("bf16", False, 1), ("bf16", True, 1), ("bf16", True, 2), ("bf16", True, 0),
               ("f32", False, 1)]


@pytest.mark.parametrize("dtype,folded,n_below", SMALL_CASES)
def test_full_prefill_stages_against_oracle(dtype, folded, n_below):
    fp = _small(dtype, folded, n_below)
    say("three-stage prefill", dtype, "folded" if folded else "plain norms", "gate at layer", n_below,
        "N", fp.dw.w.N, "K", fp.dw.w.K)
    _check_stages(fp, _staged(fp))


def _assert_one_call_equals_staged(fp: FullPrefill, st, what):
    fp.x.zero_()
    fp.kept.fill_(-5)
    fp.run()
    torch.cuda.synchronize()
    w = fp.dw.w
    assert torch.equal(fp.s, st["s"]), what
    assert torch.equal(fp.status[:w.B], st["status"][:w.B]), what
    assert torch.equal(fp.kept, st["kept"]), what
    assert torch.equal(fp.x_full, st["x1"]), what
    assert torch.equal(fp.pos_c, st["pos_c"]) and torch.equal(fp.s_c, st["s_c"]), what
    for l in range(fp.n_below):
        assert torch.equal(fp.kcache_full[l], st["below_k%d" % l]), what
        assert torch.equal(fp.vcache_full[l], st["below_v%d" % l]), what
    assert torch.equal(fp.kcache_full[fp.n_below], st["gate_k"]), what
    assert torch.equal(fp.vcache_full[fp.n_below], st["gate_v"]), what
    if w.T == 0:
        return
    for l in range(len(fp.above)):
        assert torch.equal(fp.kcache[l], st["above_k%d" % l]), what
        assert torch.equal(fp.vcache[l], st["above_v%d" % l]), what
    assert torch.equal(fp.x, st["x"]), what


@pytest.mark.parametrize("dtype,folded,n_below", SMALL_CASES)
def test_full_prefill_one_call_equals_staged_calls(dtype, folded, n_below):
    """tg_full_prefill (layers in place, one call) gives the staged calls'
    scores, selection, residual, compacted positions and scores, every K/V
    cache and the final rows, bit for bit; twice in a row."""
    fp = _small(dtype, folded, n_below)
    st = _staged(fp)
    _assert_one_call_equals_staged(fp, st, "first call")
    _assert_one_call_equals_staged(fp, st, "second call")


def test_full_prefill_nothing_kept():
    """K = 0 for every sequence: scores, status and the full-prompt K/V are
    still produced, nothing runs on kept rows."""
    fp = _small("bf16", True, 1, N=(300, 45), K=(0, 0), layers=3)
    fp.dw.keep_mask.zero_()
    fp.dw.host_gate.keep_mask[:] = 0
    st = _staged(fp)
    _check_stages(fp, st)
    _assert_one_call_equals_staged(fp, st, "K = 0")


@pytest.mark.parametrize("folded", [False, True])
def test_full_prefill_keep_all_equals_unpruned_model(folded):
    """K = N with t = 1 and g = 0 above the gate: the three-stage prefill is
    the model run unpruned (every layer on every token, plain attention).
    With the norms in their own kernels the two agree bit for bit; with the
    norms folded the gate layer's FFN half sums its input's squares in a
    kernel of its own where the whole layer does it in the O projection, so
    they agree within the bf16 tolerance."""
    dims = ModelDims(D=256, Hq=4, Hkv=2, d=64, I=512, H1=64, dtype="bf16")
    w = custom(96, N=[300, 129], K=[300, 129], F=4, dims=dims, layers=4)
    dw = DeviceWorkload(w, norms_folded=folded)
    for L in dw.layers:
        L.tensors["t"].fill_(1.0)
        L.tensors["g"].zero_()
    fp = FullPrefill(dw, n_below=1)
    x = fp.run().clone()
    torch.cuda.synchronize()
    assert fp.kept.cpu().numpy().tolist() == list(range(w.T_in))
    xu = UnprunedPrefill(dw).run()
    torch.cuda.synchronize()
    if folded:
        e = assert_close(f64(x), f64(xu), "bf16", "pruned K = N vs unpruned")
        say("  K = N vs unpruned, folded norms: max err", e)
    else:
        assert torch.equal(x, xu)


def test_full_prefill_qwen8k_sampled_rows():
    """Qwen3-1.7B shapes, N = 8192, K = 1024, the gate at layer 1 with two
    layers above, folded norms (the benchmark's launch configuration): every
    stage against the oracle, on sampled rows where the oracle is slow; the
    one native call bit-identical to the staged calls."""
    w = workload("qwen8k", layers=4)
    dw = DeviceWorkload(w, keep_host=True, norms_folded=True)
    fp = FullPrefill(dw, n_below=1)
    say("three-stage prefill qwen8k, folded norms")
    st = _staged(fp)
    _check_stages(fp, st, rows_per_seq=64)
    _assert_one_call_equals_staged(fp, st, "qwen8k")
