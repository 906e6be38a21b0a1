"""GPU parity of the backward pass of the gate's gradient path (Tencent Cloud
TokenGate article, gradient-path section): the gated attention's gradients
(tg_gated_attn_bwd: dq, dk, dv, the kept tokens' ds, dt, dg) and the scorer's
(tg_gate_score_bwd), against the fp64 oracle on the same bf16 inputs.

Gradients can be far smaller than the activations, so the bound is scaled to
each tensor: |gpu - ref| <= 2e-2 * max|ref| + 1e-2 * |ref| (the bf16
tolerance of the forward outputs, with its absolute part relative to the
tensor's own magnitude).
"""
import numpy as np
import pytest
import torch

import oracle as O
from helpers import f64, say
from learned_token_pruning_post_amd import binding as tg
from learned_token_pruning_post_amd.pipeline import to_device
from learned_token_pruning_post_amd.workloads import activations

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    tg.lib()  # raises loudly if the HIP library is missing


def assert_close_scaled(got, ref, what, frac=2e-2, rtol=1e-2):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = np.abs(got - ref)
    lim = frac * scale + rtol * np.abs(ref)
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError("%s: %d/%d outside (scale %.3g); worst at %s got %r ref %r"
                             % (what, int(bad.sum()), bad.size, scale, i, got[i], ref[i]))
    return float(err.max() / scale) if scale > 0 else 0.0


def _attn_case(seed, K, Hq, Hkv, d, t=None, g=None):
    T = int(sum(K))
    cu = np.concatenate([[0], np.cumsum(K)]).astype(np.int32)
    dev = {n: to_device(activations(seed, o, shape, "bf16"))
           for n, o, shape in (("q", 1, (T, Hq, d)), ("k", 2, (T, Hkv, d)), ("v", 3, (T, Hkv, d)),
                               ("dO", 4, (T, Hq, d)))}
    rng = np.random.default_rng(seed)
    s = rng.random(T).astype(np.float32)
    t = rng.uniform(0.8, 1.2, Hq).astype(np.float32) if t is None else np.asarray(t, dtype=np.float32)
    g = rng.uniform(0.0, 2.0, Hq).astype(np.float32) if g is None else np.asarray(g, dtype=np.float32)
    dev.update(s=torch.from_numpy(s).cuda(), t=torch.from_numpy(t).cuda(), g=torch.from_numpy(g).cuda(),
               cu=torch.from_numpy(cu).cuda())
    return dev, cu


def _attn_bwd(dev, max_k):
    o, lse = tg.gated_attn_fwd(dev["q"], dev["k"], dev["v"], dev["s"], dev["t"], dev["g"], dev["cu"], max_k,
                               want_lse=True)
    r = tg.gated_attn_bwd(dev["q"], dev["k"], dev["v"], dev["s"], dev["t"], dev["g"], dev["cu"], max_k, o, lse,
                          dev["dO"])
    torch.cuda.synchronize()
    return r


def _check_attn(seed, K, Hq, Hkv, d, t=None, g=None):
    dev, cu = _attn_case(seed, K, Hq, Hkv, d, t, g)
    max_k = int(max(K))
    r = _attn_bwd(dev, max_k)
    ref = O.gated_attention_backward(f64(dev["q"]), f64(dev["k"]), f64(dev["v"]), f64(dev["s"]),
                                     f64(dev["t"]), f64(dev["g"]), cu, f64(dev["dO"]))
    errs = {n: assert_close_scaled(r[n].cpu().numpy(), ref[n], n) for n in ("dq", "dk", "dv", "ds", "dt", "dg")}
    say("  attention backward G=%d d=%d K=%s" % (Hq // Hkv, d, list(K)[:6]),
        {n: "%.2g" % e for n, e in errs.items()})
    return dev, r


@pytest.mark.parametrize("Hq,Hkv,d", [(16, 8, 128), (4, 4, 64), (8, 2, 64), (8, 4, 64), (8, 2, 128),
                                      (4, 4, 128)])
def test_attention_backward_ragged(Hq, Hkv, d):
    # a one-token and an empty sequence, partial tiles, sequences longer than a tile pair
    _check_attn(41, [300, 1, 0, 77, 1000], Hq, Hkv, d)


def test_attention_backward_qwen_shapes_k2048():
    _check_attn(42, [2048], 16, 8, 128)


def test_attention_backward_at_the_benchmark_shape():
    """The backward leg's shape: one sequence of 4096 kept tokens, 16/8 heads x
    128, every output against the full fp64 oracle."""
    _check_attn(44, [4096], 16, 8, 128)


def test_attention_backward_signed_temperature_and_zero_gain():
    """Negative and zero temperatures and zero gains (the logit then loses its
    q.k or its bias term): dt and dg still follow the oracle."""
    t = [-1.1, 0.0, 0.9, -0.3, 1.0, 0.7, -0.8, 1.2]
    g = [0.0, 1.5, 0.0, 2.0, -1.0, 0.0, 0.5, 1.0]
    _check_attn(45, [300, 1, 0, 130], 8, 4, 64, t, g)
    _check_attn(46, [200, 65], 8, 2, 128, t, g)


def test_attention_backward_is_deterministic():
    dev, _ = _attn_case(43, [700, 129], 16, 8, 128)
    a = _attn_bwd(dev, 700)
    b = _attn_bwd(dev, 700)
    for n in a:
        assert torch.equal(a[n], b[n]), n


def _scorer_check(w, seed):
    from learned_token_pruning_post_amd.pipeline import DeviceWorkload
    dw = DeviceWorkload(w, n_layers=0, keep_host=True)
    gi = dw.host_gate
    s = tg.gate_score(dw.h, dw.W1, dw.b1, dw.w2, dw.b2)
    ds = torch.from_numpy(np.random.default_rng(seed).standard_normal(w.T_in).astype(np.float32)).cuda()
    r = tg.gate_score_bwd(dw.h, dw.W1, dw.b1, dw.w2, s, ds)
    torch.cuda.synchronize()
    ref = O.gate_score_backward(gi.h.value, gi.W1.value, gi.b1.value, gi.w2.value, gi.b2.value, f64(ds))
    errs = {n: assert_close_scaled(f64(r[n]) if n != "db2" else float(r[n].item()), ref[n], n)
            for n in ("dh", "dW1", "db1", "dw2", "db2")}
    say("  scorer backward", w.name, "T_in", w.T_in, {n: "%.2g" % e for n, e in errs.items()})


def test_scorer_backward_small_ragged():
    from learned_token_pruning_post_amd.workloads import ModelDims, custom
    dims = ModelDims(D=256, Hq=4, Hkv=2, d=64, I=512, H1=64, dtype="bf16")
    _scorer_check(custom(51, N=[700, 77], K=[10, 10], F=1, dims=dims), 51)


def test_scorer_backward_qwen8k():
    from learned_token_pruning_post_amd.workloads import workload
    _scorer_check(workload("qwen8k"), 52)


def test_scorer_backward_at_the_benchmark_shape():
    """The backward leg's scorer: 32768 prompt tokens, 2048 -> 256."""
    from learned_token_pruning_post_amd.workloads import workload
    _scorer_check(workload("qwen32k"), 54)


def test_gradient_path_scorer_select_attention():
    """Scores -> selection and compaction -> gated attention on the kept
    tokens -> its backward -> the prompt scores' gradient through the
    compaction -> the scorer's backward, each stage against the oracle fed
    the GPU's previous stage; the scatter through the compaction bit-exact."""
    from learned_token_pruning_post_amd.pipeline import DeviceWorkload
    from learned_token_pruning_post_amd.workloads import ModelDims, custom
    dims = ModelDims(D=256, Hq=4, Hkv=2, d=64, I=512, H1=64, dtype="bf16")
    w = custom(53, N=[700, 0, 300], K=[200, 0, 77], F=4, dims=dims)
    dw = DeviceWorkload(w, n_layers=0, keep_host=True)
    gi = dw.host_gate
    s = tg.gate_score(dw.h, dw.W1, dw.b1, dw.w2, dw.b2)
    kept, status, _, _, s_c = tg.select_compact(s, dw.keep_mask, dw.cu_in, dw.cu_kept, w.T, w.max_n, dw.h)
    T, dm = w.T, w.dims
    dev = {n: to_device(activations(53, o, shape, "bf16"))
           for n, o, shape in (("q", 1, (T, dm.Hq, dm.d)), ("k", 2, (T, dm.Hkv, dm.d)),
                               ("v", 3, (T, dm.Hkv, dm.d)), ("dO", 4, (T, dm.Hq, dm.d)))}
    rng = np.random.default_rng(53)
    t = torch.from_numpy(rng.uniform(0.8, 1.2, dm.Hq).astype(np.float32)).cuda()
    g = torch.from_numpy(rng.uniform(0.0, 2.0, dm.Hq).astype(np.float32)).cuda()
    o, lse = tg.gated_attn_fwd(dev["q"], dev["k"], dev["v"], s_c, t, g, dw.cu_kept, w.max_k, want_lse=True)
    ra = tg.gated_attn_bwd(dev["q"], dev["k"], dev["v"], s_c, t, g, dw.cu_kept, w.max_k, o, lse, dev["dO"])
    ds = tg.compact_scores_bwd(ra["ds"], kept, w.T_in)
    rs = tg.gate_score_bwd(dw.h, dw.W1, dw.b1, dw.w2, s, ds)
    torch.cuda.synchronize()
    assert not status.any().item()
    ref_a = O.gated_attention_backward(f64(dev["q"]), f64(dev["k"]), f64(dev["v"]), f64(s_c), f64(t), f64(g),
                                       gi.cu_kept, f64(dev["dO"]))
    assert_close_scaled(ra["ds"].cpu().numpy(), ref_a["ds"], "ds of the kept tokens")
    kept_h = kept.cpu().numpy()
    assert np.array_equal(ds.cpu().numpy(), O.compact_backward(f64(ra["ds"]), kept_h, w.T_in).astype(np.float32))
    ref_s = O.gate_score_backward(gi.h.value, gi.W1.value, gi.b1.value, gi.w2.value, gi.b2.value, f64(ds))
    for n in ("dh", "dW1", "db1", "dw2"):
        assert_close_scaled(f64(rs[n]), ref_s[n], n)
    pruned = np.setdiff1d(np.arange(w.T_in), kept_h)
    assert np.all(ds.cpu().numpy()[pruned] == 0)
