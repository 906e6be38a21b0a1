"""GPU parity of decode attention over the pruned cache (tg_decode_attn_fwd)
against the fp64 oracle (Tencent Cloud TokenGate article, engineering section:
decoding folds the gate bias fixed at prefill into the mask and runs ordinary
attention over the cache; early token filtering: generated tokens are never
gated out). Outputs within atol 2e-2 / rtol 1e-2 (bf16) or 1e-4 (fp32), the
log-sum-exp within the same bounds; bad lengths flagged and NaN; the decode
of a prefill's last kept token equal to that token's row of the prefill
attention.
"""
import numpy as np
import pytest
import torch

import oracle as O
from helpers import assert_close, f64, say, ws_view
from learned_token_pruning_post_amd import binding as tg
from learned_token_pruning_post_amd.pipeline import DeviceWorkload, GatedPrefill, to_device
from learned_token_pruning_post_amd.workloads import ModelDims, activations, custom

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    tg.lib()  # raises loudly if the HIP library is missing


def _case(seed, dtype, lenA, lenB, capB, Hq, Hkv, d):
    """Seeded cache and queries: segment A packed by lenA, segment B [B, capB]."""
    B = len(lenA)
    rng = np.random.default_rng(seed)
    rows = int(sum(lenA))
    ta = lambda o, shape: activations(seed, o, shape, dtype)
    h = {"q": ta(1, (B, Hq, d)), "kA": ta(2, (max(rows, 1), Hkv, d)), "vA": ta(3, (max(rows, 1), Hkv, d)),
         "kB": ta(4, (B, max(capB, 1), Hkv, d)), "vB": ta(5, (B, max(capB, 1), Hkv, d))}
    sA = rng.random(max(rows, 1)).astype(np.float32)
    sB = rng.random((B, max(capB, 1))).astype(np.float32)
    t = rng.uniform(0.8, 1.2, Hq).astype(np.float32)
    g = rng.uniform(0.0, 2.0, Hq).astype(np.float32)
    cuA = np.concatenate([[0], np.cumsum(lenA)]).astype(np.int32)
    dev = {k: to_device(v) for k, v in h.items()}
    dev.update(sA=torch.from_numpy(sA).cuda(), sB=torch.from_numpy(sB).cuda(), t=torch.from_numpy(t).cuda(),
               g=torch.from_numpy(g).cuda(), cuA=torch.from_numpy(cuA).cuda(),
               lenB=torch.from_numpy(np.asarray(lenB, np.int32)).cuda())
    host = {k: v.value for k, v in h.items()}
    host.update(sA=sA, sB=sB, t=t, g=g, cuA=cuA, lenB=np.asarray(lenB))
    return dev, host


def _run(dev, capB, max_len):
    return tg.decode_attn_fwd(dev["q"], dev["kA"], dev["vA"], dev["sA"], dev["cuA"],
                              dev["kB"] if capB else None, dev["vB"] if capB else None,
                              dev["sB"] if capB else None, dev["lenB"], dev["t"], dev["g"], max_len,
                              want_lse=True)


def _oracle(host):
    return O.decode_attention(host["q"], host["kA"], host["vA"], host["sA"], host["cuA"], host["kB"],
                              host["vB"], host["sB"], host["lenB"], host["t"], host["g"])


def _check(dtype, lenA, lenB, capB, Hq, Hkv, d, seed=0):
    dev, host = _case(seed, dtype, lenA, lenB, capB, Hq, Hkv, d)
    max_len = int(max(a + b for a, b in zip(lenA, lenB)))
    o, lse, status = _run(dev, capB, max_len)
    torch.cuda.synchronize()
    o_r, lse_r = _oracle(host)
    assert not status.cpu().numpy()[:len(lenA)].any()
    e = assert_close(f64(o), o_r, dtype, "decode output")
    lse_g = lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(lse_r)
    assert np.array_equal(np.isneginf(lse_g), empty)
    el = assert_close(lse_g[~empty], lse_r[~empty], dtype, "decode lse")
    say("  decode", dtype, "G", Hq // Hkv, "d", d, "lens", list(zip(lenA, lenB))[:6],
        "max err o %.3g lse %.3g" % (e, el))


@pytest.mark.parametrize("dtype,Hq,Hkv,d", [("bf16", 16, 8, 128), ("bf16", 4, 1, 64), ("bf16", 8, 1, 128),
                                           ("bf16", 8, 8, 64), ("f32", 16, 8, 128), ("f32", 4, 4, 64),
                                           ("f32", 8, 2, 64)])
def test_decode_matches_oracle_ragged(dtype, Hq, Hkv, d):
    # empty sequence, prompt only, generated only, both, and a chunk-straddling split
    _check(dtype, [0, 1, 300, 2500, 77, 0], [1, 0, 5, 64, 0, 0], 64, Hq, Hkv, d)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_single_chunk_path(dtype):
    # every sequence fits one key chunk: the first kernel writes the output itself
    assert tg.lib().tg_decode_attn_workspace_size(3, 100, 16, 8, 128, tg.dtype_code(
        torch.bfloat16 if dtype == "bf16" else torch.float32)) == 0
    _check(dtype, [37, 100, 0], [3, 0, 1], 4, 16, 8, 128, seed=1)


def test_decode_long_cache():
    _check("bf16", [131072 - 7], [7], 16, 16, 8, 128, seed=2)


def test_decode_at_the_benchmark_shape():
    """The decode leg's call: 16 sequences of 4096 kept prompt tokens plus 128
    generated ones (segment B at capacity), 16/8 heads x 128."""
    _check("bf16", [4096] * 16, [128] * 16, 128, 16, 8, 128, seed=5)


def test_decode_many_sequences():
    rng = np.random.default_rng(3)
    B = 96
    lenA = rng.integers(0, 700, B).tolist()
    lenB = rng.integers(0, 33, B).tolist()
    _check("bf16", lenA, lenB, 32, 16, 8, 128, seed=3)


@pytest.mark.parametrize("scale", [1, 100])
def test_decode_bad_lengths_are_flagged(scale):
    # scale 1: one key chunk per sequence (the first kernel writes the outputs);
    # scale 100: split over chunks (the merge kernel writes them)
    lenA = [10 * scale, 20 * scale, 30 * scale, 40 * scale]
    max_len = 40 * scale
    dev, host = _case(4, "bf16", lenA, [2, 9, 0, 3], 8, 16, 8, 128)
    # lenB[1] = 9 > capB = 8; sequence 3 has max_len + 3 keys
    o, lse, status = _run(dev, 8, max_len)
    torch.cuda.synchronize()
    need = tg.lib().tg_decode_attn_workspace_size(4, max_len, 16, 8, 128, 1)
    assert (need == 0) == (scale == 1)
    st = status.cpu().numpy()
    assert st.tolist() == [0, 8, 0, 8]
    of = o.float().cpu().numpy()
    assert np.isnan(of[[1, 3]]).all() and np.isnan(lse.cpu().numpy()[[1, 3]]).all()
    host["lenB"] = np.array([2, 0, 0, 0])
    o_r, _ = _oracle(host)
    for b in (0, 2):
        assert_close(of[b], o_r[b], "bf16", "decode beside flagged sequences")


def test_decode_of_the_last_kept_token_is_its_prefill_row():
    """After a gated prefill, the decode attention of each sequence's last kept
    token over that layer's kept-token cache (segment A = the prefill's
    kcache, vcache, s_c and cu_kept, nothing generated) equals that token's
    row of the prefill's gated attention; and a decode step with generated
    tokens matches the oracle on the same cache."""
    dims = ModelDims(D=256, Hq=4, Hkv=2, d=64, I=512, H1=64, dtype="bf16")
    w = custom(71, N=[700, 1, 260, 0], K=[300, 1, 77, 0], F=4, dims=dims)
    dw = DeviceWorkload(w, keep_host=True)
    gp = GatedPrefill(dw)
    gp.score()
    gp.select_compact()
    gp.layer(0)
    torch.cuda.synchronize()
    dm = w.dims
    lay = tg.upper_layer_ws_layout(dw.dims, w.T)
    q = ws_view(gp.ws, lay.q, (w.T, dm.Hq, dm.d), gp.x.dtype)
    attn = ws_view(gp.ws, lay.attn, (w.T, dm.Hq, dm.d), gp.x.dtype)
    cu = dw.cu_kept.cpu().numpy()
    has = np.diff(cu) > 0
    last = torch.from_numpy((cu[1:] - 1)[has].astype(np.int64)).cuda()
    cuA = torch.from_numpy(np.concatenate([[0], np.cumsum(np.diff(cu)[has])]).astype(np.int32)).cuda()
    # segment A: the sequences with kept tokens, their cache rows as the prefill wrote them
    starts = cu[:-1][has]
    assert np.array_equal(starts, cuA.cpu().numpy()[:-1])
    L0 = dw.layers[0].tensors
    nb = int(has.sum())
    lenB = torch.zeros(nb, dtype=torch.int32, device="cuda")
    o, lse, st = tg.decode_attn_fwd(q[last].contiguous(), gp.kcache[0], gp.vcache[0], gp.s_c, cuA, None, None,
                                    None, lenB, L0["t"], L0["g"], int(np.diff(cu).max()), want_lse=True)
    torch.cuda.synchronize()
    assert not st.cpu().numpy()[:nb].any()
    assert_close(f64(o), f64(attn[last]), "bf16", "decode of the last kept token vs its prefill row")
    # a decode step: a new token per sequence, three generated tokens already cached
    capB = 4
    gen = {"kB": to_device(activations(72, 1, (nb, capB, dm.Hkv, dm.d), "bf16")),
           "vB": to_device(activations(72, 2, (nb, capB, dm.Hkv, dm.d), "bf16")),
           "q": to_device(activations(72, 3, (nb, dm.Hq, dm.d), "bf16"))}
    sB = torch.rand((nb, capB), generator=torch.Generator().manual_seed(72)).cuda()
    lenB = torch.tensor([3] * nb, dtype=torch.int32, device="cuda")
    o, _, _ = tg.decode_attn_fwd(gen["q"], gp.kcache[0], gp.vcache[0], gp.s_c, cuA, gen["kB"], gen["vB"], sB,
                                 lenB, L0["t"], L0["g"], int(np.diff(cu).max()) + 3)
    torch.cuda.synchronize()
    o_r, _ = O.decode_attention(f64(gen["q"]), f64(gp.kcache[0]), f64(gp.vcache[0]), f64(gp.s_c),
                                cuA.cpu().numpy(), f64(gen["kB"]), f64(gen["vB"]), f64(sB), [3] * nb,
                                L0["t"].cpu().numpy(), L0["g"].cpu().numpy())
    assert_close(f64(o), o_r, "bf16", "decode over a prefill's cache")
