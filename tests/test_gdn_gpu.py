"""GPU parity of the Gated DeltaNet mixer of the hybrid variant (tg_gdn_fwd)
against the fp64 oracle (Tencent Cloud TokenGate article, section on the gate
position: a GDN layer above the gate has no logits to bias and runs on the
kept tokens). Outputs within atol 2e-2 / rtol 1e-2 (bf16) or 1e-4 (fp32);
the fp32 state within 1e-4 / 1e-4 for fp32 inputs and the bf16 bound for bf16.
bf16 runs the chunked form (64-token chunks, matrix cores), fp32 the token
recurrence: the cases cover partial chunks, empty and one-token sequences,
dv not a multiple of dk, a decay of exactly 0 and a carried state.
"""
import numpy as np
import pytest
import torch

import oracle as O
from helpers import assert_close, f64, say
from learned_token_pruning_post_amd import binding as tg
from learned_token_pruning_post_amd.pipeline import to_device
from learned_token_pruning_post_amd.workloads import activations

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    tg.lib()  # raises loudly if the HIP library is missing


def _case(seed, lens, H, dk, dv, dtype):
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    dev = {n: to_device(activations(seed, o, shape, dtype))
           for n, o, shape in (("q", 1, (T, H, dk)), ("k", 2, (T, H, dk)), ("v", 3, (T, H, dv)))}
    rng = np.random.default_rng(seed)
    al = rng.uniform(0.8, 1.0, (T, H)).astype(np.float32)
    be = rng.uniform(0.0, 1.0, (T, H)).astype(np.float32)
    dev.update(alpha=torch.from_numpy(al).cuda(), beta=torch.from_numpy(be).cuda(), cu=torch.from_numpy(cu).cuda())
    return dev, cu


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("bf16", 64, 64), ("bf16", 128, 64),
                                         ("bf16", 128, 96), ("bf16", 64, 160),
                                         ("f32", 128, 128), ("f32", 64, 96)])
def test_gdn_matches_oracle_ragged(dtype, dk, dv):
    lens = [300, 0, 1, 77, 1000]
    dev, cu = _case(71, lens, 4, dk, dv, dtype)
    o, st = tg.gdn_fwd(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["cu"], want_state=True)
    torch.cuda.synchronize()
    o_r, st_r = O.gdn_mixer(f64(dev["q"]), f64(dev["k"]), f64(dev["v"]), f64(dev["alpha"]), f64(dev["beta"]), cu)
    e = assert_close(f64(o), o_r, dtype, "gdn output")
    es = assert_close(st.cpu().numpy(), st_r, dtype, "gdn state")
    say("  gdn", dtype, "dk", dk, "dv", dv, "max err o %.3g state %.3g" % (e, es))


@pytest.mark.parametrize("dtype,cut", [("bf16", (384, 64)), ("f32", (400, 100))])
def test_gdn_state_carries_across_calls(dtype, cut):
    """Two sequences split over two calls with the state carried: the same bits
    as one call (bf16 splits at multiples of the 64-token chunk, so the chunks
    are the same; the fp32 recurrence splits anywhere)."""
    lens = [700, 129]
    dev, cu = _case(72, lens, 4, 128, 128, dtype)
    o, st = tg.gdn_fwd(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["cu"], want_state=True)
    a, b = cut
    idx1 = np.r_[0:a, 700:700 + b]
    idx2 = np.r_[a:700, 700 + b:829]
    pick = lambda t, idx: t[torch.from_numpy(idx).cuda()].contiguous()
    o1, s1 = tg.gdn_fwd(*(pick(dev[n], idx1) for n in ("q", "k", "v", "alpha", "beta")),
                        torch.tensor([0, a, a + b], dtype=torch.int32, device="cuda"), want_state=True)
    o2, s2 = tg.gdn_fwd(*(pick(dev[n], idx2) for n in ("q", "k", "v", "alpha", "beta")),
                        torch.tensor([0, 700 - a, 829 - a - b], dtype=torch.int32, device="cuda"), state_in=s1,
                        want_state=True)
    torch.cuda.synchronize()
    whole = torch.empty_like(o)
    whole[torch.from_numpy(idx1).cuda()] = o1
    whole[torch.from_numpy(idx2).cuda()] = o2
    assert torch.equal(whole, o) and torch.equal(s2, st)


def test_gdn_zero_decay_and_carried_state():
    """A decay of exactly 0 (the state resets inside a chunk) and a given start
    state, against the oracle."""
    lens = [150, 64, 3]
    dev, cu = _case(74, lens, 4, 128, 128, "bf16")
    al = dev["alpha"].clone()
    al[10, 0] = 0.0
    al[63, 1] = 0.0
    al[64, 2] = 0.0
    al[151, 3] = 0.0
    rng = np.random.default_rng(74)
    st0 = torch.from_numpy((0.3 * rng.standard_normal((3, 4, 128, 128))).astype(np.float32)).cuda()
    o, st = tg.gdn_fwd(dev["q"], dev["k"], dev["v"], al, dev["beta"], dev["cu"], state_in=st0, want_state=True)
    torch.cuda.synchronize()
    o_r, st_r = O.gdn_mixer(f64(dev["q"]), f64(dev["k"]), f64(dev["v"]), f64(al), f64(dev["beta"]), cu,
                            state_in=f64(st0))
    e = assert_close(f64(o), o_r, "bf16", "gdn output")
    es = assert_close(st.cpu().numpy(), st_r, "bf16", "gdn state")
    say("  gdn zero decay + state: max err o %.3g state %.3g" % (e, es))


def test_gdn_long_sequence():
    """One 2048-token sequence (32 chunks: the state crosses many chunk
    boundaries), two heads, against the oracle."""
    dev, cu = _case(75, [2048], 2, 128, 128, "bf16")
    o, st = tg.gdn_fwd(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["cu"], want_state=True)
    torch.cuda.synchronize()
    o_r, st_r = O.gdn_mixer(f64(dev["q"]), f64(dev["k"]), f64(dev["v"]), f64(dev["alpha"]), f64(dev["beta"]), cu)
    e = assert_close(f64(o), o_r, "bf16", "gdn output")
    es = assert_close(st.cpu().numpy(), st_r, "bf16", "gdn state")
    say("  gdn 2048 tokens: max err o %.3g state %.3g" % (e, es))


def test_gdn_at_the_benchmark_shape():
    """The GDN leg's shape and call: one sequence of 4096 kept tokens, 16 heads,
    dk = dv = 128, bf16, with a workspace sized by its query; every output and
    the final state against the oracle."""
    dev, cu = _case(77, [4096], 16, 128, 128, "bf16")
    need = tg.lib().tg_gdn_workspace_size(4096, 1, 16, 128, 128, tg.dtype_code(torch.bfloat16))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o, st = tg.gdn_fwd(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["cu"], want_state=True, ws=ws)
    torch.cuda.synchronize()
    o_r, st_r = O.gdn_mixer(f64(dev["q"]), f64(dev["k"]), f64(dev["v"]), f64(dev["alpha"]), f64(dev["beta"]), cu)
    e = assert_close(f64(o), o_r, "bf16", "gdn output")
    es = assert_close(st.cpu().numpy(), st_r, "bf16", "gdn state")
    say("  gdn 4096 tokens x 16 heads: max err o %.3g state %.3g" % (e, es))


def test_gdn_no_tokens():
    """Every sequence empty (T = 0): the state passes through unchanged."""
    rng = np.random.default_rng(76)
    st0 = torch.from_numpy(rng.standard_normal((2, 4, 128, 128)).astype(np.float32)).cuda()
    e = torch.empty((0, 4, 128), dtype=torch.bfloat16, device="cuda")
    z = torch.empty((0, 4), dtype=torch.float32, device="cuda")
    cu = torch.zeros(3, dtype=torch.int32, device="cuda")
    o, st = tg.gdn_fwd(e, e, e, z, z, cu, state_in=st0, want_state=True)
    torch.cuda.synchronize()
    assert o.shape == (0, 4, 128) and torch.equal(st, st0)


def test_gdn_on_the_kept_tokens():
    """The hybrid flow: prompt-level q, k, v, alpha, beta rows gathered to the
    kept tokens by the library's compaction, then the GDN mixer over the kept
    sequences; equal to the oracle's mixer over the kept rows in order."""
    N, K, H, dk, dv = [900, 300], [200, 77], 4, 128, 128
    T_in, T = sum(N), sum(K)
    dev, _ = _case(73, N, H, dk, dv, "bf16")
    rng = np.random.default_rng(73)
    s = torch.from_numpy(rng.random(T_in).astype(np.float32)).cuda()
    cu_in = torch.tensor([0, N[0], T_in], dtype=torch.int32, device="cuda")
    cu_k = torch.tensor([0, K[0], T], dtype=torch.int32, device="cuda")
    kept, status = tg.topk_select(s, None, cu_in, cu_k, T, max(N))
    rows = {}
    for n in ("q", "k", "v", "alpha", "beta"):
        src = dev[n].reshape(T_in, -1)
        rows[n], _, _ = tg.compact(src, None, s, kept, cu_in, cu_k)
    o, _ = tg.gdn_fwd(rows["q"].view(T, H, dk), rows["k"].view(T, H, dk), rows["v"].view(T, H, dv),
                      rows["alpha"].view(T, H), rows["beta"].view(T, H), cu_k)
    torch.cuda.synchronize()
    assert not status.any().item()
    kh = kept.cpu().numpy().astype(np.int64)
    o_r, _ = O.gdn_mixer(f64(dev["q"])[kh], f64(dev["k"])[kh], f64(dev["v"])[kh], f64(dev["alpha"])[kh],
                         f64(dev["beta"])[kh], np.array([0, K[0], T]))
    assert_close(f64(o), o_r, "bf16", "gdn on the kept tokens")
