"""Guard bands around every output and workspace of the C ABI.

Each output tensor and each workspace (sized exactly as the library's
workspace query says) sits between two 4 KiB bands of a sentinel byte; after
ragged batches with empty and one-token sequences, a batch with nothing kept
and an fp32 batch, every band must still hold the sentinel (no write past an
output's end or before its start, no workspace use beyond what the query
reported), and the guarded outputs must equal those of the same calls on
ordinary tensors, bit for bit.
"""
import ctypes

import numpy as np
import pytest
import torch

from helpers import say
from learned_token_pruning_post_amd import binding as tg
from learned_token_pruning_post_amd.pipeline import DeviceWorkload, FullPrefill, GatedPrefill, to_device
from learned_token_pruning_post_amd.workloads import ModelDims, activations, custom

pytestmark = pytest.mark.gpu

GUARD = 4096
SENTINEL = 0xA5


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    tg.lib()  # raises loudly if the HIP library is missing


class Guarded:
    """A tensor of `shape` placed between two guard bands of SENTINEL bytes."""

    def __init__(self, name, shape, dtype):
        self.name = name
        esz = torch.empty(0, dtype=dtype).element_size()
        self.nbytes = int(np.prod(shape)) * esz
        self.raw = torch.full((2 * GUARD + self.nbytes,), SENTINEL, dtype=torch.uint8, device="cuda")
        self.t = self.raw[GUARD:GUARD + self.nbytes].view(dtype).view(shape)

    def check(self):
        lo = self.raw[:GUARD].cpu().numpy()
        hi = self.raw[GUARD + self.nbytes:].cpu().numpy()
        bad_lo = np.flatnonzero(lo != SENTINEL)
        bad_hi = np.flatnonzero(hi != SENTINEL)
        assert bad_lo.size == 0, "%s: %d bytes written before the start (first at -%d)" % (
            self.name, bad_lo.size, GUARD - bad_lo[-1])
        assert bad_hi.size == 0, "%s: %d bytes written past the end (first at +%d)" % (
            self.name, bad_hi.size, bad_hi[0])


def _ws(name, nbytes):
    return Guarded(name, (max(int(nbytes), 0),), torch.uint8)


def _check_all(*gs):
    torch.cuda.synchronize()
    for g in gs:
        g.check()


def _dims(dtype):
    return ModelDims(D=256, Hq=4, Hkv=2, d=64, I=512, H1=64, dtype=dtype)


CASES = [
    # (dtype, N, K, forced per sequence)
    ("bf16", [300, 0, 1, 77, 1000], [150, 0, 1, 77, 333], 8),
    ("f32", [129, 64, 0, 300], [65, 64, 0, 17], 4),
    ("bf16", [200, 45], [0, 0], 0),  # nothing kept
]


@pytest.mark.parametrize("dtype,N,K,F", CASES)
def test_stage_outputs_stay_inside_their_buffers(dtype, N, K, F):
    say("canaries, per stage:", dtype, "N", N, "K", K)
    w = custom(61, N=N, K=K, F=F, dims=_dims(dtype), layers=2)
    dw = DeviceWorkload(w, norms_folded=dtype == "bf16")
    gp = GatedPrefill(dw)
    gp.run()  # ordinary tensors: the reference outputs
    torch.cuda.synchronize()
    lib = tg.lib()
    dt = dw.h.dtype
    T, T_in, B, D = w.T, w.T_in, w.B, w.dims.D
    code = tg.dtype_code(dt)

    # scorer
    s = Guarded("s", (T_in,), torch.float32)
    ws = _ws("scorer ws", lib.tg_gate_score_workspace_size(T_in, D, w.dims.H1, code))
    tg.gate_score(dw.h, dw.W1, dw.b1, dw.w2, dw.b2, s_out=s.t, ws=ws.t)
    _check_all(s, ws)
    assert torch.equal(s.t, gp.s)

    # selection alone, then compaction alone, then both in one pass
    need = lib.tg_topk_select_workspace_size(B, T_in, w.max_n)
    kept, status = Guarded("kept", (T,), torch.int32), Guarded("status", (B,), torch.int32)
    sws = _ws("select ws", need)
    tg.topk_select(gp.s, dw.keep_mask, dw.cu_in, dw.cu_kept, T, w.max_n, kept=kept.t, status=status.t,
                   ws=sws.t)
    _check_all(kept, status, sws)
    assert torch.equal(kept.t, gp.kept) and torch.equal(status.t, gp.status)
    hc, pc = Guarded("h_out", (T, D), dt), Guarded("pos_out", (T,), torch.int32)
    sc = Guarded("s_out", (T,), torch.float32)
    tg.compact(dw.h, None, gp.s, gp.kept, dw.cu_in, dw.cu_kept, h_out=hc.t, pos_out=pc.t, s_out=sc.t)
    _check_all(hc, pc, sc)
    kept2, status2 = Guarded("kept", (T,), torch.int32), Guarded("status", (B,), torch.int32)
    sws2 = _ws("ws", need)
    hc2, pc2 = Guarded("h_out", (T, D), dt), Guarded("pos_out", (T,), torch.int32)
    sc2 = Guarded("s_out", (T,), torch.float32)
    tg.select_compact(gp.s, dw.keep_mask, dw.cu_in, dw.cu_kept, T, w.max_n, dw.h, kept=kept2.t,
                      status=status2.t, h_out=hc2.t, pos_out=pc2.t, s_out=sc2.t, ws=sws2.t)
    _check_all(kept2, status2, sws2, hc2, pc2, sc2)
    assert torch.equal(kept2.t, gp.kept) and torch.equal(hc2.t, hc.t)
    assert torch.equal(pc2.t, pc.t) and torch.equal(sc2.t, sc.t)
    if T == 0:
        return

    # attention on the first layer's q/k/v shapes (random operands), with its workspace
    dm = w.dims
    q = activations(62, 1, (T, dm.Hq, dm.d), dtype)
    k = activations(62, 2, (T, dm.Hkv, dm.d), dtype)
    v = activations(62, 3, (T, dm.Hkv, dm.d), dtype)
    q, k, v = to_device(q), to_device(k), to_device(v)
    L0 = dw.layers[0].tensors
    o_ref, lse_ref = tg.gated_attn_fwd(q, k, v, gp.s_c, L0["t"], L0["g"], dw.cu_kept, w.max_k,
                                       want_lse=True)
    o, lse = Guarded("o", (T, dm.Hq, dm.d), dt), Guarded("lse", (dm.Hq, T), torch.float32)
    aws = _ws("attention ws", lib.tg_gated_attn_workspace_size(B, w.max_k, dm.Hq, dm.Hkv, dm.d, code))
    st = lib.tg_gated_attn_fwd(tg._p(q), tg._p(k), tg._p(v), tg._p(gp.s_c), tg._p(L0["t"]),
                               tg._p(L0["g"]), tg._p(dw.cu_kept), B, w.max_k, dm.Hq, dm.Hkv, dm.d, code,
                               tg._p(o.t), tg._p(lse.t), tg._p(aws.t) if aws.nbytes else None, aws.nbytes,
                               tg._stream())
    assert st == 0, tg.status_string(st)
    _check_all(o, lse, aws)
    assert torch.equal(o.t, o_ref) and torch.equal(lse.t, lse_ref)

    # one layer on the compacted rows
    dims = tg.LayerDims(*[getattr(dw.dims, f) for f, _ in tg.LayerDims._fields_])
    if dw.norms_folded:
        dims.flags |= tg.LAYER_NORMS_FOLDED
    lws = _ws("layer ws", lib.tg_upper_layer_workspace_size(ctypes.byref(dims), T, B, w.max_k))
    xo = Guarded("x_out", (T, D), dt)
    kc, vc = Guarded("k", (T, dm.Hkv, dm.d), dt), Guarded("v", (T, dm.Hkv, dm.d), dt)
    x_ref, k_ref, v_ref, _ = tg.upper_layer_fwd(dw.layers[0], dw.dims, hc.t, pc.t, sc.t, dw.cu_kept,
                                                w.max_k, norms_folded=dw.norms_folded)
    tg.upper_layer_fwd(dw.layers[0], dw.dims, hc.t, pc.t, sc.t, dw.cu_kept, w.max_k, x_out=xo.t,
                       kcache=kc.t, vcache=vc.t, ws=lws.t, norms_folded=dw.norms_folded)
    _check_all(xo, kc, vc, lws, hc)
    assert torch.equal(xo.t, x_ref) and torch.equal(kc.t, k_ref) and torch.equal(vc.t, v_ref)


@pytest.mark.parametrize("dtype,N,K,F", CASES)
def test_whole_step_and_three_stage_outputs_stay_inside_their_buffers(dtype, N, K, F):
    say("canaries, whole step and three-stage prefill:", dtype, "N", N, "K", K)
    w = custom(63, N=N, K=K, F=F, dims=_dims(dtype), layers=3)
    dw = DeviceWorkload(w, norms_folded=dtype == "bf16")
    lib = tg.lib()
    dt = dw.h.dtype
    dm = w.dims
    T, T_in, B, D = w.T, w.T_in, w.B, dm.D
    L = len(dw.layers)
    dims = tg.LayerDims(*[getattr(dw.dims, f) for f, _ in tg.LayerDims._fields_])
    if dw.norms_folded:
        dims.flags |= tg.LAYER_NORMS_FOLDED

    # tg_gated_prefill
    gp = GatedPrefill(dw)
    gp.run()
    torch.cuda.synchronize()
    outs = {"s": Guarded("s", (T_in,), torch.float32), "kept": Guarded("kept", (T,), torch.int32),
            "status": Guarded("status", (B,), torch.int32), "x": Guarded("x", (T, D), dt),
            "pos_c": Guarded("pos_c", (T,), torch.int32), "s_c": Guarded("s_c", (T,), torch.float32),
            "k": Guarded("kcache", (L, T, dm.Hkv, dm.d), dt), "v": Guarded("vcache", (L, T, dm.Hkv, dm.d), dt)}
    ws = _ws("step ws", lib.tg_gated_prefill_workspace_size(ctypes.byref(dims), dm.H1, T_in, T, B, w.max_k))
    o = {n: g.t for n, g in outs.items()}
    tg.gated_prefill(dw.h, dw.keep_mask, dw.cu_in, dw.cu_kept, T, w.max_n, w.max_k, dw.W1, dw.b1, dw.w2,
                     dw.b2, dw.layers, dw.dims, o["s"], o["kept"], o["status"], o["x"], o["pos_c"], o["s_c"],
                     o["k"], o["v"], ws=ws.t, norms_folded=dw.norms_folded)
    _check_all(ws, *outs.values())
    assert torch.equal(o["s"], gp.s) and torch.equal(o["kept"], gp.kept) and torch.equal(o["x"], gp.x)
    if T:
        assert torch.equal(o["k"], gp.kcache[:L]) and torch.equal(o["pos_c"], gp.pos_c)

    # tg_full_prefill, gate at layer 1
    fp = FullPrefill(dw, n_below=1)
    fp.run()
    torch.cuda.synchronize()
    na = L - 2
    outs = {"x_full": Guarded("x_full", (T_in, D), dt),
            "kf": Guarded("kcache_full", (2, T_in, dm.Hkv, dm.d), dt),
            "vf": Guarded("vcache_full", (2, T_in, dm.Hkv, dm.d), dt), "s": Guarded("s", (T_in,), torch.float32),
            "kept": Guarded("kept", (T,), torch.int32), "status": Guarded("status", (B,), torch.int32),
            "x": Guarded("x", (T, D), dt), "pos_c": Guarded("pos_c", (T,), torch.int32),
            "s_c": Guarded("s_c", (T,), torch.float32), "k": Guarded("kcache", (na, T, dm.Hkv, dm.d), dt),
            "v": Guarded("vcache", (na, T, dm.Hkv, dm.d), dt)}
    ws = _ws("three-stage ws", lib.tg_full_prefill_workspace_size(ctypes.byref(dims), dm.H1, T_in, T, B,
                                                                 w.max_n, w.max_k))
    o = {n: g.t for n, g in outs.items()}
    tg.full_prefill(dw.h, fp.pos, dw.keep_mask, dw.cu_in, dw.cu_kept, T, w.max_n, w.max_k, dw.W1, dw.b1, dw.w2,
                    dw.b2, fp.below, fp.gate_layer, fp.above, dw.dims, o["x_full"], o["kf"], o["vf"], o["s"],
                    o["kept"], o["status"], o["x"], o["pos_c"], o["s_c"], o["k"], o["v"], ws=ws.t,
                    norms_folded=dw.norms_folded)
    _check_all(ws, *outs.values())
    assert torch.equal(o["x_full"], fp.x_full) and torch.equal(o["kf"], fp.kcache_full)
    assert torch.equal(o["s"], fp.s) and torch.equal(o["kept"], fp.kept) and torch.equal(o["x"], fp.x)
    if T:
        assert torch.equal(o["k"], fp.kcache[:na])


@pytest.mark.parametrize("lens", [([37, 0, 100], [3, 1, 0]), ([3000, 0, 1, 700], [5, 0, 16, 16])])
def test_decode_outputs_stay_inside_their_buffers(lens):
    """Decode attention, single-chunk and split paths: o, lse, status and the
    workspace between guard bands; outputs equal to an unguarded call."""
    lenA, lenB = lens
    B, Hq, Hkv, d, capB = len(lenA), 16, 8, 128, 16
    say("canaries, decode:", lenA, lenB)
    rows = max(sum(lenA), 1)
    act = lambda o, shape: to_device(activations(64, o, shape, "bf16"))
    q, kA, vA = act(1, (B, Hq, d)), act(2, (rows, Hkv, d)), act(3, (rows, Hkv, d))
    kB, vB = act(4, (B, capB, Hkv, d)), act(5, (B, capB, Hkv, d))
    gen = torch.Generator().manual_seed(64)
    sA, sB = torch.rand(rows, generator=gen).cuda(), torch.rand((B, capB), generator=gen).cuda()
    t, g = torch.rand(Hq, generator=gen).cuda() + 0.5, torch.rand(Hq, generator=gen).cuda()
    cuA = torch.tensor([0] + list(np.cumsum(lenA)), dtype=torch.int32, device="cuda")
    lB = torch.tensor(lenB, dtype=torch.int32, device="cuda")
    max_len = max(a + b for a, b in zip(lenA, lenB))
    o_ref, lse_ref, st_ref = tg.decode_attn_fwd(q, kA, vA, sA, cuA, kB, vB, sB, lB, t, g, max_len, want_lse=True)
    lib = tg.lib()
    o, lse = Guarded("o", (B, Hq, d), torch.bfloat16), Guarded("lse", (B, Hq), torch.float32)
    st = Guarded("status", (B,), torch.int32)
    ws = _ws("decode ws", lib.tg_decode_attn_workspace_size(B, max_len, Hq, Hkv, d, 1))
    tg.decode_attn_fwd(q, kA, vA, sA, cuA, kB, vB, sB, lB, t, g, max_len, o=o.t, lse=lse.t, status=st.t,
                       ws=ws.t if ws.nbytes else None)
    _check_all(o, lse, st, ws)
    assert torch.equal(o.t, o_ref) and torch.equal(lse.t, lse_ref) and torch.equal(st.t, st_ref[:B])



@pytest.mark.parametrize("dtype,lens,dk,dv", [("bf16", [300, 0, 1, 77, 130], 128, 96),
                                              ("bf16", [64, 65], 64, 160),
                                              ("f32", [33, 0, 70], 64, 64)])
def test_gdn_outputs_stay_inside_their_buffers(dtype, lens, dk, dv):
    """Gated DeltaNet mixer (chunked bf16 path with its chunk records, fp32
    token path): o, the state and the workspace between guard bands, with a
    carried start state and partial, empty and one-token sequences; outputs
    equal to an unguarded call."""
    B, H, T = len(lens), 4, int(sum(lens))
    say("canaries, gdn:", dtype, lens, "dk", dk, "dv", dv)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    act = lambda o, shape: to_device(activations(65, o, shape, dtype))
    q, k, v = act(1, (T, H, dk)), act(2, (T, H, dk)), act(3, (T, H, dv))
    gen = torch.Generator().manual_seed(65)
    al = (0.8 + 0.2 * torch.rand((T, H), generator=gen)).cuda()
    be = torch.rand((T, H), generator=gen).cuda()
    st0 = (0.3 * torch.randn((B, H, dv, dk), generator=gen)).cuda()
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device="cuda")
    o_ref, st_ref = tg.gdn_fwd(q, k, v, al, be, cu, state_in=st0, want_state=True)
    lib = tg.lib()
    o, st = Guarded("o", (T, H, dv), dt), Guarded("state", (B, H, dv, dk), torch.float32)
    ws = _ws("gdn ws", lib.tg_gdn_workspace_size(T, B, H, dk, dv, tg.dtype_code(dt)))
    tg.gdn_fwd(q, k, v, al, be, cu, state_in=st0, o=o.t, state_out=st.t, ws=ws.t if ws.nbytes else None)
    _check_all(o, st, ws)
    assert torch.equal(o.t, o_ref) and torch.equal(st.t, st_ref)
