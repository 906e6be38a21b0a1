"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments synchronously (before any HIP
call, so these run without a GPU)."""
import ctypes
import os
import re

import pytest

from learned_token_pruning_post_amd import binding as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tokengate.h")

OK, INVALID, UNSUP, WS = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tg.LIB_PATH):
        from learned_token_pruning_post_amd import build
        build.build(verbose=False)
    return tg.lib()


def header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(tg_\w+)\s*\(", txt, flags=re.M)
    return sorted(set(names))


def test_header_and_binding_agree():
    assert header_functions() == sorted(tg.ABI_FUNCTIONS)


def test_every_declared_symbol_is_exported(L):
    for name in header_functions():
        assert hasattr(L, name), name


def test_status_strings_and_version(L):
    for code in range(5):
        assert tg.status_string(code)
    assert tg.status_string(99) == "unknown status"
    assert L.tg_abi_version() >> 16 == 3


def test_gate_score_argument_errors(L):
    f = L.tg_gate_score
    assert f(FAKE, -1, 64, 32, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None, 0, None) == INVALID
    assert f(FAKE, 8, 0, 32, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None, 0, None) == INVALID
    assert f(FAKE, 8, 64, 32, FAKE, FAKE, FAKE, FAKE, 7, FAKE, None, 0, None) == UNSUP
    assert f(None, 8, 64, 32, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None, 0, None) == INVALID
    assert f(FAKE, 8, 100, 32, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None, 0, None) == UNSUP
    # H1 > 256 needs a workspace for the partial sums
    assert L.tg_gate_score_workspace_size(8, 64, 512, 1) > 0
    assert f(FAKE, 8, 64, 512, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None, 0, None) == WS
    assert f(FAKE, 8, 64, 32, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None, 0, None) == WS  # fp32 needs z
    assert f(None, 0, 64, 32, None, None, None, None, 1, None, None, 0, None) == OK  # empty


def test_bf16_operands_of_4_gib_are_refused(L):
    """bf16 operands are addressed through 32-bit buffer ranges: a matrix of
    4 GiB or more is refused up front instead of wrapping silently."""
    f = L.tg_gate_score
    assert f(FAKE, 1 << 20, 2048, 256, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None, 0, None) == UNSUP
    a = L.tg_gated_attn_fwd
    assert a(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1 << 21, 16, 8, 128, 1, FAKE, None, None, 0,
             None) == UNSUP
    dims = tg.LayerDims(2048, 16, 8, 128, 6144, 1e6, 1e-6, 1, 0)
    w = tg.LayerWeights(*([FAKE.value] * 11))
    T = (1 << 32) // (2 * 6144) + 1  # the SwiGLU activation [T, I] reaches 4 GiB
    assert L.tg_upper_layer_fwd(ctypes.byref(w), ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, 1,
                                T, 4096, FAKE, FAKE, FAKE, 1 << 62, None) == UNSUP


def test_topk_select_argument_errors(L):
    f = L.tg_topk_select
    assert f(FAKE, None, FAKE, FAKE, -1, 10, 5, 10, FAKE, None, None, 0, None) == INVALID
    assert f(FAKE, None, FAKE, FAKE, 1, 10, 11, 10, FAKE, None, None, 0, None) == INVALID  # T > T_in
    assert f(FAKE, None, None, FAKE, 1, 10, 5, 10, FAKE, None, None, 0, None) == INVALID
    assert f(FAKE, None, FAKE, FAKE, 1, 10, 5, 10, None, None, None, 0, None) == INVALID
    assert f(None, None, None, None, 0, 0, 0, 0, None, None, None, 0, None) == OK  # B = 0


def test_topk_select_noalloc_argument_errors(L):
    """The allocation-free selection validates like tg_topk_select and refuses,
    before touching a device, a call whose workspace would exceed its scratch."""
    f = L.tg_topk_select_noalloc
    assert f(FAKE, None, FAKE, FAKE, -1, 10, 5, 10, FAKE, None, None) == INVALID
    assert f(FAKE, None, FAKE, FAKE, 1, 10, 11, 10, FAKE, None, None) == INVALID  # T > T_in
    assert f(None, None, None, None, 0, 0, 0, 0, None, None, None) == OK  # B = 0
    cap = tg.SELECT_NOALLOC_SCRATCH_BYTES
    B = 200  # about 8 bytes of scratch per token: 64 MB > 4 MiB
    assert L.tg_topk_select_workspace_size(B, B * 40000, 40000) > cap
    assert f(FAKE, None, FAKE, FAKE, B, B * 40000, B * 100, 40000, FAKE, None, None) == WS
    assert L.tg_topk_select_workspace_size(8, 8 * 40000, 40000) <= cap


def test_topk_select_workspace(L):
    """The selection's scratch: per chunk slot (T_in / CH + B + 1 of them) a
    32-byte record, two bin lists and a key array of CH words each, each block
    256-byte aligned; CH = 512 tokens per chunk, doubled until a sequence of
    max_n tokens has at most 256 chunks (at most 4096)."""
    a = lambda x: (x + 255) // 256 * 256
    for B, T_in, max_n, CH in ((3, 200000, 100000, 512), (1, 32768, 32768, 512), (1, 8192, 100, 512),
                               (8, 131072, 16384, 512), (1, 300000, 262145, 2048),
                               (2, 1 << 21, 1 << 20, 4096)):
        slots = T_in // CH + B + 1
        need = L.tg_topk_select_workspace_size(B, T_in, max_n)
        assert need == a(slots * 32) + 3 * a(slots * CH * 4), (B, T_in, max_n)
    assert L.tg_topk_select_workspace_size(0, 10, 10) == 0
    assert L.tg_topk_select_workspace_size(1, 1 << 23, (1 << 20) + 1) == 0  # unsupported length
    B, T_in, max_n = 3, 200000, 100000
    need = L.tg_topk_select_workspace_size(B, T_in, max_n)
    f = L.tg_topk_select
    assert f(FAKE, None, FAKE, FAKE, B, T_in, 5, max_n, FAKE, None, None, 0, None) == WS
    assert f(FAKE, None, FAKE, FAKE, B, T_in, 5, max_n, FAKE, None, FAKE, need - 1, None) == WS
    odd = ctypes.c_void_p(0x100000 + 16)
    assert f(FAKE, None, FAKE, FAKE, B, T_in, 5, max_n, FAKE, None, odd, need, None) == INVALID
    assert f(FAKE, None, FAKE, FAKE, 1, 1 << 23, 5, (1 << 20) + 1, FAKE, None, FAKE, 1 << 30, None) == UNSUP


def test_select_compact_argument_errors(L):
    """The fused selection + compaction validates like tg_topk_select plus the
    row arguments of tg_compact."""
    f = L.tg_select_compact
    B, T_in, T, max_n = 1, 1000, 100, 1000
    need = L.tg_topk_select_workspace_size(B, T_in, max_n)
    args = lambda **k: [k.get("s", FAKE), None, FAKE, FAKE, B, T_in, k.get("T", T), max_n,
                        k.get("h", FAKE), None, k.get("D", 64), k.get("dt", 1), FAKE, None,
                        k.get("h_out", FAKE), k.get("pos_out", FAKE), None, k.get("ws", FAKE),
                        k.get("wsb", need), None]
    assert f(*args(D=0)) == INVALID
    assert f(*args(dt=5)) == UNSUP
    assert f(*args(h=None)) == INVALID
    assert f(*args(h_out=None)) == INVALID
    assert f(*args(pos_out=None)) == INVALID
    assert f(*args(T=T_in + 1)) == INVALID
    assert f(*args(wsb=need - 1)) == WS
    assert f(*args(ws=None)) == WS


def test_compact_argument_errors(L):
    f = L.tg_compact
    assert f(FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 4, 0, 1, FAKE, FAKE, FAKE, None) == INVALID
    assert f(FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 4, 8, 5, FAKE, FAKE, FAKE, None) == UNSUP
    assert f(None, None, FAKE, FAKE, FAKE, FAKE, 1, 4, 8, 1, FAKE, FAKE, FAKE, None) == INVALID
    assert f(FAKE, None, FAKE, FAKE, None, FAKE, 1, 4, 8, 1, FAKE, FAKE, FAKE, None) == INVALID
    assert f(FAKE, None, None, FAKE, FAKE, FAKE, 1, 4, 8, 1, FAKE, FAKE, FAKE, None) == INVALID
    assert f(None, None, None, None, None, None, 1, 0, 8, 1, None, None, None, None) == OK


def test_attention_argument_errors(L):
    f = L.tg_gated_attn_fwd
    a = [FAKE] * 7
    assert f(*a, 1, 64, 6, 4, 128, 1, FAKE, None, None, 0, None) == INVALID  # Hq % Hkv
    assert f(*a, 1, 64, 8, 4, 96, 1, FAKE, None, None, 0, None) == UNSUP    # head dim
    assert f(*a, 1, 64, 16, 2, 128, 1, FAKE, None, None, 0, None) == UNSUP  # bf16 group of 8
    assert f(*a, 1, 64, 8, 4, 128, 9, FAKE, None, None, 0, None) == UNSUP   # dtype
    assert f(*([None] * 7), 0, 64, 8, 4, 128, 1, None, None, None, 0, None) == OK
    assert f(FAKE, FAKE, None, *([FAKE] * 4), 1, 64, 8, 4, 128, 1, FAKE, None, None, 0, None) == INVALID


def test_decode_attention_argument_errors(L):
    """Every check fails before any launch (FAKE pointers are never dereferenced)."""
    ws = L.tg_decode_attn_workspace_size
    assert ws(1, 100, 16, 8, 128, 1) == 0            # one key chunk per sequence: no workspace
    big = ws(64, 4224, 16, 8, 128, 1)
    assert big >= 64 * 16 * 5 * (128 + 2) * 4        # partial outputs and (max, sum) per chunk
    assert ws(64, 4224, 16, 8, 128, 7) == 0 and ws(0, 4224, 16, 8, 128, 1) == 0
    f = L.tg_decode_attn_fwd

    def call(q=FAKE, kA=FAKE, kB=FAKE, capB=8, B=64, max_len=4224, Hq=16, Hkv=8, d=128, dt=1, o=FAKE,
             w=None, wsb=0):
        return f(q, kA, FAKE, FAKE, FAKE, kB, FAKE, FAKE, FAKE, capB, FAKE, FAKE, B, max_len, Hq, Hkv, d, dt,
                 o, None, None, w, wsb, None)
    assert call(Hq=12) == INVALID                  # Hq % Hkv
    assert call(d=96) == UNSUP                     # head dim
    assert call(Hq=32, Hkv=2) == UNSUP             # group of 16
    assert call(dt=7) == UNSUP                     # dtype code
    assert call(max_len=-1) == INVALID
    assert call(q=None) == INVALID
    assert call(kA=None) == INVALID                # segment A is required even when empty
    assert call(kB=None) == INVALID                # capB > 0 needs segment B
    assert call(q=ctypes.c_void_p(0x100008)) == INVALID  # 16-byte alignment
    assert call() == WS                            # split over chunks: workspace needed
    assert call(w=FAKE, wsb=big - 1) == WS
    assert call(w=ctypes.c_void_p(0x100010), wsb=big) == INVALID  # workspace alignment
    assert call(B=0) == OK                         # nothing to do


def test_attention_backward_argument_errors(L):
    ws = L.tg_gated_attn_bwd_workspace_size
    need = ws(1, 4096, 4096, 16, 8, 128, 1)
    assert need >= 2 * 16 * 4096 * 4 + 8 * 4096 * 4     # lse2 and D per (head, query), ds per kv head
    assert ws(1, 4096, 4096, 16, 8, 128, 0) == 0 and ws(1, 4096, 4096, 16, 2, 128, 1) == 0  # fp32, G=8
    f = L.tg_gated_attn_bwd

    def call(B=1, T=4096, max_k=4096, Hq=16, Hkv=8, d=128, dt=1, q=FAKE, dq=FAKE, w=None, wsb=0):
        return f(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, T, max_k, Hq, Hkv, d, dt, FAKE, FAKE, FAKE, dq, FAKE,
                 FAKE, FAKE, FAKE, FAKE, w, wsb, None)
    assert call(Hq=12) == INVALID
    assert call(dt=0) == UNSUP                      # bf16 only
    assert call(Hkv=2) == UNSUP                     # group of 8
    assert call(d=96) == UNSUP
    assert call(max_k=1 << 20) == UNSUP             # q rows of one sequence reach 4 GiB (32-bit ranges)
    assert call(T=-1) == INVALID
    assert call(q=None) == INVALID
    assert call(dq=None) == INVALID
    assert call(q=ctypes.c_void_p(0x100008)) == INVALID
    assert call() == WS
    assert call(w=FAKE, wsb=need - 1) == WS
    assert call(w=ctypes.c_void_p(0x100010), wsb=need) == INVALID
    assert call(B=0) == OK and call(T=0) == OK and call(max_k=0) == OK


def test_scorer_backward_argument_errors(L):
    assert L.tg_gate_score_bwd_workspace_size(32768, 2048, 256, 1) >= 2 * 32768 * 256 * 2 + 16 * 256 * 2048 * 4
    assert L.tg_gate_score_bwd_workspace_size(32768, 2048, 256, 0) == 0
    f = L.tg_gate_score_bwd

    def call(T=1000, D=256, H1=64, dt=1, h=FAKE, dW1=FAKE, w=None, wsb=0):
        return f(h, T, D, H1, FAKE, FAKE, FAKE, dt, FAKE, FAKE, FAKE, dW1, FAKE, FAKE, FAKE, w, wsb, None)
    assert call(dt=0) == UNSUP
    assert call(D=200) == UNSUP and call(H1=96) == UNSUP
    assert call(T=-1) == INVALID
    assert call(h=None) == INVALID and call(dW1=None) == INVALID
    assert call(h=ctypes.c_void_p(0x100008)) == INVALID
    assert call() == WS
    g = L.tg_compact_scores_bwd
    assert g(FAKE, FAKE, 11, 10, FAKE, None) == INVALID   # more kept than tokens
    assert g(FAKE, None, 5, 10, FAKE, None) == INVALID
    assert g(None, None, 0, 0, None, None) == OK


def test_gdn_argument_errors(L):
    f = L.tg_gdn_fwd

    def call(B=1, H=4, dk=128, dv=128, dt=1, q=FAKE, o=FAKE, T=1000, st=None, ws=None, nws=0):
        return f(q, FAKE, FAKE, FAKE, FAKE, FAKE, T, B, H, dk, dv, dt, st, o, None, ws, nws, None)
    assert call(dk=96) == UNSUP and call(dv=48) == UNSUP and call(dt=5) == UNSUP
    assert call(H=0) == INVALID and call(B=-1) == INVALID and call(T=-1) == INVALID
    assert call(q=None) == INVALID and call(o=None) == INVALID
    assert call(q=ctypes.c_void_p(0x100004)) == INVALID
    assert call(st=ctypes.c_void_p(0x100008)) == INVALID       # the state is read 16 bytes at a time
    need = L.tg_gdn_workspace_size(1000, 1, 4, 128, 128, 1)
    assert need > 0 and L.tg_gdn_workspace_size(1000, 1, 4, 128, 128, 0) == 0   # fp32: no workspace
    assert L.tg_gdn_workspace_size(0, 1, 4, 128, 128, 1) == 0
    assert call() == WS and call(ws=FAKE, nws=need - 1) == WS                 # bf16 needs the chunk records
    assert call(ws=ctypes.c_void_p(0x100010), nws=need) == WS                 # 256-byte aligned
    assert call(B=0) == OK


def test_layer_stack_argument_errors(L):
    f = L.tg_upper_layer_stack_fwd
    dm = _dims()
    good = tg.LayerWeights(*([0x100000] * 11))
    bad = tg.LayerWeights(*([0x100000] * 11))
    bad.wd = None
    args = lambda arr, n, dims: (arr, n, ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, 1, 1000, 1000,
                                 FAKE, FAKE, FAKE, 1 << 40, None)
    two = (tg.LayerWeights * 2)(good, bad)
    assert f(*args(two, -1, dm)) == INVALID
    assert f(*args(None, 0, dm)) == OK          # no layers: nothing to do
    assert f(*args(None, 2, dm)) == INVALID
    assert f(*args(two, 2, dm)) == INVALID      # layer 1's weights checked before any launch
    rope = _dims()
    rope.flags = tg.LAYER_ROPE_READY            # set per layer by the stack itself
    assert f(*args(two, 1, rope)) == INVALID


def test_gated_prefill_argument_errors(L):
    f = L.tg_gated_prefill
    dm = _dims()
    lw = (tg.LayerWeights * 1)(tg.LayerWeights(*([0x100000] * 11)))
    gate = tg.GateWeights(FAKE, FAKE, FAKE, FAKE, 64)
    call = lambda g, dims: f(FAKE, None, None, FAKE, FAKE, 1, 1000, 100, 1000, 100, g, lw, 1, dims,
                             FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert call(None, ctypes.byref(dm)) == INVALID
    assert call(ctypes.byref(gate), None) == INVALID
    bad = tg.GateWeights(FAKE, FAKE, FAKE, FAKE, 6)  # bf16 scorer needs H1 % 4 == 0
    assert call(ctypes.byref(bad), ctypes.byref(dm)) == UNSUP
    ws = L.tg_gated_prefill_workspace_size(ctypes.byref(dm), 64, 1000, 100, 1, 100)
    lay = tg.LayerWsLayout()
    assert L.tg_upper_layer_ws_layout(ctypes.byref(dm), 100, ctypes.byref(lay)) == OK
    assert ws >= lay.total and ws >= L.tg_gate_score_workspace_size(1000, 256, 64, 1)


def test_fold_norm_weights_argument_errors(L):
    f = L.tg_fold_norm_weights
    assert f(FAKE, FAKE, -1, 8, 1, None) == INVALID
    assert f(FAKE, FAKE, 8, -1, 1, None) == INVALID
    assert f(None, FAKE, 8, 8, 1, None) == INVALID
    assert f(FAKE, None, 8, 8, 0, None) == INVALID
    assert f(FAKE, FAKE, 8, 8, 7, None) == UNSUP
    assert f(None, None, 0, 8, 1, None) == OK  # empty
    with pytest.raises(ValueError):
        import torch
        tg.fold_norm_weights(torch.ones(3, dtype=torch.bfloat16), torch.ones(2, 4, dtype=torch.bfloat16))


def _dims(**kw):
    base = dict(D=256, Hq=4, Hkv=2, d=64, I=512, rope_base=1e6, rms_eps=1e-6, dtype=1)
    base.update(kw)
    return tg.LayerDims(base["D"], base["Hq"], base["Hkv"], base["d"], base["I"],
                        base["rope_base"], base["rms_eps"], base["dtype"])


def test_layer_layout_and_errors(L):
    dm = _dims()
    lay = tg.LayerWsLayout()
    assert L.tg_upper_layer_ws_layout(ctypes.byref(dm), 1000, ctypes.byref(lay)) == OK
    offs = [lay.norm, lay.q, lay.attn, lay.x1, lay.act, lay.rope, lay.ssq, lay.total]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.q - lay.norm >= 1000 * 256 * 2 and lay.ssq - lay.rope >= 1000 * 64 * 4
    assert lay.total - lay.ssq >= 2 * 1000 * (256 // 64) * 4  # [2][T][D/64] fp32
    assert L.tg_upper_layer_workspace_size(ctypes.byref(dm), 1000, 1, 1000) == lay.total
    w = tg.LayerWeights(*([0x100000] * 11))
    f = L.tg_upper_layer_fwd
    args = lambda dims, ws_bytes: (ctypes.byref(w), ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE,
                                  FAKE, 1, 1000, 1000, FAKE, FAKE, FAKE, ws_bytes, None)
    assert f(*args(dm, 16)) == WS
    assert f(*args(_dims(d=96), 1 << 40)) == UNSUP
    assert f(*args(_dims(Hq=6, Hkv=4), 1 << 40)) == INVALID
    assert f(*args(_dims(D=200), 1 << 40)) == UNSUP  # bf16 needs D % 64 == 0
    bad_flags = _dims()
    bad_flags.flags = 32  # bits 1, 2, 4, 8 and 16 are the defined ones
    assert f(*args(bad_flags, 1 << 40)) == INVALID
    assert L.tg_upper_layer_ws_layout(ctypes.byref(bad_flags), 1000, ctypes.byref(lay)) == INVALID
    both_halves = _dims()
    both_halves.flags = tg.LAYER_ATTN_ONLY | tg.LAYER_FFN_ONLY
    assert f(*args(both_halves, 1 << 40)) == INVALID
    ssq_alone = _dims()
    ssq_alone.flags = tg.LAYER_INPUT_SSQ  # needs NORMS_FOLDED
    assert f(*args(ssq_alone, 1 << 40)) == INVALID
    folded32 = _dims(dtype=0)
    folded32.flags = tg.LAYER_NORMS_FOLDED  # bf16 only
    assert f(*args(folded32, 1 << 40)) == UNSUP
    # folded norms: the norm weight pointers may be NULL (rejected without the flag)
    w_nonorm = tg.LayerWeights(None, *([0x100000] * 4), None, *([0x100000] * 5))
    no_norm = (ctypes.byref(w_nonorm), ctypes.byref(dm), FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1000, 1000,
               FAKE, FAKE, FAKE, 16, None)
    assert f(*no_norm) == INVALID
    folded = _dims()
    folded.flags = tg.LAYER_NORMS_FOLDED | tg.LAYER_INPUT_SSQ
    assert f(ctypes.byref(w_nonorm), *no_norm[1:1], ctypes.byref(folded), *no_norm[2:]) == WS
    assert f(None, ctypes.byref(dm), *([FAKE] * 5), 1, 1000, 1000, FAKE, FAKE, FAKE, 1 << 40, None) == INVALID
    # fp32 layout carries the raw projections too
    lay32 = tg.LayerWsLayout()
    assert L.tg_upper_layer_ws_layout(ctypes.byref(_dims(dtype=0)), 1000, ctypes.byref(lay32)) == OK
    assert lay32.total > lay32.rope + 1000 * 64 * 4


def test_full_prefill_argument_errors(L):
    """The three-stage prefill validates every stage's arguments before the
    first launch (FAKE pointers are never dereferenced)."""
    dm = _dims()
    w = tg.LayerWeights(*([0x100000] * 11))
    gate = tg.GateWeights(FAKE, FAKE, FAKE, FAKE, 64)
    arr = (tg.LayerWeights * 1)(w)
    need = L.tg_full_prefill_workspace_size(ctypes.byref(dm), 64, 1000, 100, 1, 1000, 100)
    assert need >= L.tg_upper_layer_workspace_size(ctypes.byref(dm), 1000, 1, 1000)
    f = L.tg_full_prefill

    def call(**k):
        return f(FAKE, k.get("pos", FAKE), None, FAKE, FAKE, 1, 1000, k.get("T", 100), 1000, 100,
                 ctypes.byref(gate), arr, k.get("nb", 1), ctypes.byref(w), arr, 1, ctypes.byref(k.get("dm", dm)),
                 FAKE, FAKE, FAKE, FAKE, FAKE, None, k.get("x", FAKE), FAKE, FAKE, FAKE, FAKE,
                 k.get("ws", FAKE), k.get("wsb", need), None)
    assert call(T=1001) == INVALID        # more kept than tokens
    assert call(x=None) == INVALID        # kept rows need an output
    assert call(pos=None) == INVALID      # positions are required
    assert call(nb=-1) == INVALID
    assert call(wsb=need - 1) == WS
    assert call(ws=None) == WS
    bad = _dims()
    bad.flags = tg.LAYER_ROPE_READY       # only NORMS_FOLDED may be set
    assert call(dm=bad) == INVALID
    nul = tg.LayerWeights(*([0x100000] * 6), None, *([0x100000] * 4))  # wg missing
    arr_bad = (tg.LayerWeights * 1)(nul)
    assert f(FAKE, FAKE, None, FAKE, FAKE, 1, 1000, 100, 1000, 100, ctypes.byref(gate), arr_bad, 1,
             ctypes.byref(w), arr, 1, ctypes.byref(dm), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
             FAKE, FAKE, FAKE, FAKE, need, None) == INVALID
