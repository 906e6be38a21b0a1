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


def test_topk_select_argument_errors(L):
    f = L.tg_topk_select
    assert f(FAKE, None, FAKE, FAKE, -1, 10, 5, 10, FAKE, None, None, 0, None) == INVALID
    assert f(FAKE, None, FAKE, FAKE, 1, 10, 11, 10, FAKE, None, None, 0, None) == INVALID  # T > T_in
    assert f(FAKE, None, None, FAKE, 1, 10, 5, 10, FAKE, None, None, 0, None) == INVALID
    assert f(FAKE, None, FAKE, FAKE, 1, 10, 5, 10, None, None, None, 0, None) == INVALID
    assert f(None, None, None, None, 0, 0, 0, 0, None, None, None, 0, None) == OK  # B = 0
    assert L.tg_topk_select_workspace_size(8, 1 << 17, 1 << 14) == 0


def test_topk_select_long_path_workspace(L):
    """Above 32768 tokens per sequence the selection needs scratch: three
    4096-bin histograms per sequence and a 32-byte record per 4096-token
    chunk slot, each block 256-byte aligned."""
    B, T_in, max_n = 3, 200000, 100000
    a = lambda x: (x + 255) // 256 * 256
    need = L.tg_topk_select_workspace_size(B, T_in, max_n)
    assert need == a(B * 3 * 4096 * 4) + a((T_in // 4096 + B + 1) * 32)
    assert L.tg_topk_select_workspace_size(B, T_in, 32768) == 0
    assert L.tg_topk_select_workspace_size(B, T_in, 32769) == need
    f = L.tg_topk_select
    assert f(FAKE, None, FAKE, FAKE, B, T_in, 5, max_n, FAKE, None, None, 0, None) == WS
    assert f(FAKE, None, FAKE, FAKE, B, T_in, 5, max_n, FAKE, None, FAKE, need - 1, None) == WS
    odd = ctypes.c_void_p(0x100000 + 16)
    assert f(FAKE, None, FAKE, FAKE, B, T_in, 5, max_n, FAKE, None, odd, need, None) == INVALID


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
    bad_flags.flags = 8  # TG_LAYER_ROPE_READY | NORMS_FOLDED | INPUT_SSQ are the defined bits
    assert f(*args(bad_flags, 1 << 40)) == INVALID
    assert L.tg_upper_layer_ws_layout(ctypes.byref(bad_flags), 1000, ctypes.byref(lay)) == INVALID
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
