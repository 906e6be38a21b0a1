"""ctypes binding of libtokengate.so (argument marshalling only).

Every function takes torch tensors that already live on the GPU, passes their
device pointers and the current HIP stream to the C ABI declared in
include/tokengate.h, and raises TokenGateError on a non-zero status. No step
of the computation happens here, and there is no fallback: if the library is
missing this module raises on first use.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# TG_LIBRARY names another build of the same library to load instead (the
# host-side sanitizer build of build.py --sanitize); by default the in-tree one
LIB_PATH = os.environ.get("TG_LIBRARY") or os.path.join(_HERE, "libtokengate.so")

TG_F32 = 0
TG_BF16 = 1
DEV_FORCED_GT_BUDGET = 1
DEV_BUDGET_GT_LEN = 2
DEV_NAN_SCORE = 4
DEV_LEN_GT_MAX_N = 8

# every entry point declared in include/tokengate.h
ABI_FUNCTIONS = (
    "tg_status_string", "tg_abi_version",
    "tg_gate_score_workspace_size", "tg_gate_score",
    "tg_topk_select_workspace_size", "tg_topk_select", "tg_topk_select_noalloc",
    "tg_compact", "tg_select_compact",
    "tg_gated_attn_workspace_size", "tg_gated_attn_fwd",
    "tg_upper_layer_ws_layout", "tg_upper_layer_workspace_size", "tg_upper_layer_fwd",
    "tg_upper_layer_fwd_timed", "tg_fold_norm_weights", "tg_upper_layer_stack_fwd",
    "tg_gated_prefill_workspace_size", "tg_gated_prefill",
    "tg_full_prefill_workspace_size", "tg_full_prefill",
    "tg_decode_attn_workspace_size", "tg_decode_attn_fwd",
    "tg_gated_attn_bwd_workspace_size", "tg_gated_attn_bwd",
    "tg_gate_score_bwd_workspace_size", "tg_gate_score_bwd", "tg_compact_scores_bwd",
    "tg_gdn_workspace_size", "tg_gdn_fwd",
)
LAYER_STAGES = 8
LAYER_STAGE_NAMES = ("rope_table", "rmsnorm_attn", "qkv_rope_kv", "gated_attn", "o_proj_resid",
                     "rmsnorm_ffn", "gate_up_swiglu", "down_proj_resid")


class TokenGateError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, status_string(status), status))


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "wg", "wu", "wd", "t", "g")]


class GateWeights(ctypes.Structure):
    _fields_ = [("W1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("b2", ctypes.c_void_p), ("H1", ctypes.c_int)]


class LayerDims(ctypes.Structure):
    _fields_ = [("D", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int),
                ("d", ctypes.c_int), ("I", ctypes.c_int), ("rope_base", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int), ("flags", ctypes.c_int)]

LAYER_ROPE_READY = 1  # tg_layer_dims.flags: the workspace already holds this RoPE table
LAYER_NORMS_FOLDED = 2  # norm weights folded into wq/wk/wv and wg/wu: RMSNorms fused into the GEMMs
LAYER_INPUT_SSQ = 4  # with NORMS_FOLDED: the workspace holds x_in's row sums of squares
LAYER_ATTN_ONLY = 8  # the attention half only: x_out = the post-attention residual
LAYER_FFN_ONLY = 16  # the FFN half only: x_in is the post-attention residual


class LayerWsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("norm", "q", "attn", "x1", "act", "rope", "ssq", "total")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtokengate.so (built in-tree by build.py); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libtokengate.so not built (%s); run "
                           "learned_token_pruning_post_amd/build.py" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    L.tg_status_string.argtypes = [i32]
    L.tg_status_string.restype = ctypes.c_char_p
    L.tg_abi_version.argtypes = []
    L.tg_abi_version.restype = i32
    L.tg_gate_score_workspace_size.argtypes = [i64, i32, i32, i32]
    L.tg_gate_score_workspace_size.restype = sz
    L.tg_gate_score.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, i32, vp, vp, sz, vp]
    L.tg_gate_score.restype = i32
    L.tg_topk_select_workspace_size.argtypes = [i32, i64, i32]
    L.tg_topk_select_workspace_size.restype = sz
    L.tg_topk_select.argtypes = [vp, vp, vp, vp, i32, i64, i64, i32, vp, vp, vp, sz, vp]
    L.tg_topk_select.restype = i32
    L.tg_topk_select_noalloc.argtypes = [vp, vp, vp, vp, i32, i64, i64, i32, vp, vp, vp]
    L.tg_topk_select_noalloc.restype = i32
    L.tg_compact.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, vp, vp, vp, vp]
    L.tg_compact.restype = i32
    L.tg_select_compact.argtypes = [vp, vp, vp, vp, i32, i64, i64, i32, vp, vp, i32, i32, vp, vp, vp, vp,
                                    vp, vp, sz, vp]
    L.tg_select_compact.restype = i32
    L.tg_gated_attn_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    L.tg_gated_attn_workspace_size.restype = sz
    L.tg_gated_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                    vp, vp, vp, sz, vp]
    L.tg_gated_attn_fwd.restype = i32
    L.tg_upper_layer_ws_layout.argtypes = [ctypes.POINTER(LayerDims), i64, ctypes.POINTER(LayerWsLayout)]
    L.tg_upper_layer_ws_layout.restype = i32
    L.tg_upper_layer_workspace_size.argtypes = [ctypes.POINTER(LayerDims), i64, i32, i32]
    L.tg_upper_layer_workspace_size.restype = sz
    L.tg_upper_layer_fwd.argtypes = [ctypes.POINTER(LayerWeights), ctypes.POINTER(LayerDims),
                                     vp, vp, vp, vp, vp, i32, i64, i32, vp, vp, vp, sz, vp]
    L.tg_upper_layer_fwd.restype = i32
    L.tg_upper_layer_fwd_timed.argtypes = L.tg_upper_layer_fwd.argtypes + [vp]
    L.tg_upper_layer_fwd_timed.restype = i32
    L.tg_upper_layer_stack_fwd.argtypes = [ctypes.POINTER(LayerWeights), i32, ctypes.POINTER(LayerDims),
                                           vp, vp, vp, vp, i32, i64, i32, vp, vp, vp, sz, vp]
    L.tg_upper_layer_stack_fwd.restype = i32
    L.tg_gated_prefill_workspace_size.argtypes = [ctypes.POINTER(LayerDims), i32, i64, i64, i32, i32]
    L.tg_gated_prefill_workspace_size.restype = sz
    L.tg_gated_prefill.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i32, i32, ctypes.POINTER(GateWeights),
                                   ctypes.POINTER(LayerWeights), i32, ctypes.POINTER(LayerDims),
                                   vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.tg_gated_prefill.restype = i32
    L.tg_full_prefill_workspace_size.argtypes = [ctypes.POINTER(LayerDims), i32, i64, i64, i32, i32, i32]
    L.tg_full_prefill_workspace_size.restype = sz
    L.tg_full_prefill.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i32, i32, ctypes.POINTER(GateWeights),
                                  ctypes.POINTER(LayerWeights), i32, ctypes.POINTER(LayerWeights),
                                  ctypes.POINTER(LayerWeights), i32, ctypes.POINTER(LayerDims),
                                  vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.tg_full_prefill.restype = i32
    L.tg_gated_attn_bwd_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32]
    L.tg_gated_attn_bwd_workspace_size.restype = sz
    L.tg_gated_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, i32, vp, vp, vp,
                                    vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.tg_gated_attn_bwd.restype = i32
    L.tg_gate_score_bwd_workspace_size.argtypes = [i64, i32, i32, i32]
    L.tg_gate_score_bwd_workspace_size.restype = sz
    L.tg_gate_score_bwd.argtypes = [vp, i64, i32, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.tg_gate_score_bwd.restype = i32
    L.tg_compact_scores_bwd.argtypes = [vp, vp, i64, i64, vp, vp]
    L.tg_compact_scores_bwd.restype = i32
    L.tg_gdn_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32]
    L.tg_gdn_workspace_size.restype = sz
    L.tg_gdn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.tg_gdn_fwd.restype = i32
    L.tg_decode_attn_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    L.tg_decode_attn_workspace_size.restype = sz
    L.tg_decode_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                     i32, vp, vp, vp, vp, sz, vp]
    L.tg_decode_attn_fwd.restype = i32
    L.tg_fold_norm_weights.argtypes = [vp, vp, i64, i32, i32, vp]
    L.tg_fold_norm_weights.restype = i32
    _lib = L
    return L


def status_string(s: int) -> str:
    return lib().tg_status_string(int(s)).decode()


def _check(st: int, what: str):
    if st != 0:
        raise TokenGateError(st, what)


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return TG_BF16
    if dt == torch.float32:
        return TG_F32
    raise ValueError("unsupported dtype %s" % dt)


def _empty_ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
def gate_score(h, W1, b1, w2, b2, s_out=None, ws=None):
    T_in, D = h.shape
    H1 = W1.shape[0]
    dt = dtype_code(h.dtype)
    if s_out is None:
        s_out = torch.empty(T_in, dtype=torch.float32, device=h.device)
    need = lib().tg_gate_score_workspace_size(T_in, D, H1, dt)
    if ws is None or ws.numel() < need:
        ws = _empty_ws(need, h.device)
    _check(lib().tg_gate_score(_p(h), T_in, D, H1, _p(W1), _p(b1), _p(w2), _p(b2), dt,
                               _p(s_out), _p(ws), ws.numel(), _stream()), "tg_gate_score")
    return s_out


def topk_select(s, keep_mask, cu_in, cu_kept, T: int, max_n: int, kept=None, status=None, ws=None):
    B = cu_in.numel() - 1
    if kept is None:
        kept = torch.empty(max(T, 0), dtype=torch.int32, device=s.device)
    if status is None:
        status = torch.empty(max(B, 1), dtype=torch.int32, device=s.device)
    need = lib().tg_topk_select_workspace_size(max(B, 0), s.numel(), max_n)
    if ws is None or ws.numel() < need:
        ws = _empty_ws(need, s.device)
    _check(lib().tg_topk_select(_p(s), _p(keep_mask), _p(cu_in), _p(cu_kept), B, s.numel(), T,
                                max_n, _p(kept), _p(status), _p(ws), ws.numel(), _stream()),
           "tg_topk_select")
    return kept, status


SELECT_NOALLOC_SCRATCH_BYTES = 4 << 20  # TG_SELECT_NOALLOC_SCRATCH_BYTES


def topk_select_noalloc(s, keep_mask, cu_in, cu_kept, T: int, max_n: int, kept, status):
    """tg_topk_select_noalloc: the selection on the library's own device scratch
    (no workspace argument); the caller passes the outputs."""
    B = cu_in.numel() - 1
    _check(lib().tg_topk_select_noalloc(_p(s), _p(keep_mask), _p(cu_in), _p(cu_kept), B, s.numel(),
                                        T, max_n, _p(kept), _p(status), _stream()),
           "tg_topk_select_noalloc")
    return kept, status


def compact(h, pos, s, kept, cu_in, cu_kept, h_out=None, pos_out=None, s_out=None):
    T = kept.numel()
    D = h.shape[1]
    B = cu_kept.numel() - 1
    if h_out is None:
        h_out = torch.empty((T, D), dtype=h.dtype, device=h.device)
    if pos_out is None:
        pos_out = torch.empty(T, dtype=torch.int32, device=h.device)
    if s_out is None:
        s_out = torch.empty(T, dtype=torch.float32, device=h.device)
    _check(lib().tg_compact(_p(h), _p(pos), _p(s), _p(kept), _p(cu_in), _p(cu_kept), B, T, D,
                            dtype_code(h.dtype), _p(h_out), _p(pos_out), _p(s_out), _stream()),
           "tg_compact")
    return h_out, pos_out, s_out


def select_compact(s, keep_mask, cu_in, cu_kept, T: int, max_n: int, h, pos=None, kept=None,
                   status=None, h_out=None, pos_out=None, s_out=None, ws=None):
    """tg_select_compact: the selection and the compaction of the kept rows in
    one pass (outputs as topk_select followed by compact)."""
    B = cu_in.numel() - 1
    dev = s.device
    D = h.shape[1]
    if kept is None:
        kept = torch.empty(max(T, 0), dtype=torch.int32, device=dev)
    if status is None:
        status = torch.empty(max(B, 1), dtype=torch.int32, device=dev)
    if h_out is None:
        h_out = torch.empty((T, D), dtype=h.dtype, device=dev)
    if pos_out is None:
        pos_out = torch.empty(T, dtype=torch.int32, device=dev)
    if s_out is None:
        s_out = torch.empty(T, dtype=torch.float32, device=dev)
    need = lib().tg_topk_select_workspace_size(max(B, 0), s.numel(), max_n)
    if ws is None or ws.numel() < need:
        ws = _empty_ws(need, dev)
    _check(lib().tg_select_compact(_p(s), _p(keep_mask), _p(cu_in), _p(cu_kept), B, s.numel(), T, max_n,
                                   _p(h), _p(pos), D, dtype_code(h.dtype), _p(kept), _p(status),
                                   _p(h_out), _p(pos_out), _p(s_out), _p(ws), ws.numel(), _stream()),
           "tg_select_compact")
    return kept, status, h_out, pos_out, s_out


def gated_attn_fwd(q, k, v, s_c, t, g, cu_kept, max_k: int, o=None, lse=None, want_lse=False):
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    B = cu_kept.numel() - 1
    if o is None:
        o = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    _check(lib().tg_gated_attn_fwd(_p(q), _p(k), _p(v), _p(s_c), _p(t), _p(g), _p(cu_kept), B,
                                   max_k, Hq, Hkv, d, dtype_code(q.dtype), _p(o), _p(lse), None, 0,
                                   _stream()), "tg_gated_attn_fwd")
    return o, lse


def gated_attn_bwd(q, k, v, s_c, t, g, cu_kept, max_k: int, o, lse, dO, ws=None):
    """tg_gated_attn_bwd: gradients of the gated attention (fp32). Returns a dict
    dq, dk, dv, ds, dt, dg."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    B = cu_kept.numel() - 1
    dev = q.device
    f = lambda shape: torch.empty(shape, dtype=torch.float32, device=dev)
    r = {"dq": f((T, Hq, d)), "dk": f((T, Hkv, d)), "dv": f((T, Hkv, d)), "ds": f((T,)), "dt": f((Hq,)),
         "dg": f((Hq,))}
    need = lib().tg_gated_attn_bwd_workspace_size(B, T, max_k, Hq, Hkv, d, dtype_code(q.dtype))
    if ws is None or ws.numel() < need:
        ws = _empty_ws(max(need, 1), dev)
    _check(lib().tg_gated_attn_bwd(_p(q), _p(k), _p(v), _p(s_c), _p(t), _p(g), _p(cu_kept), B, T, max_k, Hq,
                                   Hkv, d, dtype_code(q.dtype), _p(o), _p(lse), _p(dO), _p(r["dq"]), _p(r["dk"]),
                                   _p(r["dv"]), _p(r["ds"]), _p(r["dt"]), _p(r["dg"]), _p(ws), ws.numel(),
                                   _stream()), "tg_gated_attn_bwd")
    return r


def gate_score_bwd(h, W1, b1, w2, s, ds, ws=None):
    """tg_gate_score_bwd: returns dict dh (h's dtype), dW1, db1, dw2, db2 (fp32)."""
    T_in, D = h.shape
    H1 = W1.shape[0]
    dev = h.device
    r = {"dh": torch.empty_like(h), "dW1": torch.empty((H1, D), dtype=torch.float32, device=dev),
         "db1": torch.empty(H1, dtype=torch.float32, device=dev),
         "dw2": torch.empty(H1, dtype=torch.float32, device=dev),
         "db2": torch.empty(1, dtype=torch.float32, device=dev)}
    need = lib().tg_gate_score_bwd_workspace_size(T_in, D, H1, dtype_code(h.dtype))
    if need and (ws is None or ws.numel() < need):
        ws = _empty_ws(need, dev)
    _check(lib().tg_gate_score_bwd(_p(h), T_in, D, H1, _p(W1), _p(b1), _p(w2), dtype_code(h.dtype), _p(s),
                                   _p(ds), _p(r["dh"]), _p(r["dW1"]), _p(r["db1"]), _p(r["dw2"]), _p(r["db2"]),
                                   _p(ws) if need else None, ws.numel() if need else 0, _stream()),
           "tg_gate_score_bwd")
    return r


def compact_scores_bwd(ds_c, kept, T_in: int, ds=None):
    """tg_compact_scores_bwd: the prompt scores' gradient (zeros off the kept tokens)."""
    if ds is None:
        ds = torch.empty(T_in, dtype=torch.float32, device=ds_c.device)
    _check(lib().tg_compact_scores_bwd(_p(ds_c), _p(kept), kept.numel(), T_in, _p(ds), _stream()),
           "tg_compact_scores_bwd")
    return ds


def gdn_fwd(q, k, v, alpha, beta, cu, state_in=None, o=None, state_out=None, want_state=False, ws=None):
    """tg_gdn_fwd: the Gated DeltaNet mixer over the packed sequences of cu.
    Returns (o, state_out)."""
    T, H, dk = q.shape
    dv = v.shape[2]
    B = cu.numel() - 1
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    if want_state and state_out is None:
        state_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    code = dtype_code(q.dtype)
    need = lib().tg_gdn_workspace_size(T, B, H, dk, dv, code)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib().tg_gdn_fwd(_p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(cu), T, B, H, dk, dv, code,
                            _p(state_in), _p(o), _p(state_out), _p(ws), ws.numel() if ws is not None else 0,
                            _stream()), "tg_gdn_fwd")
    return o, state_out


def decode_attn_fwd(q, kA, vA, sA, cuA, kB, vB, sB, lenB, t, g, max_len: int, o=None, lse=None,
                    status=None, ws=None, want_lse=False):
    """tg_decode_attn_fwd: q [B, Hq, d]; segment A = the prefill's kept-token
    cache (kA, vA [rows, Hkv, d], sA [rows], cuA [B+1]); segment B = generated
    tokens (kB, vB [B, capB, Hkv, d], sB [B, capB], lenB [B]; capB may be 0).
    Returns (o, lse, status)."""
    B, Hq, d = q.shape
    Hkv = kA.shape[1]
    capB = kB.shape[1] if kB is not None else 0
    dev = q.device
    if o is None:
        o = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if status is None:
        status = torch.empty(max(B, 1), dtype=torch.int32, device=dev)
    code = dtype_code(q.dtype)
    need = lib().tg_decode_attn_workspace_size(B, max_len, Hq, Hkv, d, code)
    if need and (ws is None or ws.numel() < need):
        ws = _empty_ws(need, dev)
    _check(lib().tg_decode_attn_fwd(_p(q), _p(kA), _p(vA), _p(sA), _p(cuA), _p(kB), _p(vB), _p(sB), _p(lenB),
                                    capB, _p(t), _p(g), B, max_len, Hq, Hkv, d, code, _p(o), _p(lse),
                                    _p(status), _p(ws) if need else None, ws.numel() if need else 0,
                                    _stream()), "tg_decode_attn_fwd")
    return o, lse, status


def layer_dims(D, Hq, Hkv, d, I, dtype: torch.dtype, rope_base=1.0e6, rms_eps=1.0e-6) -> LayerDims:
    return LayerDims(D, Hq, Hkv, d, I, rope_base, rms_eps, dtype_code(dtype), 0)


def upper_layer_ws_layout(dims: LayerDims, T: int) -> LayerWsLayout:
    out = LayerWsLayout()
    _check(lib().tg_upper_layer_ws_layout(ctypes.byref(dims), T, ctypes.byref(out)),
           "tg_upper_layer_ws_layout")
    return out


class UpperLayerWeights:
    """Device weights of one upper layer (keys as in tg_layer_weights)."""

    def __init__(self, tensors: Dict[str, torch.Tensor]):
        self.tensors = tensors
        self.c = LayerWeights(*[_p(tensors[n]) for n, _ in LayerWeights._fields_])


def upper_layer_stack_fwd(layers, dims: LayerDims, x, pos_c, s_c, cu_kept, max_k: int, kcache, vcache,
                          ws=None, norms_folded=False):
    """All layers of ``layers`` (UpperLayerWeights) on x in place, one native
    call; kcache / vcache are [n_layers, T, Hkv, d]. Returns x."""
    n = len(layers)
    T = x.shape[0]
    B = cu_kept.numel() - 1
    if norms_folded:
        dims = LayerDims(*[getattr(dims, f) for f, _ in LayerDims._fields_])
        dims.flags |= LAYER_NORMS_FOLDED
    need = lib().tg_upper_layer_workspace_size(ctypes.byref(dims), T, B, max_k)
    if ws is None or ws.numel() < need:
        ws = _empty_ws(need, x.device)
    arr = (LayerWeights * max(n, 1))(*[l.c for l in layers])
    _check(lib().tg_upper_layer_stack_fwd(arr, n, ctypes.byref(dims), _p(x), _p(pos_c), _p(s_c), _p(cu_kept),
                                          B, T, max_k, _p(kcache), _p(vcache), _p(ws), ws.numel(), _stream()),
           "tg_upper_layer_stack_fwd")
    return x


def gated_prefill(h, keep_mask, cu_in, cu_kept, T: int, max_n: int, max_k: int, W1, b1, w2, b2,
                  layers, dims: LayerDims, s, kept, status, x, pos_c, s_c, kcache, vcache, ws=None,
                  norms_folded=False, pos=None):
    """The whole step in one native call (tg_gated_prefill): scorer, select,
    compact, then every layer of ``layers`` on the kept tokens. All outputs
    are caller-allocated tensors; returns x."""
    B = cu_in.numel() - 1
    T_in = h.shape[0]
    if norms_folded:
        dims = LayerDims(*[getattr(dims, f) for f, _ in LayerDims._fields_])
        dims.flags |= LAYER_NORMS_FOLDED
    H1 = W1.shape[0]
    need = lib().tg_gated_prefill_workspace_size(ctypes.byref(dims), H1, T_in, T, B, max_k)
    if ws is None or ws.numel() < need:
        ws = _empty_ws(need, h.device)
    gate = GateWeights(_p(W1), _p(b1), _p(w2), _p(b2), H1)
    n = len(layers)
    arr = (LayerWeights * max(n, 1))(*[l.c for l in layers])
    _check(lib().tg_gated_prefill(_p(h), _p(pos), _p(keep_mask), _p(cu_in), _p(cu_kept), B, T_in, T, max_n,
                                  max_k, ctypes.byref(gate), arr, n, ctypes.byref(dims), _p(s), _p(kept),
                                  _p(status), _p(x), _p(pos_c), _p(s_c), _p(kcache), _p(vcache), _p(ws),
                                  ws.numel(), _stream()), "tg_gated_prefill")
    return x


def full_prefill(h, pos, keep_mask, cu_in, cu_kept, T: int, max_n: int, max_k: int, W1, b1, w2, b2,
                 below, gate_layer, above, dims: LayerDims, x_full, kcache_full, vcache_full, s, kept,
                 status, x, pos_c, s_c, kcache, vcache, ws=None, norms_folded=False):
    """The three-stage prefill in one native call (tg_full_prefill): the layers
    ``below`` and ``gate_layer``'s attention on every row of h, the scorer on
    that residual, selection with compaction, ``gate_layer``'s FFN and the
    layers ``above`` on the kept rows. All outputs are caller-allocated; returns x."""
    B = cu_in.numel() - 1
    T_in = h.shape[0]
    if norms_folded:
        dims = LayerDims(*[getattr(dims, f) for f, _ in LayerDims._fields_])
        dims.flags |= LAYER_NORMS_FOLDED
    H1 = W1.shape[0]
    need = lib().tg_full_prefill_workspace_size(ctypes.byref(dims), H1, T_in, T, B, max_n, max_k)
    if ws is None or ws.numel() < need:
        ws = _empty_ws(need, h.device)
    gate = GateWeights(_p(W1), _p(b1), _p(w2), _p(b2), H1)
    nb, na = len(below), len(above)
    arr_b = (LayerWeights * max(nb, 1))(*[l.c for l in below])
    arr_a = (LayerWeights * max(na, 1))(*[l.c for l in above])
    gl = gate_layer.c
    _check(lib().tg_full_prefill(_p(h), _p(pos), _p(keep_mask), _p(cu_in), _p(cu_kept), B, T_in, T, max_n,
                                 max_k, ctypes.byref(gate), arr_b, nb, ctypes.byref(gl), arr_a, na,
                                 ctypes.byref(dims), _p(x_full), _p(kcache_full), _p(vcache_full), _p(s),
                                 _p(kept), _p(status), _p(x), _p(pos_c), _p(s_c), _p(kcache), _p(vcache),
                                 _p(ws), ws.numel(), _stream()), "tg_full_prefill")
    return x


def fold_norm_weights(norm_w: torch.Tensor, W: torch.Tensor) -> torch.Tensor:
    """W[r, c] *= norm_w[c] in place (fp32 product rounded to W's dtype); returns W."""
    if W.dim() != 2 or norm_w.numel() != W.shape[1] or norm_w.dtype != W.dtype:
        raise ValueError("fold_norm_weights: W [rows, cols] and norm_w [cols] of one dtype")
    _check(lib().tg_fold_norm_weights(_p(norm_w.contiguous()), _p(W), W.shape[0], W.shape[1],
                                      dtype_code(W.dtype), _stream()), "tg_fold_norm_weights")
    return W


def upper_layer_fwd(w: UpperLayerWeights, dims: LayerDims, x_in, pos_c, s_c, cu_kept, max_k: int,
                    x_out=None, kcache=None, vcache=None, ws=None, events=None, rope_ready=False,
                    norms_folded=False, input_ssq=False, attn_only=False, ffn_only=False):
    """One upper layer. ``events``: optional ctypes array of LAYER_STAGES + 1
    hipEvent_t handles; when given, the instrumented entry point records them
    between the layer's stages. ``rope_ready``: ``ws`` already holds the RoPE
    table of these positions (an earlier layer of the same stack ran on it).
    ``norms_folded``: the weights went through fold_norm_weights and the RMSNorms
    run fused into the GEMMs; ``input_ssq``: ``ws`` holds x_in's row sums of
    squares from the previous folded layer of the stack. ``attn_only``: the
    attention half only (x_out = the post-attention residual); ``ffn_only``:
    the FFN half only (x_in is that residual; no K/V, positions or scores are
    read and none of kcache / vcache is written)."""
    flags = (LAYER_ROPE_READY if rope_ready else 0) | (LAYER_NORMS_FOLDED if norms_folded else 0) | \
        (LAYER_INPUT_SSQ if input_ssq else 0) | (LAYER_ATTN_ONLY if attn_only else 0) | \
        (LAYER_FFN_ONLY if ffn_only else 0)
    if (rope_ready or input_ssq) and ws is None:
        raise ValueError("rope_ready / input_ssq need the workspace that holds the table / sums")
    if flags:
        dims = LayerDims(*[getattr(dims, n) for n, _ in LayerDims._fields_])
        dims.flags |= flags
    T = x_in.shape[0]
    B = cu_kept.numel() - 1
    dev = x_in.device
    if x_out is None:
        x_out = torch.empty_like(x_in)
    if kcache is None and not ffn_only:
        kcache = torch.empty((T, dims.Hkv, dims.d), dtype=x_in.dtype, device=dev)
    if vcache is None and not ffn_only:
        vcache = torch.empty((T, dims.Hkv, dims.d), dtype=x_in.dtype, device=dev)
    need = lib().tg_upper_layer_workspace_size(ctypes.byref(dims), T, B, max_k)
    if ws is None or ws.numel() < need:
        ws = _empty_ws(need, dev)
    args = (ctypes.byref(w.c), ctypes.byref(dims), _p(x_in), _p(x_out), _p(pos_c), _p(s_c),
            _p(cu_kept), B, T, max_k, _p(kcache), _p(vcache), _p(ws), ws.numel(), _stream())
    if events is None:
        _check(lib().tg_upper_layer_fwd(*args), "tg_upper_layer_fwd")
    else:
        _check(lib().tg_upper_layer_fwd_timed(*args, events), "tg_upper_layer_fwd_timed")
    return x_out, kcache, vcache, ws
