"""The gated prefill above layer L's attention, driven through the C ABI.

Uploads a seeded workload to the GPU once, allocates every buffer once, and
runs scorer -> Top-K select -> compaction -> the stack of upper layers
(three-stage forward: Tencent Cloud TokenGate article, early token filtering;
farwalk.ai summary, the method). All compute happens in libtokengate.so.
"""
from __future__ import annotations

import concurrent.futures as cf
from typing import List, Optional

import numpy as np
import torch

from . import binding as tg
from .workloads import Workload, gate_inputs, layer_weights, Tensor


def to_device(t: Tensor, device="cuda") -> torch.Tensor:
    if t.bits is not None:
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(t.value)).to(device)


def torch_dtype(w: Workload) -> torch.dtype:
    return torch.bfloat16 if w.dims.dtype == "bf16" else torch.float32


class DeviceWorkload:
    """Seeded inputs and weights of a workload, resident in HBM."""

    def __init__(self, w: Workload, n_layers: Optional[int] = None, device="cuda", keep_host=False,
                 norms_folded: bool = False):
        """``norms_folded`` (bf16): fold each layer's RMSNorm weights into its
        projections once here, so the layers run with the norms fused into the
        GEMMs (tg_layer_dims flag TG_LAYER_NORMS_FOLDED)."""
        self.w = w
        self.norms_folded = bool(norms_folded) and w.dims.dtype == "bf16"
        self.device = device
        gi = gate_inputs(w)
        self.host_gate = gi if keep_host else None
        self.h = to_device(gi.h, device)
        self.W1 = to_device(gi.W1, device)
        self.b1 = to_device(gi.b1, device)
        self.w2 = to_device(gi.w2, device)
        self.b2 = to_device(gi.b2, device)
        self.keep_mask = torch.from_numpy(gi.keep_mask).to(device)
        self.cu_in = torch.from_numpy(gi.cu_in).to(device)
        self.cu_kept = torch.from_numpy(gi.cu_kept).to(device)
        L = w.layers if n_layers is None else n_layers
        self.layers: List[tg.UpperLayerWeights] = []
        self.host_layers = [] if keep_host else None
        self.extend_layers(L)
        dm = w.dims
        self.dims = tg.layer_dims(dm.D, dm.Hq, dm.Hkv, dm.d, dm.I, torch_dtype(w), dm.rope_base, dm.rms_eps)

    def extend_layers(self, n_total: int):
        """Generate and upload the seeded layers len(self.layers) .. n_total - 1."""
        w, device = self.w, self.device
        with cf.ThreadPoolExecutor(4) as ex:
            for lw in ex.map(lambda l: layer_weights(w, l), range(len(self.layers), n_total)):
                if self.host_layers is not None:
                    self.host_layers.append(lw)
                tens = {
                    "attn_norm": to_device(lw.attn_norm, device), "wq": to_device(lw.wq, device),
                    "wk": to_device(lw.wk, device), "wv": to_device(lw.wv, device),
                    "wo": to_device(lw.wo, device), "ffn_norm": to_device(lw.ffn_norm, device),
                    "wg": to_device(lw.wg, device), "wu": to_device(lw.wu, device),
                    "wd": to_device(lw.wd, device),
                    "t": torch.from_numpy(lw.t).to(device), "g": torch.from_numpy(lw.g).to(device),
                }
                if self.norms_folded:
                    for n in ("wq", "wk", "wv"):
                        tg.fold_norm_weights(tens["attn_norm"], tens[n])
                    for n in ("wg", "wu"):
                        tg.fold_norm_weights(tens["ffn_norm"], tens[n])
                self.layers.append(tg.UpperLayerWeights(tens))


class GatedPrefill:
    """Preallocated buffers plus one call per step of the path."""

    def __init__(self, dw: DeviceWorkload):
        self.dw = dw
        w, dev = dw.w, dw.device
        dt = torch_dtype(w)
        T, T_in, D = w.T, w.T_in, w.dims.D
        self.s = torch.empty(T_in, dtype=torch.float32, device=dev)
        self.kept = torch.empty(T, dtype=torch.int32, device=dev)
        self.status = torch.empty(w.B, dtype=torch.int32, device=dev)
        self.x = torch.empty((T, D), dtype=dt, device=dev)
        self.pos_c = torch.empty(T, dtype=torch.int32, device=dev)
        self.s_c = torch.empty(T, dtype=torch.float32, device=dev)
        n = len(dw.layers)
        self.kcache = torch.empty((max(n, 1), T, w.dims.Hkv, w.dims.d), dtype=dt, device=dev)
        self.vcache = torch.empty_like(self.kcache)
        lib = tg.lib()
        need = lib.tg_upper_layer_workspace_size(tg.ctypes.byref(dw.dims), T, w.B, w.max_k)
        need = max(need, lib.tg_gate_score_workspace_size(T_in, D, w.dims.H1, tg.dtype_code(dt)))
        need = max(need, lib.tg_topk_select_workspace_size(w.B, T_in, w.max_n))
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def score(self):
        d = self.dw
        tg.gate_score(d.h, d.W1, d.b1, d.w2, d.b2, s_out=self.s, ws=self.ws)

    def select(self):
        d = self.dw
        tg.topk_select(self.s, d.keep_mask, d.cu_in, d.cu_kept, d.w.T, d.w.max_n,
                       kept=self.kept, status=self.status, ws=self.ws)

    def compact(self):
        d = self.dw
        tg.compact(d.h, None, self.s, self.kept, d.cu_in, d.cu_kept,
                   h_out=self.x, pos_out=self.pos_c, s_out=self.s_c)

    def select_compact(self):
        """Selection and compaction in one pass (tg_select_compact): the same
        outputs as select() then compact(), as the whole-step call runs them."""
        d = self.dw
        tg.select_compact(self.s, d.keep_mask, d.cu_in, d.cu_kept, d.w.T, d.w.max_n, d.h,
                          kept=self.kept, status=self.status, h_out=self.x, pos_out=self.pos_c,
                          s_out=self.s_c, ws=self.ws)

    def layer(self, l: int):
        d = self.dw
        # layers after the first reuse the RoPE table the first one left in the
        # workspace and, with folded norms, the row sums of squares of their input
        # that the previous layer's down projection wrote there
        tg.upper_layer_fwd(d.layers[l], d.dims, self.x, self.pos_c, self.s_c, d.cu_kept, d.w.max_k,
                           x_out=self.x, kcache=self.kcache[l], vcache=self.vcache[l], ws=self.ws,
                           rope_ready=l > 0, norms_folded=d.norms_folded,
                           input_ssq=d.norms_folded and l > 0)

    def run(self):
        """One step in one native call (tg_gated_prefill): the same kernels as
        score(), select_compact() and layer(l) for every l, in that order."""
        d = self.dw
        tg.gated_prefill(d.h, d.keep_mask, d.cu_in, d.cu_kept, d.w.T, d.w.max_n, d.w.max_k,
                         d.W1, d.b1, d.w2, d.b2, d.layers, d.dims, self.s, self.kept, self.status,
                         self.x, self.pos_c, self.s_c, self.kcache, self.vcache, ws=self.ws,
                         norms_folded=d.norms_folded)
        return self.x


def local_positions(cu_in: np.ndarray) -> np.ndarray:
    """Each token's index inside its own sequence (the positions of a plain prompt)."""
    cu_in = np.asarray(cu_in, dtype=np.int64)
    parts = [np.arange(int(cu_in[b + 1] - cu_in[b]), dtype=np.int32) for b in range(len(cu_in) - 1)]
    return np.concatenate(parts) if parts else np.zeros(0, np.int32)


class FullPrefill:
    """The three-stage prefill with the gate at layer L = ``n_below`` (Tencent
    Cloud TokenGate article, early token filtering; farwalk.ai summary, the
    method): ``dw.layers[:n_below]`` below the gate, ``dw.layers[n_below]``
    the gate layer, the rest above it. Preallocated buffers, one native call
    per step (tg_full_prefill)."""

    def __init__(self, dw: DeviceWorkload, n_below: int = 1):
        self.dw = dw
        w, dev = dw.w, dw.device
        dt = torch_dtype(w)
        dm = w.dims
        T, T_in, D = w.T, w.T_in, dm.D
        self.n_below = n_below
        self.below = dw.layers[:n_below]
        self.gate_layer = dw.layers[n_below]
        self.above = dw.layers[n_below + 1:]
        gi_cu = dw.cu_in.cpu().numpy()
        self.pos = torch.from_numpy(local_positions(gi_cu)).to(dev)
        self.s = torch.empty(T_in, dtype=torch.float32, device=dev)
        self.kept = torch.empty(T, dtype=torch.int32, device=dev)
        self.status = torch.empty(w.B, dtype=torch.int32, device=dev)
        self.x_full = torch.empty((T_in, D), dtype=dt, device=dev)
        self.kcache_full = torch.empty((n_below + 1, T_in, dm.Hkv, dm.d), dtype=dt, device=dev)
        self.vcache_full = torch.empty_like(self.kcache_full)
        self.x = torch.empty((T, D), dtype=dt, device=dev)
        self.pos_c = torch.empty(T, dtype=torch.int32, device=dev)
        self.s_c = torch.empty(T, dtype=torch.float32, device=dev)
        na = max(len(self.above), 1)
        self.kcache = torch.empty((na, T, dm.Hkv, dm.d), dtype=dt, device=dev)
        self.vcache = torch.empty_like(self.kcache)
        dims = dw.dims
        if dw.norms_folded:
            dims = tg.LayerDims(*[getattr(dims, f) for f, _ in tg.LayerDims._fields_])
            dims.flags |= tg.LAYER_NORMS_FOLDED
        need = tg.lib().tg_full_prefill_workspace_size(tg.ctypes.byref(dims), dm.H1, T_in, T, w.B,
                                                        w.max_n, w.max_k)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def run(self):
        d = self.dw
        w = d.w
        tg.full_prefill(d.h, self.pos, d.keep_mask, d.cu_in, d.cu_kept, w.T, w.max_n, w.max_k,
                        d.W1, d.b1, d.w2, d.b2, self.below, self.gate_layer, self.above, d.dims,
                        self.x_full, self.kcache_full, self.vcache_full, self.s, self.kept,
                        self.status, self.x, self.pos_c, self.s_c, self.kcache, self.vcache,
                        ws=self.ws, norms_folded=d.norms_folded)
        return self.x


def plain_attention_layer(L: tg.UpperLayerWeights, Hq: int, device) -> tg.UpperLayerWeights:
    """The same layer with t = 1 and g = 0: plain causal attention."""
    t = dict(L.tensors)
    t["t"] = torch.ones(Hq, dtype=torch.float32, device=device)
    t["g"] = torch.zeros(Hq, dtype=torch.float32, device=device)
    return tg.UpperLayerWeights(t)


class UnprunedPrefill:
    """The same model without the gate, the baseline of the prefill-time and
    memory comparisons (Tencent Cloud TokenGate article, section on token
    pruning lowering the prefill cost; ai.866data.com article, benchmark
    results): every layer of ``dw.layers`` on every prompt token with
    plain causal attention and the full prompt's K/V in every layer, one
    native call (tg_upper_layer_stack_fwd) on a copy of the input rows."""

    def __init__(self, dw: DeviceWorkload):
        self.dw = dw
        w, dev = dw.w, dw.device
        dt = torch_dtype(w)
        dm = w.dims
        self.layers = [plain_attention_layer(L, dm.Hq, dev) for L in dw.layers]
        self.pos = torch.from_numpy(local_positions(dw.cu_in.cpu().numpy())).to(dev)
        self.s0 = torch.zeros(w.T_in, dtype=torch.float32, device=dev)
        self.x = torch.empty((w.T_in, dm.D), dtype=dt, device=dev)
        n = max(len(self.layers), 1)
        self.kcache = torch.empty((n, w.T_in, dm.Hkv, dm.d), dtype=dt, device=dev)
        self.vcache = torch.empty_like(self.kcache)
        dims = dw.dims
        if dw.norms_folded:
            dims = tg.LayerDims(*[getattr(dims, f) for f, _ in tg.LayerDims._fields_])
            dims.flags |= tg.LAYER_NORMS_FOLDED
        need = tg.lib().tg_upper_layer_workspace_size(tg.ctypes.byref(dims), w.T_in, w.B, w.max_n)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def run(self):
        d = self.dw
        self.x.copy_(d.h)
        tg.upper_layer_stack_fwd(self.layers, d.dims, self.x, self.pos, self.s0, d.cu_in, d.w.max_n,
                                 self.kcache, self.vcache, ws=self.ws, norms_folded=d.norms_folded)
        return self.x
