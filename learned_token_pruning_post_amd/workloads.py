"""Seeded synthetic workloads for the TokenGate gated-prefill path.

This module only draws inputs. It holds none of the method's arithmetic, so
both the HIP path and the CPU oracle can consume exactly the same values:
every tensor is drawn in fp32 from ``numpy.random.default_rng([cfg_id,
ordinal])`` and, for bf16 workloads, rounded to bf16 (round to nearest even)
before either side sees it. The fp32 array returned next to the bf16 bits is
the exact value of those bits.

Shapes follow the Qwen3-1.7B-shaped layer named by the pages (Token-Gated
Language Models, Tencent Cloud article, section on early token filtering:
Qwen3-1.7B with the gate at layer 1) and the long-context lengths they report
(16K training, 32K/64K/128K extrapolation; same article, section on prefill
cost). The pages' datasets are not used: hidden states are Gaussian with a
small fraction of "salient" rows scaled up, and the unprunable
question/instruction tokens are a tail of each sequence.

Tensor ordinals (the second seed word):
  0 hidden states h, 1 salient-row choice, 2 W1, 3 b1, 4 w2, 5 b2,
  8 per-sequence budgets (multi-budget batch only),
  100 + 16*l + {0 wq, 1 wk, 2 wv, 3 wo, 4 wg, 5 wu, 6 wd, 7 t, 8 g} for
  upper layer l.
Norm weights are ones and are not drawn.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np


@dataclass(frozen=True)
class ModelDims:
    D: int          # hidden size
    Hq: int         # query heads
    Hkv: int        # key/value heads
    d: int          # head dim
    I: int          # SwiGLU intermediate size
    H1: int         # gate-scorer hidden size
    dtype: str      # "bf16" or "f32": storage/compute type of activations and weights
    rope_base: float = 1.0e6
    rms_eps: float = 1.0e-6


QWEN3_1P7B = ModelDims(D=2048, Hq=16, Hkv=8, d=128, I=6144, H1=256, dtype="bf16")
TINY = ModelDims(D=256, Hq=4, Hkv=2, d=64, I=512, H1=64, dtype="f32")


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    N: tuple            # tokens per sequence
    K: tuple            # kept budget per sequence (forced tokens included)
    F: int              # unprunable tail tokens per sequence
    dims: ModelDims
    layers: int         # upper layers on the timed path
    salient: bool       # 5% of rows scaled x4

    @property
    def B(self) -> int:
        return len(self.N)

    @property
    def T_in(self) -> int:
        return int(sum(self.N))

    @property
    def T(self) -> int:
        return int(sum(self.K))

    @property
    def max_n(self) -> int:
        return int(max(self.N))

    @property
    def max_k(self) -> int:
        return int(max(self.K))


def _budgets_multi(cfg_id: int, B: int, N: int) -> tuple:
    rng = np.random.default_rng([cfg_id, 8])
    small = rng.integers(256, 4096, size=B - 1, endpoint=True)
    return (N,) + tuple(int(x) for x in small)


def workload(name: str, k: Optional[int] = None, n: Optional[int] = None,
             layers: Optional[int] = None) -> Workload:
    """Named presets. ``k``/``n``/``layers`` override where the preset allows."""
    if name == "tiny":
        w = Workload("tiny", 1, (512,), (128,), 32, TINY, 1, False)
    elif name == "qwen8k":
        w = Workload("qwen8k", 2, (8192,), (1024,), 256, QWEN3_1P7B, 1, True)
    elif name == "qwen32k":
        kk = 4096 if k is None else k
        w = Workload("qwen32k", 3, (32768,), (kk,), 512, QWEN3_1P7B, 27, True)
    elif name == "long":
        nn = 65536 if n is None else n
        w = Workload("long", 4, (nn,), (4096,), 512, QWEN3_1P7B, 1, True)
    elif name == "multibudget":
        w = Workload("multibudget", 5, (16384,) * 8, _budgets_multi(5, 8, 16384),
                     256, QWEN3_1P7B, 1, True)
    else:
        raise KeyError(name)
    if k is not None and name not in ("qwen32k",):
        w = Workload(w.name, w.cfg_id, w.N, tuple(k for _ in w.N), w.F, w.dims, w.layers, w.salient)
    if n is not None and name != "long":
        w = Workload(w.name, w.cfg_id, tuple(n for _ in w.N), w.K, w.F, w.dims, w.layers, w.salient)
    if layers is not None:
        w = Workload(w.name, w.cfg_id, w.N, w.K, w.F, w.dims, layers, w.salient)
    return w


def custom(cfg_id: int, N, K, F: int, dims: ModelDims, layers: int = 1,
           salient: bool = False, name: str = "custom") -> Workload:
    """An ad-hoc workload (used by tests for ragged and edge-case shapes)."""
    return Workload(name, cfg_id, tuple(int(x) for x in N), tuple(int(x) for x in K),
                    int(F), dims, layers, salient)


# ----------------------------------------------------------------------------
# bf16 storage helpers (pure representation changes, no model arithmetic)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns as fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Tensor:
    """One generated tensor: exact fp32 values plus the bits the device stores."""
    value: np.ndarray                 # float32, exact value of what the device sees
    bits: Optional[np.ndarray] = None  # uint16 bf16 bits (bf16 workloads) or None (fp32)

    @property
    def device_array(self) -> np.ndarray:
        return self.value if self.bits is None else self.bits


def _draw(cfg_id: int, ordinal: int, shape, scale: float, dtype: str) -> Tensor:
    rng = np.random.default_rng([cfg_id, ordinal])
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        v *= np.float32(scale)
    return _finish(v, dtype)


def _finish(v: np.ndarray, dtype: str) -> Tensor:
    if dtype == "bf16":
        bits = f32_to_bf16_bits(v)
        return Tensor(bf16_bits_to_f32(bits), bits)
    return Tensor(np.ascontiguousarray(v, dtype=np.float32), None)


@dataclass
class GateInputs:
    h: Tensor                 # [T_in, D]
    W1: Tensor                # [H1, D]
    b1: Tensor                # [H1]
    w2: Tensor                # [H1]
    b2: Tensor                # [1]
    keep_mask: np.ndarray     # [T_in] uint8
    cu_in: np.ndarray         # [B+1] int32
    cu_kept: np.ndarray       # [B+1] int32
    pos: np.ndarray           # [T_in] int32, original position of each token


@dataclass
class LayerWeights:
    wq: Tensor   # [Hq*d, D]
    wk: Tensor   # [Hkv*d, D]
    wv: Tensor   # [Hkv*d, D]
    wo: Tensor   # [D, Hq*d]
    wg: Tensor   # [I, D]
    wu: Tensor   # [I, D]
    wd: Tensor   # [D, I]
    attn_norm: Tensor  # [D] ones
    ffn_norm: Tensor   # [D] ones
    t: np.ndarray      # [Hq] fp32, per-head temperature
    g: np.ndarray      # [Hq] fp32, per-head gain


def gate_inputs(w: Workload) -> GateInputs:
    dm = w.dims
    T_in = w.T_in
    rng_h = np.random.default_rng([w.cfg_id, 0])
    h = rng_h.standard_normal(size=(T_in, dm.D), dtype=np.float32)
    cu_in = np.zeros(w.B + 1, dtype=np.int32)
    cu_in[1:] = np.cumsum(np.asarray(w.N, dtype=np.int64)).astype(np.int32)
    if w.salient:
        rng_s = np.random.default_rng([w.cfg_id, 1])
        for b in range(w.B):
            nb = w.N[b]
            cnt = int(np.floor(0.05 * nb))
            if cnt:
                rows = rng_s.choice(nb, size=cnt, replace=False) + cu_in[b]
                h[rows] *= np.float32(4.0)
    ht = _finish(h, dm.dtype)
    W1 = _draw(w.cfg_id, 2, (dm.H1, dm.D), 0.02, dm.dtype)
    b1 = _draw(w.cfg_id, 3, (dm.H1,), 0.02, dm.dtype)
    w2 = _draw(w.cfg_id, 4, (dm.H1,), 0.02, dm.dtype)
    b2 = _draw(w.cfg_id, 5, (1,), 0.02, dm.dtype)
    keep = np.zeros(T_in, dtype=np.uint8)
    for b in range(w.B):
        e = int(cu_in[b + 1])
        keep[max(int(cu_in[b]), e - w.F):e] = 1
    cu_kept = np.zeros(w.B + 1, dtype=np.int32)
    cu_kept[1:] = np.cumsum(np.asarray(w.K, dtype=np.int64)).astype(np.int32)
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in w.N]) if T_in else np.zeros(0, np.int32)
    return GateInputs(ht, W1, b1, w2, b2, keep, cu_in, cu_kept, pos)


def layer_weights(w: Workload, layer: int) -> LayerWeights:
    dm = w.dims
    base = 100 + 16 * layer
    c = w.cfg_id
    wq = _draw(c, base + 0, (dm.Hq * dm.d, dm.D), 0.02, dm.dtype)
    wk = _draw(c, base + 1, (dm.Hkv * dm.d, dm.D), 0.02, dm.dtype)
    wv = _draw(c, base + 2, (dm.Hkv * dm.d, dm.D), 0.02, dm.dtype)
    wo = _draw(c, base + 3, (dm.D, dm.Hq * dm.d), 0.02, dm.dtype)
    wg = _draw(c, base + 4, (dm.I, dm.D), 0.02, dm.dtype)
    wu = _draw(c, base + 5, (dm.I, dm.D), 0.02, dm.dtype)
    wd = _draw(c, base + 6, (dm.D, dm.I), 0.02, dm.dtype)
    ones = _finish(np.ones(dm.D, dtype=np.float32), dm.dtype)
    t = np.random.default_rng([c, base + 7]).uniform(0.8, 1.2, size=dm.Hq).astype(np.float32)
    g = np.random.default_rng([c, base + 8]).uniform(0.0, 2.0, size=dm.Hq).astype(np.float32)
    return LayerWeights(wq, wk, wv, wo, wg, wu, wd, ones, ones, t, g)


def activations(cfg_id: int, ordinal: int, shape, dtype: str, scale: float = 1.0) -> Tensor:
    """A free-standing N(0, scale^2) activation tensor (q/k/v or layer input for stage tests)."""
    return _draw(cfg_id, ordinal, shape, scale, dtype)


def scores_with_ties(cfg_id: int, T_in: int, n_distinct: int) -> np.ndarray:
    """fp32 scores in (0, 1) drawn from only ``n_distinct`` values: exercises tie-breaks."""
    rng = np.random.default_rng([cfg_id, 50])
    vals = rng.uniform(0.3, 0.7, size=max(1, n_distinct)).astype(np.float32)
    return vals[rng.integers(0, len(vals), size=T_in)]
