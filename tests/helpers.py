"""Shared helpers of the GPU parity tests (no method arithmetic here)."""
import sys

import numpy as np
import torch

# tolerances: bf16 inputs with fp32 accumulation / fp32 end to end
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.detach().cpu().view(torch.int16).numpy()
    return t.detach().cpu().view(torch.int32).numpy()


def assert_close(got, ref, dtype: str, what: str):
    atol, rtol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    lim = atol + rtol * np.abs(ref)
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError("%s: %d/%d outside atol=%g rtol=%g; worst at %s got %r ref %r"
                             % (what, int(bad.sum()), bad.size, atol, rtol, i, got[i], ref[i]))
    return float(err.max()) if err.size else 0.0


def ws_view(ws: torch.Tensor, off: int, shape, dtype: torch.dtype) -> torch.Tensor:
    n = int(np.prod(shape))
    nbytes = n * torch.tensor([], dtype=dtype).element_size()
    return ws[off:off + nbytes].view(dtype).reshape(shape)


def layer_dict(lw) -> dict:
    """Host layer weights (exact fp32 values) as the oracle's dict."""
    return {"wq": lw.wq.value, "wk": lw.wk.value, "wv": lw.wv.value, "wo": lw.wo.value,
            "wg": lw.wg.value, "wu": lw.wu.value, "wd": lw.wd.value,
            "attn_norm": lw.attn_norm.value, "ffn_norm": lw.ffn_norm.value,
            "t": lw.t, "g": lw.g}


def sample_rows(cu, per_seq: int, seed: int):
    """Rows to check in each sequence: first, last, a ragged boundary and random ones."""
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(len(cu) - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi <= lo:
            continue
        n = hi - lo
        cand = {lo, hi - 1, lo + min(n - 1, 63), lo + min(n - 1, 64)}
        cand.update((lo + rng.choice(n, size=min(n, per_seq), replace=False)).tolist())
        rows.extend(sorted(cand))
    return np.asarray(rows, dtype=np.int64)
