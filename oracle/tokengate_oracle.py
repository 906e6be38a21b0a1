"""CPU oracle for the TokenGate gated-prefill path (test infrastructure only).

This module is the slow, plain, float64 statement of what the gated prefill
path computes. It exists to check the HIP library, and only the tests, the
smoke check and the CPU-baseline leg of the benchmark may import it. It shares
no code with the HIP path and imports nothing from the package.

Sources (five web pages about "Token-Gated Language Models", cited by page and
section):
  [TC]  Tencent Cloud developer article on TokenGate (Chinese): sections
        "TokenGate 提前筛选 Token" (early token filtering),
        "门控机制为评分网络建立梯度路径" (the gate gives the scorer a gradient path),
        "选择器与模型主干共同适应剪枝" (selector and backbone co-adapt),
        "TokenGate 的工程验证仍有限" (engineering validation is limited).
  [FW]  farwalk.ai news summary: section "论文的方法" (the method).
  [HF]  Hugging Face paper-page mirror: the abstract.
  [AI]  ai.866data.com article: section "可学习剪枝的机制设计" (mechanism design).

What the pages leave open is fixed by the specification of this project and
stated at each function: the logit form L = t_h * q.k / sqrt(d) + g_h * s_j,
an erf-GELU / sigmoid two-layer scorer with biases, forced tokens counted
inside the budget K, lowest-index tie-break, rotate-half RoPE at the tokens'
original positions (base 1e6), RMSNorm with eps 1e-6, contiguous GQA groups.

Every function here has pins in the CPU test suite (closed forms, brute force
on tiny inputs, reductions to library routines and invariants). The only part
with no pin beyond its own definition is fidelity to the authors' unpublished
implementation: parity unpinned for that, since no code or worked numbers are
published.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np
from scipy.special import erf as _erf

# Device status flags (mirrors of the library's documented values; the oracle
# reports the same conditions for the same inputs).
FORCED_GT_BUDGET = 1
BUDGET_GT_LEN = 2
NAN_SCORE = 4


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------
# Gate scorer
# ----------------------------------------------------------------------------

def gelu(z):
    """Exact (erf) GELU: z * Phi(z) = z/2 * (1 + erf(z / sqrt 2)).

    The pages call the scorer a lightweight MLP ([AI] mechanism design;
    [TC] early token filtering); its hidden activation is GELU by the
    project's specification, in the exact erf form.
    """
    z = _f64(z)
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def sigmoid(u):
    """Logistic function 1 / (1 + exp(-u)); maps the scorer logit into (0, 1)."""
    u = _f64(u)
    return 1.0 / (1.0 + np.exp(-u))


def gate_score(h, W1, b1, w2, b2) -> np.ndarray:
    """Importance score of every token from its post-attention residual at layer L.

    [TC] early token filtering and [AI] mechanism design: after layer L's
    attention, a small MLP reads each token's current representation and
    emits an importance score. Form: s = sigmoid(w2 . GELU(W1 h + b1) + b2),
    W1 in nn.Linear layout [H1, D]. No normalisation precedes the scorer.
    """
    h = _f64(h)
    z = h @ _f64(W1).T + _f64(b1)[None, :]
    u = gelu(z) @ _f64(w2) + float(_f64(b2).reshape(-1)[0])
    return sigmoid(u)


# ----------------------------------------------------------------------------
# Top-K selection with forced keep
# ----------------------------------------------------------------------------

def _canon(s: np.ndarray) -> np.ndarray:
    """Scores as float64 with -0.0 folded onto +0.0 (they compare equal)."""
    s = _f64(s).copy()
    s[s == 0.0] = 0.0
    return s


def select_one(s, forced, K: int):
    """Kept local indices (ascending) of one sequence, and its status flags.

    [TC] early token filtering: a Top-K selector keeps K of the N tokens and
    designated tokens such as the user's question are never pruned; [AI]
    mechanism design: only the document body may be pruned. Reading fixed by
    the specification: the forced tokens count inside K, the remaining
    K - |F| slots go to the highest scores among the others, equal scores are
    broken by the lower index, NaN ranks below every number.
    """
    s = _canon(s)
    forced = np.asarray(forced, dtype=bool)
    n = s.shape[0]
    flags = 0
    if np.isnan(s).any():
        flags |= NAN_SCORE
    nf = int(forced.sum())
    if K > n:
        flags |= BUDGET_GT_LEN
    if nf > K:
        flags |= FORCED_GT_BUDGET
    if flags & (BUDGET_GT_LEN | FORCED_GT_BUDGET):
        return None, flags
    r = K - nf
    cand = np.flatnonzero(~forced)
    cs = s[cand]
    isn = np.isnan(cs)
    neg = np.where(isn, 0.0, -cs)
    # lexsort: last key is primary -> (isnan, -s, index)
    order = np.lexsort((cand, neg, isn))
    chosen = cand[order[:r]]
    kept = np.sort(np.concatenate([np.flatnonzero(forced), chosen]))
    return kept.astype(np.int64), flags


def topk_select(s, keep_mask, cu_in, cu_kept):
    """Per-sequence selection over a packed batch.

    Returns (kept_idx [T] int64 global indices, ascending within each
    sequence and laid out at cu_kept offsets; flags [B] int). Sequences with
    an error flag leave their slots at -1.
    """
    s = np.asarray(s)
    cu_in = np.asarray(cu_in, dtype=np.int64)
    cu_kept = np.asarray(cu_kept, dtype=np.int64)
    B = len(cu_in) - 1
    mask = np.zeros(s.shape[0], dtype=bool) if keep_mask is None else np.asarray(keep_mask).astype(bool)
    out = np.full(int(cu_kept[-1]), -1, dtype=np.int64)
    flags = np.zeros(B, dtype=np.int64)
    for b in range(B):
        lo, hi = int(cu_in[b]), int(cu_in[b + 1])
        K = int(cu_kept[b + 1] - cu_kept[b])
        kept, f = select_one(s[lo:hi], mask[lo:hi], K)
        flags[b] = f
        if kept is not None:
            out[int(cu_kept[b]):int(cu_kept[b + 1])] = kept + lo
    return out, flags


# ----------------------------------------------------------------------------
# Compaction
# ----------------------------------------------------------------------------

def compact(h, pos, s, kept_idx, cu_in, cu_kept):
    """Gather kept rows, their original positions and their scores.

    [TC] early token filtering: only the selected tokens continue into layer
    L's FFN and the layers above; [FW] the method: above the gate only the K
    kept tokens are processed. ``pos`` None means each token's position is its
    index inside its own sequence.
    """
    kept = np.asarray(kept_idx, dtype=np.int64)
    h = np.asarray(h)
    s = np.asarray(s)
    if pos is None:
        cu_in = np.asarray(cu_in, dtype=np.int64)
        cu_kept = np.asarray(cu_kept, dtype=np.int64)
        pos_c = np.empty(kept.shape[0], dtype=np.int64)
        for b in range(len(cu_in) - 1):
            sl = slice(int(cu_kept[b]), int(cu_kept[b + 1]))
            pos_c[sl] = kept[sl] - cu_in[b]
    else:
        pos_c = np.asarray(pos, dtype=np.int64)[kept]
    return h[kept], pos_c, s[kept]


# ----------------------------------------------------------------------------
# Upper-layer pieces
# ----------------------------------------------------------------------------

def rmsnorm(x, w, eps: float):
    """x / sqrt(mean(x^2) + eps) * w, per row (pre-norm of a Qwen3-style layer)."""
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _f64(w)


def rope(x, pos, base: float):
    """Rotate-half rotary embedding at the given positions.

    x: [T, H, d]; pos: [T]. For i < d/2, theta_i = pos * base^(-2i/d);
    x'_i = x_i cos - x_{i+d/2} sin, x'_{i+d/2} = x_{i+d/2} cos + x_i sin.
    Kept tokens keep their original positions (specification reading: the
    pages do not say; the original position is the only one under which a
    kept token's relative offsets are unchanged).
    """
    x = _f64(x)
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    inv = base ** (-2.0 * i / d)
    theta = _f64(pos)[:, None] * inv[None, :]          # [T, d/2]
    c = np.cos(theta)[:, None, :]
    sn = np.sin(theta)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * sn, b * c + a * sn], axis=-1)


def gated_attention(q, k, v, s_c, t, g, cu_kept, rows: Optional[Sequence[int]] = None,
                    chunk: int = 512):
    """Token-gated causal GQA attention over the kept tokens.

    [TC] gradient-path section: the selected tokens' scores keep entering the
    upper layers' attention and shape its weights, with a per-head learnable
    gain and temperature; [TC] engineering section: the score enters as a
    bias on the attention logit of each key; [AI] mechanism design: a bias on
    the logits above the gate layer. Logit (specification):
        L_ij = t_h * (q_i,h . k_j,h') / sqrt(d) + g_h * s_c[j],  j <= i,
    h' = h // (Hq / Hkv); P = softmax_j L; o_i = sum_j P_ij v_j. Causality is
    within each sequence of the packed batch, in compacted (= ascending
    position) order.

    Returns (o [T, Hq, d], lse [Hq, T] natural-log log-sum-exp). With
    ``rows`` only those global rows are computed (others stay zero).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    s_c, t, g = _f64(s_c), _f64(t), _f64(g)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    o = np.zeros((T, Hq, d))
    lse = np.zeros((Hq, T))
    cu = np.asarray(cu_kept, dtype=np.int64)
    want = None if rows is None else np.asarray(sorted(set(int(r) for r in rows)), dtype=np.int64)
    scale = 1.0 / math.sqrt(d)
    for b in range(len(cu) - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi <= lo:
            continue
        if want is None:
            rs = np.arange(lo, hi)
        else:
            rs = want[(want >= lo) & (want < hi)]
        if rs.size == 0:
            continue
        for h in range(Hq):
            hk = h // grp
            kk = k[lo:hi, hk, :]
            vv = v[lo:hi, hk, :]
            for c0 in range(0, rs.size, chunk):
                rr = rs[c0:c0 + chunk]
                logits = t[h] * (q[rr, h, :] @ kk.T) * scale + g[h] * s_c[lo:hi][None, :]
                jj = np.arange(lo, hi)[None, :]
                logits = np.where(jj <= rr[:, None], logits, -np.inf)
                m = logits.max(axis=1, keepdims=True)
                p = np.exp(logits - m)
                den = p.sum(axis=1, keepdims=True)
                o[rr, h, :] = (p @ vv) / den
                lse[h, rr] = (m + np.log(den))[:, 0]
    return o, lse


def decode_attention(q, kA, vA, sA, cuA, kB, vB, sB, lenB, t, g):
    """One new token per sequence attending to its pruned K/V cache.

    [TC] engineering section: once prefill has fixed the gate bias, decoding
    can fold it into the attention mask and run ordinary attention over the
    cache; [TC] early token filtering: tokens generated while decoding are
    never gated out, so each one joins the cache. The keys of sequence b are
    its kept prompt tokens (rows cuA[b] .. cuA[b+1]-1 of kA / vA, scores sA)
    followed by its first lenB[b] generated tokens (rows 0 .. lenB[b]-1 of
    kB[b] / vB[b], scores sB[b]); every one of them precedes the query, so
    there is no causal mask. Same logit as the prefill's gated attention:
        L_j = t_h * (q_h . k_j,h') / sqrt(d) + g_h * s_j,  h' = h // (Hq / Hkv).
    q: [B, Hq, d]; kA, vA: [rows, Hkv, d]; kB, vB: [B, cap, Hkv, d];
    sB: [B, cap]. Returns o [B, Hq, d] and lse [B, Hq] (natural log); a
    sequence with no keys gives o = 0 and lse = -inf.
    """
    q = _f64(q)
    kA, vA, sA = _f64(kA), _f64(vA), _f64(sA)
    kB, vB, sB = _f64(kB), _f64(vB), _f64(sB)
    t, g = _f64(t), _f64(g)
    B, Hq, d = q.shape
    Hkv = kA.shape[1] if kA.ndim == 3 else kB.shape[2]
    grp = Hq // Hkv
    cuA = np.asarray(cuA, dtype=np.int64)
    lenB = np.asarray(lenB, dtype=np.int64)
    o = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        a0, a1 = int(cuA[b]), int(cuA[b + 1])
        nb = int(lenB[b])
        keys = np.concatenate([kA[a0:a1], kB[b, :nb]], axis=0)      # [L, Hkv, d]
        vals = np.concatenate([vA[a0:a1], vB[b, :nb]], axis=0)
        s = np.concatenate([sA[a0:a1], sB[b, :nb]])
        if keys.shape[0] == 0:
            continue
        for h in range(Hq):
            hk = h // grp
            logits = t[h] * (keys[:, hk, :] @ q[b, h]) / math.sqrt(d) + g[h] * s
            m = logits.max()
            p = np.exp(logits - m)
            den = p.sum()
            o[b, h] = (p @ vals[:, hk, :]) / den
            lse[b, h] = m + math.log(den)
    return o, lse


# ----------------------------------------------------------------------------
# Hybrid variant: the Gated DeltaNet token mixer on the kept tokens
# ----------------------------------------------------------------------------

def gdn_mixer(q, k, v, alpha, beta, cu, state_in=None, eps: float = 1e-6):
    """Gated DeltaNet recurrence over each sequence of a packed batch.

    [TC] section on the gate position: in a hybrid model (Qwen3.5-2B) only
    some layers use full attention and the rest are Gated DeltaNet; the
    scorer reads hidden states, so the gate can sit on a GDN layer, and a GDN
    layer above the gate has no attention logits to bias, so it simply runs
    on the kept tokens. The recurrence (the Gated DeltaNet layer's, per head,
    state S [dv, dk], zero or ``state_in`` at a sequence's start):
        k^ = k / |k|, q^ = q / (|q| sqrt(dk))
        S <- alpha_t S;  S <- S + beta_t (v_t - S k^_t) k^_t^T;  o_t = S q^_t
    i.e. S_t = alpha_t S_{t-1} (I - beta_t k^ k^T) + beta_t v_t k^T.
    q, k: [T, H, dk]; v: [T, H, dv]; alpha, beta: [T, H]; cu: [B+1].
    Returns (o [T, H, dv], state [B, H, dv, dk] after each sequence's last token).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, beta = _f64(alpha), _f64(beta)
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = np.asarray(cu, dtype=np.int64)
    B = len(cu) - 1
    o = np.zeros((T, H, dv))
    state = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk)) if state_in is None else _f64(state_in)[b, h].copy()
            for tt in range(int(cu[b]), int(cu[b + 1])):
                kh = k[tt, h] / math.sqrt(float(k[tt, h] @ k[tt, h]) + eps)
                qh = q[tt, h] / (math.sqrt(float(q[tt, h] @ q[tt, h]) + eps) * math.sqrt(dk))
                S = alpha[tt, h] * S
                S = S + beta[tt, h] * np.outer(v[tt, h] - S @ kh, kh)
                o[tt, h] = S @ qh
            state[b, h] = S
    return o, state


# ----------------------------------------------------------------------------
# Backward: the gradient path from the upper attention to the scorer
# ----------------------------------------------------------------------------

def gated_attention_backward(q, k, v, s_c, t, g, cu_kept, do):
    """Gradients of the token-gated attention with respect to q, k, v, the
    kept tokens' scores and the per-head temperature and gain.

    [TC] gradient-path section: because the scores enter the upper layers'
    attention logits, the loss reaches the scorer through them, and the
    per-head gain and temperature are learned with it. With the forward of
    gated_attention (L_ij = t_h q_i.k_j / sqrt(d) + g_h s_j for j <= i,
    P = softmax_j L, o_i = sum_j P_ij v_j) and an upstream gradient dO:
        dv_j   = sum_i P_ij dO_i
        dP_ij  = dO_i . v_j
        dL_ij  = P_ij (dP_ij - sum_k P_ik dP_ik)      (softmax Jacobian)
        dq_i   = t_h / sqrt(d) sum_j dL_ij k_j
        dk_j   = t_h / sqrt(d) sum_i dL_ij q_i
        ds_j   = sum_h g_h sum_i dL_ij
        dg_h   = sum_ij dL_ij s_j,   dt_h = sum_ij dL_ij q_i.k_j / sqrt(d)
    For GQA, dk and dv of a kv head add up over the query heads of its group.
    Returns {"dq" [T,Hq,d], "dk" [T,Hkv,d], "dv" [T,Hkv,d], "ds" [T], "dt" [Hq], "dg" [Hq]}.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    s_c, t, g = _f64(s_c), _f64(t), _f64(g)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    ds, dt, dg = np.zeros(T), np.zeros(Hq), np.zeros(Hq)
    cu = np.asarray(cu_kept, dtype=np.int64)
    rd = 1.0 / math.sqrt(d)
    for b in range(len(cu) - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        n = hi - lo
        if n <= 0:
            continue
        causal = np.tril(np.ones((n, n), dtype=bool))
        for h in range(Hq):
            hk = h // grp
            qq, kk, vv, dd = q[lo:hi, h], k[lo:hi, hk], v[lo:hi, hk], do[lo:hi, h]
            qk = qq @ kk.T * rd
            L = np.where(causal, t[h] * qk + g[h] * s_c[lo:hi][None, :], -np.inf)
            P = np.exp(L - L.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            dv[lo:hi, hk] += P.T @ dd
            dP = dd @ vv.T
            dL = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dq[lo:hi, h] = t[h] * rd * (dL @ kk)
            dk[lo:hi, hk] += t[h] * rd * (dL.T @ qq)
            ds[lo:hi] += g[h] * dL.sum(axis=0)
            dg[h] += float((dL * s_c[lo:hi][None, :]).sum())
            dt[h] += float((dL * qk).sum())
    return {"dq": dq, "dk": dk, "dv": dv, "ds": ds, "dt": dt, "dg": dg}


def gelu_grad(z):
    """d GELU(z) / dz = Phi(z) + z phi(z) for the exact (erf) GELU."""
    z = _f64(z)
    return 0.5 * (1.0 + _erf(z / math.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def gate_score_backward(h, W1, b1, w2, b2, ds):
    """Gradients of the scorer s = sigmoid(w2 . GELU(W1 h + b1) + b2) given ds
    per token ([TC] gradient-path section: the gate gives the scoring network
    a gradient path, so it trains with the model):
        z = W1 h + b1, a = GELU(z), u = w2.a + b2, s = sigmoid(u)
        du = ds s (1 - s);  dw2 = sum_t du_t a_t;  db2 = sum_t du_t
        dz = du w2 GELU'(z); dW1 = sum_t dz_t h_t^T; db1 = sum_t dz_t; dh = dz W1
    Returns {"dh" [T,D], "dW1" [H1,D], "db1" [H1], "dw2" [H1], "db2" scalar}.
    """
    h, W1, b1, w2 = _f64(h), _f64(W1), _f64(b1), _f64(w2)
    b2v = float(_f64(b2).reshape(-1)[0])
    ds = _f64(ds)
    z = h @ W1.T + b1[None, :]
    a = gelu(z)
    sv = sigmoid(a @ w2 + b2v)
    du = ds * sv * (1.0 - sv)
    dz = du[:, None] * w2[None, :] * gelu_grad(z)
    return {"dh": dz @ W1, "dW1": dz.T @ h, "db1": dz.sum(axis=0), "dw2": a.T @ du,
            "db2": float(du.sum())}


def compact_backward(ds_c, kept_idx, T_in):
    """Gradient of the prompt scores through the compaction: compacted row r
    is prompt row kept_idx[r], so it carries ds_c[r] back there; a pruned
    token's score gets none ([TC] early token filtering: pruned tokens stop
    at layer L and never reach the layers whose attention reads the scores)."""
    ds = np.zeros(int(T_in))
    np.add.at(ds, np.asarray(kept_idx, dtype=np.int64), _f64(ds_c))
    return ds


def silu(x):
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def qkv_rope(x, pos_c, W: Dict[str, np.ndarray], dims, rows=None):
    """Pre-attention half of an upper layer: n1 = RMSNorm(x) * attn_norm;
    q, k, v = n1 Wq^T, n1 Wk^T, n1 Wv^T; RoPE on q and k at pos_c.
    Returns (n1, q [T,Hq,d], k [T,Hkv,d], v [T,Hkv,d]); with ``rows`` q is
    filled only there (k and v always for every token)."""
    x = _f64(x)
    T = x.shape[0]
    Hq, Hkv, d = dims.Hq, dims.Hkv, dims.d
    n1 = rmsnorm(x, W["attn_norm"], dims.rms_eps)
    k = rope((n1 @ _f64(W["wk"]).T).reshape(T, Hkv, d), pos_c, dims.rope_base)
    v = (n1 @ _f64(W["wv"]).T).reshape(T, Hkv, d)
    sel = np.arange(T) if rows is None else np.asarray(sorted(set(int(r) for r in rows)), dtype=np.int64)
    q = np.zeros((T, Hq, d))
    q[sel] = rope((n1[sel] @ _f64(W["wq"]).T).reshape(-1, Hq, d), _f64(pos_c)[sel], dims.rope_base)
    return n1, q, k, v


def o_proj(x, o, Wo):
    """Attention output projection with the residual: x1 = x + o_flat Wo^T."""
    o = _f64(o)
    return _f64(x) + o.reshape(o.shape[0], -1) @ _f64(Wo).T


def swiglu_act(x1, W: Dict[str, np.ndarray], eps: float):
    """n2 = RMSNorm(x1) * ffn_norm; act = silu(n2 Wg^T) * (n2 Wu^T). Returns (n2, act)."""
    n2 = rmsnorm(x1, W["ffn_norm"], eps)
    return n2, silu(n2 @ _f64(W["wg"]).T) * (n2 @ _f64(W["wu"]).T)


def down_proj(x1, act, Wd):
    """FFN down projection with the residual: x2 = x1 + act Wd^T."""
    return _f64(x1) + _f64(act) @ _f64(Wd).T


def upper_layer(x, pos_c, s_c, W: Dict[str, np.ndarray], dims, cu_kept,
                rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """One decoder layer above the gate, run on the kept tokens only.

    [TC] early token filtering: only kept tokens get the FFN and later layers,
    and no KV is made for pruned tokens. Layer (Qwen3-shaped, specification):
      n1 = RMSNorm(x) * attn_norm; q,k,v = n1 Wq^T, n1 Wk^T, n1 Wv^T;
      RoPE on q, k at pos_c; o = gated attention; x1 = x + o Wo^T;
      n2 = RMSNorm(x1) * ffn_norm; x2 = x1 + (silu(n2 Wg^T) * (n2 Wu^T)) Wd^T.
    W keys: wq wk wv wo wg wu wd attn_norm ffn_norm t g (float arrays).
    Returns every intermediate. With ``rows`` (global row ids) the k/v cache
    is computed for all tokens and the rest only for those rows.
    """
    x = _f64(x)
    T = x.shape[0]
    n1, q, k, v = qkv_rope(x, pos_c, W, dims, rows)
    sel = np.arange(T) if rows is None else np.asarray(sorted(set(int(r) for r in rows)), dtype=np.int64)
    o, lse = gated_attention(q, k, v, s_c, W["t"], W["g"], cu_kept,
                             rows=None if rows is None else sel)
    x1 = np.zeros_like(x)
    x1[sel] = o_proj(x[sel], o[sel], W["wo"])
    n2 = np.zeros_like(x)
    act = np.zeros((T, _f64(W["wg"]).shape[0]))
    n2[sel], act[sel] = swiglu_act(x1[sel], W, dims.rms_eps)
    x2 = np.zeros_like(x)
    x2[sel] = down_proj(x1[sel], act[sel], W["wd"])
    return {"n1": n1, "q": q, "k": k, "v": v, "o": o, "lse": lse, "rows": sel,
            "x1": x1, "n2": n2, "act": act, "x2": x2}


def attention_half(x, pos, s, W: Dict[str, np.ndarray], dims, cu, t=None, g=None):
    """The attention half of a decoder layer, up to the post-attention residual:
    n1 = RMSNorm(x) * attn_norm; q, k, v projections; RoPE at ``pos``;
    attention with temperature ``t`` and gain ``g`` (default: W's; pass
    t = 1, g = 0 for plain causal attention); x1 = x + o Wo^T.

    [TC] early token filtering and [AI] mechanism design: the gate scorer
    reads this residual of layer L, after its attention and before its FFN.
    Returns {"x1", "k", "v"}.
    """
    x = _f64(x)
    _, q, k, v = qkv_rope(x, pos, W, dims)
    tt = W["t"] if t is None else t
    gg = W["g"] if g is None else g
    o, _ = gated_attention(q, k, v, s, tt, gg, cu)
    return {"x1": o_proj(x, o, W["wo"]), "k": k, "v": v}


def ffn_half(x1, W: Dict[str, np.ndarray], dims):
    """The FFN half of a decoder layer: x2 = x1 + SwiGLU(RMSNorm(x1) * ffn_norm) Wd^T."""
    _, act = swiglu_act(x1, W, dims.rms_eps)
    return down_proj(x1, act, W["wd"])


def plain_layer(x, pos, W: Dict[str, np.ndarray], dims, cu):
    """A layer below the gate: both halves, plain causal attention (t = 1,
    g = 0; the gate's bias only exists above it). Returns {"x2", "k", "v"}."""
    a = attention_half(x, pos, np.zeros(_f64(x).shape[0]), W, dims, cu,
                       t=np.ones(dims.Hq), g=np.zeros(dims.Hq))
    return {"x2": ffn_half(a["x1"], W, dims), "k": a["k"], "v": a["v"]}


def local_positions(cu_in):
    """Each token's index inside its own sequence (the original positions)."""
    cu_in = np.asarray(cu_in, dtype=np.int64)
    return np.concatenate([np.arange(int(cu_in[b + 1] - cu_in[b])) for b in range(len(cu_in) - 1)]
                          or [np.zeros(0, dtype=np.int64)])


def full_prefill(h, gate, below, gate_layer, above, keep_mask, cu_in, cu_kept, dims):
    """The three-stage forward with the gate at layer L = len(below).

    [FW] the method and [AI] mechanism design: the forward splits in three;
    [TC] early token filtering: all prompt tokens go through the layers below
    the gate and through layer L's attention (full-prompt KV there, [TC]
    engineering section); the scorer reads layer L's post-attention residual
    and the selector keeps K tokens; only those go on into layer L's FFN and
    the layers above, whose attention is gated.
      h: [T_in, D] the rows entering layer 0; gate: (W1, b1, w2, b2);
      below: L layer dicts; gate_layer: layer L's dict; above: layer dicts.
    Selection runs on the oracle's own scores.
    """
    pos = local_positions(cu_in)
    x = _f64(h)
    kv_below = []
    for W in below:
        r = plain_layer(x, pos, W, dims, cu_in)
        kv_below.append((r["k"], r["v"]))
        x = r["x2"]
    x_below = x
    a = attention_half(x, pos, np.zeros(x.shape[0]), gate_layer, dims, cu_in,
                       t=np.ones(dims.Hq), g=np.zeros(dims.Hq))
    kv_below.append((a["k"], a["v"]))
    x1 = a["x1"]
    s = gate_score(x1, *gate)
    kept, flags = topk_select(s, keep_mask, cu_in, cu_kept)
    x1c, pos_c, s_c = compact(x1, pos, s, kept, cu_in, cu_kept)
    xk = ffn_half(x1c, gate_layer, dims)
    x_gate = xk
    kv_above = []
    for W in above:
        r = upper_layer(xk, pos_c, s_c, W, dims, cu_kept)
        kv_above.append((r["k"], r["v"]))
        xk = r["x2"]
    return {"x_below": x_below, "x1": x1, "s": s, "kept": kept, "flags": flags, "pos_c": pos_c,
            "s_c": s_c, "x_gate": x_gate, "x": xk, "kv_below": kv_below, "kv_above": kv_above}


def unpruned_prefill(h, layers, cu_in, dims):
    """The same model without the gate: every layer on every token with plain
    attention (the baseline the pages' prefill speedups are measured against)."""
    pos = local_positions(cu_in)
    x = _f64(h)
    for W in layers:
        x = plain_layer(x, pos, W, dims, cu_in)["x2"]
    return x


# ----------------------------------------------------------------------------
# The whole gated prefill above layer L's attention
# ----------------------------------------------------------------------------

def gated_prefill(h, W1, b1, w2, b2, keep_mask, cu_in, cu_kept, layers, dims, pos=None):
    """Scorer, selection, compaction and the stack of upper layers.

    [FW] the method and [AI] mechanism design: the forward splits in three;
    below the gate all N tokens are processed, the gate keeps the top K, and
    above it only those K tokens run. This function covers the part from the
    gate on. Selection here runs on the oracle's own scores.
    """
    s = gate_score(h, W1, b1, w2, b2)
    kept, flags = topk_select(s, keep_mask, cu_in, cu_kept)
    hc, pc, sc = compact(h, pos, s, kept, cu_in, cu_kept)
    x = _f64(hc)
    kv = []
    for W in layers:
        r = upper_layer(x, pc, sc, W, dims, cu_kept)
        kv.append((r["k"], r["v"]))
        x = r["x2"]
    return {"s": s, "kept": kept, "flags": flags, "pos_c": pc, "s_c": sc, "x": x, "kv": kv}
