"""Plain, slow, fp64 CPU oracle for TokenGate's gated-prefill path.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only
the tests, the smoke check and the benchmark's CPU-baseline leg may call it.
It shares no code with the HIP path: it is written from the pages' statement
of the method, in numpy float64, one definition per function, with no
blocking, fusion or reordering beyond what that definition states.

Sources (the pages this library is built from):

* [paper] "TokenGate: Adapting LLMs for Fast and Memory-Efficient Prefill with
  Learned Token Pruning", paper page on thelatestinai.com: Abstract and
  Figure 1 (a)-(c).
* [aitualizate] the aitualizate.com news article on TokenGate, sections
  "2. Una red MLP aprende qué tokens conservar", "3. Las capas superiores
  procesan únicamente los tokens seleccionados" and "Cómo consigue entrenar
  una selección top-K".

Readings of points the pages leave open are marked READING and are the same
ones the library documents.  Every function here is pinned by the
``-m "not gpu"`` tests against closed forms, brute force, invariants and
independent library routines.
"""
from __future__ import annotations

import numpy as np

FLT_MIN = float(np.finfo(np.float32).tiny)  # 2**-126, smallest normal fp32

__all__ = [
    "FLT_MIN",
    "ref_gate",
    "ref_select",
    "ref_select_varlen",
    "ref_gather",
    "ref_gather_varlen",
    "ref_rope",
    "ref_rope_kv",
    "ref_attn",
    "ref_attn_varlen",
    "ref_decode",
    "ref_linear",
    "ref_swiglu",
    "ref_mlp",
]


def _f64(x) -> np.ndarray:
    """Any array-like (numpy, or a CPU torch tensor of fp32/bf16) as float64."""
    if hasattr(x, "detach"):  # torch tensor: widen exactly before leaving torch
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.asarray(x, dtype=np.int64)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


# --------------------------------------------------------------------------
# Stage 1: gate MLP.
# [paper] Figure 1(b): the gate module scores every hidden state with a small
# scoring network; [aitualizate] section 2: a small MLP reads each token's
# post-attention residual state at the selection layer and gives it a score.
# [paper] Figure 1(c): the score enters attention as a gate value g_j.
# READING: the network is Linear(d->H) + b1, SiLU, Linear(H->1) + b2, and the
# gate value is g = sigmoid(s) in (0, 1); the pages do not print its form.
# --------------------------------------------------------------------------
def ref_gate(h, w1, b1, w2, b2):
    """Gate MLP over every token.

    h  [n, d], w1 [H, d] (row k holds hidden unit k's input weights),
    b1 [H] or None, w2 [H], b2 scalar.
    Returns (g [n], s [n]) in float64: s is the score (logit), g = sigmoid(s).
    """
    h = _f64(h)
    w1 = _f64(w1)
    w2 = _f64(w2).reshape(-1)
    b1 = np.zeros(w1.shape[0]) if b1 is None else _f64(b1).reshape(-1)
    a = h @ w1.T + b1[None, :]          # pre-activation of the hidden layer [n, H]
    z = a * _sigmoid(a)                 # SiLU(a) = a * sigmoid(a)
    s = z @ w2 + float(b2)              # score [n]
    g = _sigmoid(s)                     # gate value in (0, 1)
    return g, s


# --------------------------------------------------------------------------
# Stage 2: top-K selection.
# [paper] Figure 1(a),(b): at layer L a top-K selector keeps K of the N tokens.
# [aitualizate] section 3: only the document part of the prompt may be pruned;
# the question is never removed.
# READINGS: K counts every kept token, question included, so min(K, N) - q_len
# document tokens are chosen; K >= N keeps everything.  Scores are compared as
# fp32 numbers; -0 equals +0; a NaN ranks below every number.  Ties go to the
# lower index.  The kept indices come out in ascending (prompt) order, so the
# question tail comes last.
# --------------------------------------------------------------------------
def ref_select(g, k: int, q_len: int) -> np.ndarray:
    """Indices (int64, ascending) of the tokens kept out of ``len(g)``."""
    g = np.asarray(g.detach().cpu().numpy() if hasattr(g, "detach") else g, dtype=np.float32)
    n = int(g.shape[0])
    k = int(k)
    q_len = int(q_len)
    kept_total = min(k, n)
    if q_len < 0 or q_len > kept_total:
        raise ValueError("q_len must lie in [0, min(k, n)]")
    doc = n - q_len
    kd = kept_total - q_len
    if kd >= doc:
        return np.arange(n, dtype=np.int64)
    vals = g[:doc].astype(np.float64)
    is_nan = np.isnan(vals)
    vals = np.where(is_nan, 0.0, vals)
    index = np.arange(doc)
    # Primary: not-NaN first; then larger value first; then lower index first.
    order = np.lexsort((index, -vals, is_nan))
    chosen = np.sort(order[:kd])
    return np.concatenate([chosen, np.arange(doc, n)]).astype(np.int64)


def ref_select_varlen(g, cu_seqlens, q_lens, k: int):
    """Per-prompt ``ref_select`` over a packed score vector.

    Returns (idx_local, cu_kept): idx_local holds each prompt's kept positions
    relative to the prompt's start, concatenated; cu_kept [B+1] the offsets.
    """
    g = np.asarray(g.detach().cpu().numpy() if hasattr(g, "detach") else g, dtype=np.float32)
    cu = _i64(cu_seqlens)
    qs = _i64(q_lens)
    out, cu_kept = [], [0]
    for b in range(len(qs)):
        sel = ref_select(g[cu[b]:cu[b + 1]], k, int(qs[b]))
        out.append(sel)
        cu_kept.append(cu_kept[-1] + len(sel))
    return np.concatenate(out).astype(np.int64), np.asarray(cu_kept, dtype=np.int64)


# --------------------------------------------------------------------------
# Stage 3: gather.
# [paper] Figure 1(b): the selector forwards the kept hidden states together
# with their importance scores; [aitualizate] section 3: the layers above L
# receive only the kept tokens.  READING: each kept token also carries its
# original 0-based position in the prompt.
# --------------------------------------------------------------------------
def ref_gather(h, g, idx):
    """Rows of h and entries of g at idx (a copy), and pos = idx."""
    h = np.asarray(h)
    g = np.asarray(g)
    idx = _i64(idx)
    return h[idx].copy(), g[idx].copy(), idx.copy()


def ref_gather_varlen(h, g, idx_local, cu_seqlens, cu_kept):
    """Packed variant: prompt b's rows are h[cu_seqlens[b] + idx_local[i]]."""
    cu = _i64(cu_seqlens)
    ck = _i64(cu_kept)
    idx_local = _i64(idx_local)
    rows = np.empty_like(idx_local)
    for b in range(len(cu) - 1):
        rows[ck[b]:ck[b + 1]] = cu[b] + idx_local[ck[b]:ck[b + 1]]
    h = np.asarray(h)
    g = np.asarray(g)
    return h[rows].copy(), g[rows].copy(), idx_local.copy()


# --------------------------------------------------------------------------
# Stage 5: RoPE at the kept tokens' original positions, and a KV cache that
# holds only the kept tokens.
# [aitualizate] section 3: discarded tokens make no entries in the key/value
# cache of the layers above L.  READING: RoPE is the rotate-half form (pairs
# (i, i + Dh/2)), angle pos * base**(-2i/Dh), applied at the token's original
# position; the pages do not describe position encoding.
# --------------------------------------------------------------------------
def ref_rope(x, pos, base: float):
    """Rotate x [n, heads, dh] at positions pos [n]; float64 result."""
    x = _f64(x)
    pos = _f64(_i64(pos))
    dh = x.shape[-1]
    half = dh // 2
    i = np.arange(half, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / dh)            # [half]
    phi = pos[:, None] * theta[None, :]                       # [n, half]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def ref_rope_kv(q, k, v, pos, base: float):
    """Rotated q, the key cache (rotated k) and the value cache (v), float64."""
    return ref_rope(q, pos, base), ref_rope(k, pos, base), _f64(v).copy()


# --------------------------------------------------------------------------
# Stage 4: token-gated causal attention over the kept tokens.
# [paper] Figure 1(c): every attention weight is multiplied by the gate value
# g_j of its key (and, being attention weights, they are renormalised);
# [paper] Abstract and [aitualizate] "Cómo consigue entrenar una selección
# top-K": the importance score re-weights the attention logits as a bias.
# Both say the same thing: softmax_j(s_ij + ln g_j).
# READINGS: scale 1/sqrt(Dh) applied to q.k before the bias; gain 1 and
# temperature 1 (the pages' raw-bias form); g is clamped below at FLT_MIN so
# the bias stays finite; key j is visible to query i iff pos_j <= pos_i; query
# head h uses KV head h // (Hq / Hkv).
# --------------------------------------------------------------------------
def ref_attn(q, k, v, g, pos, scale: float | None = None, rows=None, head_gain=None):
    """q [n, hq, dh], k/v [n, hkv, dh], g [n] or None, pos [n].

    Returns (o [n, hq, dh], lse [hq, n]) in float64; lse is the natural-log
    normaliser of the biased logits.  With ``rows`` (query indices) only those
    queries are computed, against all n keys: o [len(rows), hq, dh] and
    lse [hq, len(rows)].

    ``g=None`` is the ungated attention of the full-context layers (bias 0).
    READING (per-head gain and temperature on the bias, named by the TokenGate
    paper page without their forms): head h adds ``head_gain[h] * ln max(g_j,
    FLT_MIN)``; ``head_gain=None`` means 1 for every head.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    pos = _i64(pos)
    n, hq, dh = q.shape
    hkv = k.shape[1]
    rows = np.arange(n) if rows is None else _i64(rows)
    if scale is None:
        scale = 1.0 / np.sqrt(dh)
    group = hq // hkv
    bias = np.zeros(n) if g is None else np.log(np.maximum(_f64(g), FLT_MIN))   # [n]
    gain = np.ones(hq) if head_gain is None else _f64(head_gain)
    visible = pos[None, :] <= pos[rows][:, None]              # [query i, key j]
    o = np.empty((len(rows), hq, dh))
    lse = np.empty((hq, len(rows)))
    for h in range(hq):
        kvh = h // group
        s = scale * (q[rows, h, :] @ k[:, kvh, :].T) + gain[h] * bias[None, :]
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        o[:, h, :] = (p @ v[:, kvh, :]) / l
        lse[h, :] = (m + np.log(l))[:, 0]
    return o, lse


def ref_attn_varlen(q, k, v, g, pos, cu_seqlens, scale: float | None = None, head_gain=None):
    """Packed variant: each prompt b attends only within its own rows."""
    cu = _i64(cu_seqlens)
    q = _f64(q)
    n, hq, dh = q.shape
    o = np.empty((n, hq, dh))
    lse = np.empty((hq, n))
    k = _f64(k)
    v = _f64(v)
    g = None if g is None else _f64(g)
    pos = _i64(pos)
    for b in range(len(cu) - 1):
        a, e = cu[b], cu[b + 1]
        if e == a:
            continue
        ob, lb = ref_attn(q[a:e], k[a:e], v[a:e], None if g is None else g[a:e], pos[a:e], scale,
                          head_gain=head_gain)
        o[a:e] = ob
        lse[:, a:e] = lb
    return o, lse


def ref_decode(q, k_cache, v_cache, g, cu_seqlens, scale: float | None = None, head_gain=None):
    """One new query per sequence over its whole cache (no causal mask: every
    cached key precedes the new token).

    q [B, hq, dh]; k_cache, v_cache [total, hkv, dh] packed by ``cu_seqlens``
    [B + 1]; g [total] or None.  Returns (o [B, hq, dh], lse [B, hq]) float64;
    a sequence with an empty cache gives o = 0 and lse = -inf.

    READING (decode is not described on the pages): the compact cache keeps
    the kept prompt tokens' gate bias ln max(g_j, FLT_MIN) (times the head's
    gain), exactly as in the gated prefill attention; generated tokens carry
    g = 1 (bias 0), and g=None means no bias at all.
    """
    q = _f64(q)
    kc = _f64(k_cache)
    vc = _f64(v_cache)
    cu = _i64(cu_seqlens)
    B, hq, dh = q.shape
    hkv = kc.shape[1]
    group = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(dh)
    gain = np.ones(hq) if head_gain is None else _f64(head_gain)
    bias_all = None if g is None else np.log(np.maximum(_f64(g), FLT_MIN))
    o = np.zeros((B, hq, dh))
    lse = np.full((B, hq), -np.inf)
    for b in range(B):
        a, e = cu[b], cu[b + 1]
        if e == a:
            continue
        bias = np.zeros(e - a) if bias_all is None else bias_all[a:e]
        for h in range(hq):
            kvh = h // group
            s = scale * (kc[a:e, kvh, :] @ q[b, h, :]) + gain[h] * bias
            m = s.max()
            p = np.exp(s - m)
            l = p.sum()
            o[b, h, :] = (p @ vc[a:e, kvh, :]) / l
            lse[b, h] = m + np.log(l)
    return o, lse


# ---------------------------------------------------------------------------
# Upper-layer dense work on the kept tokens.
#
# [aitualizate] section 3: every layer above the selection layer processes only
# the kept tokens, so its projections and MLP run on K rows instead of N.  The
# layer shape is the base model the pages evaluate (the paper page's setup
# table: Qwen3-1.7B in bf16): QKV and O projections without bias and a SwiGLU
# MLP.  READING: the LoRA adapters of that setup (rank 16, alpha 32, on the
# query and value projections) are merged into the weights before the path,
# W' = W + (alpha / r) B A, so each projection is one plain product with W'.


def ref_linear(x, w, residual=None):
    """y = x W^T (+ residual): x [M, Kin], w [Nout, Kin] (nn.Linear layout),
    residual [M, Nout] or None.  float64."""
    y = _f64(x) @ _f64(w).T
    if residual is not None:
        y = y + _f64(residual)
    return y


def _silu(z: np.ndarray) -> np.ndarray:
    return z * _sigmoid(z)


def ref_swiglu(x, w_gate, w_up):
    """SwiGLU hidden activation: SiLU(x W_gate^T) * (x W_up^T), with
    w_gate, w_up [F, Kin].  Returns [M, F] float64."""
    return _silu(ref_linear(x, w_gate)) * ref_linear(x, w_up)


def ref_mlp(x, w_gate, w_up, w_down, residual=None):
    """The MLP block: SwiGLU(x) W_down^T (+ residual), w_down [d, F]."""
    return ref_linear(ref_swiglu(x, w_gate, w_up), w_down, residual)
