"""Exact scaled-dot-product attention, float64, CPU.  TEST INFRASTRUCTURE ONLY.

What it computes, and where that comes from:

* The FlashAttention v1 post (DeepSchool #630), section «Проблема базового
  attention», describes standard attention as forming the whole n x n matrix
  Q K^T and applying a softmax to it.  Its formula images were not captured,
  so this module takes the textbook reading that the rest of the page
  supports:  O = softmax(scale * Q K^T [+ causal mask]) V, softmax along each
  row (over keys).
* Section «Онлайн-Softmax» of the same post defines the softmax denominator
  as the row sum of exponentials, and states that the tiled method gives a
  result fully equivalent to this classic softmax.  So the oracle is the
  classic form, written out: pass 1 takes the row maximum, pass 2
  exponentiates the shifted scores, sums them and normalises.  The maximum
  only guards against overflow; it cancels mathematically.
* The per-row log-sum-exp LSE_i = m_i + ln(l_i) (natural log) is the one
  extra output the forward pass writes besides O.  The pages do not mention
  it; it is the log of the softmax denominator of the *scaled, masked*
  scores.
* Causal mask: query i attends to keys j <= i (one shared length N, so
  top-left and bottom-right alignment coincide).
* Grouped-query attention: H query heads share Hkv key/value heads in
  contiguous groups, query head h reads KV head h // (H // Hkv).  The pages
  only raise GQA as a question (FlashAttention-3 summary, section
  «Comentários no Hacker News»).
* A row with no visible key (impossible with the causal mask, since key 0 is
  always visible) is defined here as O = 0, LSE = -inf.

Parity status: pinned by tests/test_oracle_attention.py against a scalar
brute-force triple loop, torch's float64 CPU attention routine, closed forms
(zero queries, constant values, single visible key) and invariances (key
permutation, key shift, GQA = repeated-KV MHA), and against hand-derived
values in tests/golden/.  attention_kv (Nq x Nk, bottom-right causal) is
pinned by tests/test_oracle_decode.py: a scalar brute force, torch's
float64 attention with an explicit mask, the square case, the last row of
square causal attention and the merge of a key split.  attention_varlen
(sequences of different lengths, sliding window) is pinned by
tests/test_oracle_varlen.py: a scalar brute force, torch's float64
attention with an explicit mask, the unwindowed case and closed forms of
the narrowest windows.  attention_masked (an arbitrary boolean mask) is
pinned by tests/test_oracle_masked.py: a scalar brute force, torch's
float64 attention with the same mask, and the causal, windowed and
all-visible masks against the oracle's own closed-form paths.
"""

from __future__ import annotations

import numpy as np


def _as_f64(x) -> np.ndarray:
    """Upcast any float array (fp32, or bf16 values already widened to fp32)
    to float64.  Widening is exact."""
    return np.asarray(x, dtype=np.float64)


def _head(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, rows: np.ndarray,
          causal: bool, scale: float, offset: int = 0, left: int = -1,
          right: int = -1, allow=None):
    """One (batch, head): qh [Nq,d], kh/vh [Nk,d], rows = query indices.
    Causal: query i sees key j iff j <= i + offset.  A window (left, right
    >= 0; -1 = unbounded) further requires i + offset - left <= j <=
    i + offset + right.  allow, if given, is a boolean [len(rows), Nk]
    array: key j is visible to row r only where allow[r, j] is true.
    Returns O [len(rows), d] and LSE [len(rows)] in float64."""
    n_keys = kh.shape[0]
    # Scores for the selected query rows against every key: the full row of
    # the n x n matrix Q K^T, times the scale.
    s = scale * (qh[rows] @ kh.T)                       # [R, N]
    key_idx = np.arange(n_keys)[None, :]
    diag = rows[:, None] + offset
    if causal:
        s = np.where(key_idx <= diag, s, -np.inf)
    if left >= 0:
        s = np.where(key_idx >= diag - left, s, -np.inf)
    if right >= 0:
        s = np.where(key_idx <= diag + right, s, -np.inf)
    if allow is not None:
        s = np.where(allow, s, -np.inf)
    # Pass 1: row maximum over visible keys.
    m = s.max(axis=1)                                   # [R]
    dead = ~np.isfinite(m)                              # no visible key
    m_safe = np.where(dead, 0.0, m)
    # Pass 2: exponentials of the shifted scores, their sum, normalisation.
    e = np.exp(s - m_safe[:, None])                     # exp(-inf) = 0
    l = e.sum(axis=1)                                   # [R]
    with np.errstate(divide="ignore", invalid="ignore"):
        p = e / l[:, None]
    o = p @ vh                                          # [R, d]
    with np.errstate(divide="ignore"):                  # l = 0 where dead
        lse = m_safe + np.log(l)
    o[dead] = 0.0
    lse[dead] = -np.inf
    return o, lse


def attention_rows(q, k, v, rows, *, causal: bool = False, scale=None,
                   heads=None):
    """Attention for a subset of query rows.

    q: [B, H, N, d]; k, v: [B, Hkv, N, d]; rows: 1-D int array of query
    indices (the same rows for every head); heads: optional list of
    (b, h) pairs to evaluate (default: all).

    Returns (O, LSE) with O: [len(heads), len(rows), d], LSE:
    [len(heads), len(rows)], float64.  Each output row depends only on its
    own query and on all keys/values, so evaluating a subset is exact.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, H, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, Nk, dk) != (B, N, d) or v.shape != k.shape:
        raise ValueError("shape mismatch between q and k/v")
    if Hkv <= 0 or H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    group = H // Hkv
    rows = np.asarray(rows, dtype=np.int64)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    o = np.zeros((len(heads), len(rows), d))
    lse = np.zeros((len(heads), len(rows)))
    for i, (b, h) in enumerate(heads):
        kvh = h // group
        o[i], lse[i] = _head(q[b, h], k[b, kvh], v[b, kvh], rows, causal,
                             float(scale))
    return o, lse


def attention(q, k, v, *, causal: bool = False, scale=None):
    """Full attention.  q: [B,H,N,d]; k, v: [B,Hkv,N,d] (any float dtype).

    Returns O [B,H,N,d] and LSE [B,H,N], both float64.  scale=None means
    1/sqrt(d)."""
    q = _as_f64(q)
    B, H, N, d = q.shape
    o, lse = attention_rows(q, k, v, np.arange(N), causal=causal, scale=scale)
    return o.reshape(B, H, N, d), lse.reshape(B, H, N)


def attention_kv(q, k, v, *, causal: bool = False, scale=None):
    """Attention of Nq queries against Nk keys (decode and split-KV).

    q: [B, H, Nq, d]; k, v: [B, Hkv, Nk, d].  With causal, the queries are
    the last Nq positions of a sequence of Nk (bottom-right alignment):
    query i sees key j iff j <= i + Nk - Nq, so a query sees no key when
    Nq > Nk and i < Nq - Nk (O = 0, LSE = -inf there).  The pages motivate
    this case only as long-context processing (FlashAttention-3 summary,
    sections «Importância do Attention» and «Melhorias de desempenho do
    FlashAttention-3»); the alignment is the plainest reading for queries
    appended after Nk - Nq earlier positions.

    Returns O [B, H, Nq, d] and LSE [B, H, Nq], float64."""
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, H, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, dk) != (B, d) or v.shape != k.shape:
        raise ValueError("shape mismatch between q and k/v")
    if Hkv <= 0 or H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    group = H // Hkv
    rows = np.arange(Nq)
    o = np.zeros((B, H, Nq, d))
    lse = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            kvh = h // group
            o[b, h], lse[b, h] = _head(q[b, h], k[b, kvh], v[b, kvh], rows,
                                       causal, float(scale), Nk - Nq)
    return o, lse


def attention_varlen(qs, ks, vs, *, causal: bool = False, window_left=-1,
                     window_right=-1, scale=None):
    """Attention over a batch of sequences of different lengths, each with
    an optional sliding window.

    qs: list of [H, Nq_b, d]; ks, vs: lists of [Hkv, Nk_b, d] (one entry per
    sequence).  Sequences never see each other.  Within sequence b, with
    off = Nk_b - Nq_b (bottom-right alignment), query i sees key j iff
    (not causal or j <= i + off) and (window_left < 0 or j >= i + off -
    window_left) and (window_right < 0 or j <= i + off + window_right).  A
    query that sees no key gets O = 0, LSE = -inf.  The pages raise variable
    masking (slow in FlashAttention, the FlashAttention-3 summary, section
    «Comentários no Hacker News») and sliding-window attention (same
    section) only as questions; this is the plainest reading of both.

    Returns lists of O [H, Nq_b, d] and LSE [H, Nq_b], float64."""
    outs, lses = [], []
    for q, k, v in zip(qs, ks, vs):
        q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
        H, Nq, d = q.shape
        Hkv, Nk, _ = k.shape
        if H % Hkv != 0 or k.shape != v.shape or k.shape[2] != d:
            raise ValueError("shape mismatch")
        sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
        group = H // Hkv
        o = np.zeros((H, Nq, d))
        lse = np.zeros((H, Nq))
        for h in range(H):
            o[h], lse[h] = _head(q[h], k[h // group], v[h // group],
                                 np.arange(Nq), causal, sc, Nk - Nq,
                                 int(window_left), int(window_right))
        outs.append(o)
        lses.append(lse)
    return outs, lses


def attention_masked(q, k, v, mask, *, scale=None, rows=None):
    """Attention under an arbitrary visibility mask.

    q: [B, H, Nq, d]; k, v: [B, Hkv, Nk, d]; mask: boolean array that
    broadcasts to [B, H, Nq, Nk] (size-1 batch or head axes are shared):
    query i of (b, h) sees key j iff mask[b, h, i, j].  A query that sees no
    key gets O = 0, LSE = -inf.  The pages raise arbitrary and variable
    masks only as a question (FlashAttention-3 summary, section
    «Comentários no Hacker News»: FlashAttention is said to be much slower
    with them); the plainest reading is the softmax over the visible keys
    only, which is what masking scores to -inf gives.  rows (optional) picks
    the query rows to evaluate, for every (b, h).

    Returns O [B, H, R, d] and LSE [B, H, R] (R = Nq or len(rows)), float64.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, H, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, dk) != (B, d) or v.shape != k.shape:
        raise ValueError("shape mismatch between q and k/v")
    if Hkv <= 0 or H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    mask = np.asarray(mask, dtype=bool)
    if mask.ndim != 4:
        raise ValueError("mask must have 4 axes [B|1, H|1, Nq, Nk]")
    mask = np.broadcast_to(mask, (B, H, Nq, Nk))
    sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
    rows = np.arange(Nq) if rows is None else np.asarray(rows, np.int64)
    group = H // Hkv
    o = np.zeros((B, H, len(rows), d))
    lse = np.zeros((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            kvh = h // group
            o[b, h], lse[b, h] = _head(q[b, h], k[b, kvh], v[b, kvh], rows,
                                       False, sc, allow=mask[b, h][rows])
    return o, lse
