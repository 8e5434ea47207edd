"""Gradients of exact attention, float64, CPU.  TEST INFRASTRUCTURE ONLY.

What it computes, and where that comes from:

* The pages describe the backward pass only in outline: the FlashAttention-4
  page (smntcn.com), paragraph 2, says its bottleneck is shared-memory
  traffic, and the FlashAttention-3 summary (GeekNews), section «Resumo do
  FlashAttention», says FlashAttention relies on tiling and recomputation.
  They give no formulas.  The plainest reading, which this module takes, is
  the exact gradient of the forward definition the forward oracle uses,
  O = softmax(scale * Q K^T [+ causal mask]) V, given dO = dL/dO, with the
  softmax matrix P recomputed (here: from scratch, two passes, exactly as
  the forward oracle forms it).
* Written out for one (batch, head), with P the [N, N] softmax matrix
  (rows = queries):
      dV = P^T dO
      dP = dO V^T
      D_i = sum_j P_ij dP_ij
      dS = P * (dP - D)            (elementwise; D broadcast along rows)
      dQ = scale * dS K
      dK = scale * dS^T Q
  Masked entries have P = 0, so they get no gradient.
* Grouped-query attention: the Hkv key/value heads are shared by H / Hkv
  query heads each, so dK and dV of a KV head are the sums over its query
  heads.

Parity status: pinned by tests/test_oracle_backward.py against central
finite differences of sum(dO * O) through the forward oracle, torch's
float64 CPU autograd of its attention routine, and closed forms (the
gradients of a key shift and of a constant V, the column sums of dV).
"""

from __future__ import annotations

import numpy as np

from .attention import attention_rows


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax of a score block whose rows all have a visible key
    (two passes: row maximum, then exponentials and their sum)."""
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def _head_backward(qh, kh, vh, doh, causal: bool, scale: float):
    """One (batch, head), all rows.  Returns dQ, dK, dV, each [N, d]."""
    n = qh.shape[0]
    s = scale * (qh @ kh.T)
    if causal:
        s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
    p = _softmax_rows(s)                     # masked entries: exp(-inf) = 0
    dv = p.T @ doh
    dp = doh @ vh.T
    d_row = (p * dp).sum(axis=1, keepdims=True)
    ds = p * (dp - d_row)
    dq = scale * (ds @ kh)
    dk = scale * (ds.T @ qh)
    return dq, dk, dv


def _check(q, k, v, do):
    B, H, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, Nk, dk) != (B, N, d) or v.shape != k.shape or do.shape != q.shape:
        raise ValueError("shape mismatch")
    if Hkv <= 0 or H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    return B, H, Hkv, N, d


def attention_backward(q, k, v, do, *, causal: bool = False, scale=None):
    """Gradients of O = attention(q, k, v) against dO.

    q, do: [B, H, N, d]; k, v: [B, Hkv, N, d] (any float dtype).
    Returns (dq [B,H,N,d], dk [B,Hkv,N,d], dv [B,Hkv,N,d]) in float64.
    scale=None means 1/sqrt(d)."""
    q, k, v, do = (_as_f64(x) for x in (q, k, v, do))
    B, H, Hkv, N, d = _check(q, k, v, do)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    group = H // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            kvh = h // group
            gq, gk, gv = _head_backward(q[b, h], k[b, kvh], v[b, kvh],
                                        do[b, h], causal, float(scale))
            dq[b, h] = gq
            dk[b, kvh] += gk
            dv[b, kvh] += gv
    return dq, dk, dv


def attention_backward_sampled(q, k, v, do, q_rows, k_rows, kv_heads, *,
                               causal: bool = False, scale=None,
                               chunk: int = 1024):
    """The same gradients at sampled rows, without forming any N x N matrix.

    q_rows: query indices whose dQ is wanted; k_rows: key indices whose dK
    and dV are wanted; kv_heads: list of (b, kv_head).  For each (b, kvh)
    returns dQ at q_rows for every query head of the group, and dK, dV at
    k_rows summed over the group:
      dq [len(kv_heads), group, len(q_rows), d],
      dk, dv [len(kv_heads), len(k_rows), d].

    dQ row i needs only row i of P and dP.  dK / dV row j needs column j of
    P for every query, hence every query's LSE, and D_i for every query; D_i
    is taken as dO_i . O_i, which equals sum_j P_ij dP_ij because
    dP_ij = dO_i . V_j and sum_j P_ij V_j = O_i."""
    q, k, v, do = (_as_f64(x) for x in (q, k, v, do))
    B, H, Hkv, N, d = _check(q, k, v, do)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    scale = float(scale)
    group = H // Hkv
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    out_dq = np.zeros((len(kv_heads), group, len(q_rows), d))
    out_dk = np.zeros((len(kv_heads), len(k_rows), d))
    out_dv = np.zeros((len(kv_heads), len(k_rows), d))
    for t, (b, kvh) in enumerate(kv_heads):
        kh, vh = k[b, kvh], v[b, kvh]
        for g in range(group):
            h = kvh * group + g
            qh, doh = q[b, h], do[b, h]
            # dQ at the sampled query rows: full rows of P and dP.
            s = scale * (qh[q_rows] @ kh.T)
            if causal:
                s = np.where(np.arange(N)[None, :] <= q_rows[:, None], s,
                             -np.inf)
            p = _softmax_rows(s)
            dp = doh[q_rows] @ vh.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            out_dq[t, g] = scale * (ds @ kh)
            # dK, dV at the sampled key rows: every query, in chunks.
            for i0 in range(0, N, chunk):
                rows = np.arange(i0, min(N, i0 + chunk))
                o, lse = attention_rows(qh[None, None], kh[None, None],
                                        vh[None, None], rows, causal=causal,
                                        scale=scale)
                o, lse = o[0], lse[0]
                sc = scale * (qh[rows] @ kh[k_rows].T)       # [R, Ks]
                if causal:
                    sc = np.where(k_rows[None, :] <= rows[:, None], sc,
                                  -np.inf)
                pc = np.exp(sc - lse[:, None])
                dpc = doh[rows] @ vh[k_rows].T
                d_row = (doh[rows] * o).sum(axis=1, keepdims=True)
                dsc = pc * (dpc - d_row)
                out_dv[t] += pc.T @ doh[rows]
                out_dk[t] += scale * (dsc.T @ qh[rows])
    return out_dq, out_dk, out_dv
