"""Pins of the CPU attention oracle against things other than itself.

Each check is chosen so that a plausible slip in the oracle (a dropped scale,
a transposed operand, the mask on the wrong side, a wrong GQA head map, LSE
in the wrong base, a missing max-shift) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _brute(q, k, v, causal, scale):
    """Scalar triple loop with math.exp / math.fsum and no max-shift."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    g = H // Hkv
    o = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            kh = h // g
            for i in range(N):
                keys = range(i + 1) if causal else range(N)
                w = []
                for j in keys:
                    dot = math.fsum(float(q[b, h, i, t]) * float(k[b, kh, j, t])
                                    for t in range(d))
                    w.append(math.exp(scale * dot))
                z = math.fsum(w)
                lse[b, h, i] = math.log(z)
                for t in range(d):
                    o[b, h, i, t] = math.fsum(wj * float(v[b, kh, j, t])
                                              for wj, j in zip(w, keys)) / z
    return o, lse


@pytest.mark.parametrize("B,H,Hkv,N,d", [(1, 1, 1, 1, 1), (1, 2, 1, 5, 3),
                                         (2, 4, 2, 9, 5), (1, 3, 3, 7, 4)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force(B, H, Hkv, N, d, causal):
    q = _rand((B, H, N, d), 1)
    k = _rand((B, Hkv, N, d), 2)
    v = _rand((B, Hkv, N, d), 3)
    scale = 0.7
    o, lse = oracle.attention(q, k, v, causal=causal, scale=scale)
    ob, lb = _brute(q, k, v, causal, scale)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Hkv,N,d", [(2, 4, 2, 33, 16), (1, 8, 1, 130, 64)])
def test_torch_sdpa_fp64(B, H, Hkv, N, d, causal):
    """Library routine: torch's CPU scaled_dot_product_attention in float64
    (and torch.logsumexp for the LSE)."""
    q = _rand((B, H, N, d), 4)
    k = _rand((B, Hkv, N, d), 5)
    v = _rand((B, Hkv, N, d), 6)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention(q, k, v, causal=causal, scale=scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=(H != Hkv))
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    tk_rep = tk.repeat_interleave(H // Hkv, dim=1)
    s = torch.matmul(tq, tk_rep.transpose(-1, -2)) * scale
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(),
                               rtol=0, atol=1e-12)


def _ln(expr):
    assert expr.startswith("ln")
    return math.log(float(expr[2:]))


def test_golden_hand_worked():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        scale = _ln(c["scale"])
        q = np.array(c["q"])[None, None]
        k = np.array(c["k"])[None, None]
        v = np.array(c["v"])[None, None]
        for mode, causal in (("noncausal", False), ("causal", True)):
            o, lse = oracle.attention(q, k, v, causal=causal, scale=scale)
            np.testing.assert_allclose(o[0, 0], np.array(c[mode]["o"]),
                                       rtol=0, atol=1e-14)
            np.testing.assert_allclose(
                lse[0, 0], [_ln(e) for e in c[mode]["lse"]], rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v(causal):
    """Softmax rows sum to one: V with every row equal to c gives O = c."""
    q = _rand((1, 2, 40, 8), 7) * 3
    k = _rand((1, 2, 40, 8), 8)
    c = _rand((8,), 9)
    v = np.broadcast_to(c, (1, 2, 40, 8)).copy()
    o, _ = oracle.attention(q, k, v, causal=causal)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0,
                               atol=1e-12)


def test_key_permutation_noncausal():
    q = _rand((1, 2, 50, 16), 10)
    k = _rand((1, 2, 50, 16), 11)
    v = _rand((1, 2, 50, 16), 12)
    perm = np.random.default_rng(13).permutation(50)
    o1, l1 = oracle.attention(q, k, v)
    o2, l2 = oracle.attention(q, k[:, :, perm], v[:, :, perm])
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_causal_first_row_single_key():
    q = _rand((2, 3, 20, 8), 14)
    k = _rand((2, 3, 20, 8), 15)
    v = _rand((2, 3, 20, 8), 16)
    scale = 0.3
    o, lse = oracle.attention(q, k, v, causal=True, scale=scale)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])           # exactly V[0]
    np.testing.assert_allclose(
        lse[:, :, 0], scale * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
        rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_closed_form(causal):
    """Q = 0: uniform weights over the visible keys."""
    N = 37
    q = np.zeros((1, 2, N, 4))
    k = _rand((1, 2, N, 4), 17)
    v = _rand((1, 2, N, 4), 18)
    o, lse = oracle.attention(q, k, v, causal=causal)
    if causal:
        cnt = np.arange(1, N + 1)
        mean = np.cumsum(v, axis=2) / cnt[:, None]
        np.testing.assert_allclose(lse, np.broadcast_to(np.log(cnt), lse.shape),
                                   rtol=0, atol=1e-13)
    else:
        mean = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        np.testing.assert_allclose(lse, math.log(N), rtol=0, atol=1e-13)
    np.testing.assert_allclose(o, mean, rtol=0, atol=1e-13)


def test_zero_scale_equals_zero_query():
    q = _rand((1, 1, 30, 8), 19)
    k = _rand((1, 1, 30, 8), 20)
    v = _rand((1, 1, 30, 8), 21)
    o1, l1 = oracle.attention(q, k, v, causal=True, scale=0.0)
    o2, l2 = oracle.attention(np.zeros_like(q), k, v, causal=True)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift(causal):
    """K_j -> K_j + u for every key: O unchanged, LSE_i += scale * q_i.u."""
    q = _rand((1, 2, 25, 8), 22)
    k = _rand((1, 2, 25, 8), 23)
    v = _rand((1, 2, 25, 8), 24)
    u = _rand((8,), 25)
    scale = 0.4
    o1, l1 = oracle.attention(q, k, v, causal=causal, scale=scale)
    o2, l2 = oracle.attention(q, k + u, v, causal=causal, scale=scale)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, scale * q @ u, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_repeated_kv(causal):
    B, H, Hkv, N, d = 2, 8, 2, 21, 8
    q = _rand((B, H, N, d), 26)
    k = _rand((B, Hkv, N, d), 27)
    v = _rand((B, Hkv, N, d), 28)
    o1, l1 = oracle.attention(q, k, v, causal=causal)
    rep = H // Hkv
    o2, l2 = oracle.attention(q, np.repeat(k, rep, axis=1),
                              np.repeat(v, rep, axis=1), causal=causal)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=0)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=0)


def test_large_scores_stay_finite():
    """Scores in the hundreds: finite, and the weights tend to the argmax."""
    q = _rand((1, 1, 16, 8), 29)
    k = _rand((1, 1, 16, 8), 30)
    v = _rand((1, 1, 16, 8), 31)
    scale = 100.0
    o, lse = oracle.attention(q, k, v, scale=scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    s = scale * q[0, 0] @ k[0, 0].T
    top = np.argmax(s, axis=1)
    gap = np.sort(s, axis=1)[:, -1] - np.sort(s, axis=1)[:, -2]
    sure = gap > 40.0       # runner-up weight below e^-40
    assert sure.any()
    np.testing.assert_allclose(o[0, 0][sure], v[0, 0][top[sure]], atol=1e-12)
    np.testing.assert_allclose(lse[0, 0][sure], s.max(axis=1)[sure], atol=1e-12)


def test_rows_subset_matches_full():
    q = _rand((1, 4, 64, 16), 32)
    k = _rand((1, 2, 64, 16), 33)
    v = _rand((1, 2, 64, 16), 34)
    rows = np.array([0, 5, 31, 63])
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, causal=causal)
        os_, ls_ = oracle.attention_rows(q, k, v, rows, causal=causal)
        np.testing.assert_allclose(os_.reshape(1, 4, 4, 16), o[:, :, rows],
                                   rtol=0, atol=1e-14)
        np.testing.assert_allclose(ls_.reshape(1, 4, 4), lse[:, :, rows],
                                   rtol=0, atol=1e-14)


def test_bad_shapes_raise():
    q = np.zeros((1, 3, 4, 2))
    k = np.zeros((1, 2, 4, 2))
    with pytest.raises(ValueError):
        oracle.attention(q, k, k)
