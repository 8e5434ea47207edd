"""Pins of the oracle's Nq x Nk attention (decode / split-KV) against things
other than itself: a scalar brute force with the bottom-right causal rule,
torch's float64 attention with an explicit mask, the square oracle, the last
row of square causal attention, and the log-sum-exp merge of a key split.
"""

import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _brute(q, k, v, causal, scale):
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = H // Hkv
    o = np.zeros((B, H, Nq, d))
    lse = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        for h in range(H):
            kh = h // g
            for i in range(Nq):
                keys = [j for j in range(Nk)
                        if not causal or j <= i + Nk - Nq]
                if not keys:
                    continue
                w = [math.exp(scale * math.fsum(
                    float(q[b, h, i, t]) * float(k[b, kh, j, t])
                    for t in range(d))) for j in keys]
                z = math.fsum(w)
                lse[b, h, i] = math.log(z)
                for t in range(d):
                    o[b, h, i, t] = math.fsum(
                        wj * float(v[b, kh, j, t]) for wj, j in zip(w, keys)) / z
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d", [(1, 2, 1, 1, 7, 3),
                                             (2, 2, 2, 3, 5, 2),
                                             (1, 4, 2, 6, 4, 3)])
def test_brute_force(B, H, Hkv, Nq, Nk, d, causal):
    q, k, v = _rand((B, H, Nq, d), 1), _rand((B, Hkv, Nk, d), 2), _rand(
        (B, Hkv, Nk, d), 3)
    o, lse = oracle.attention_kv(q, k, v, causal=causal, scale=0.8)
    ob, lb = _brute(q, k, v, causal, 0.8)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_torch_masked_fp64(causal):
    B, H, Hkv, Nq, Nk, d = 2, 4, 2, 9, 70, 16
    q, k, v = _rand((B, H, Nq, d), 4), _rand((B, Hkv, Nk, d), 5), _rand(
        (B, Hkv, Nk, d), 6)
    o, _ = oracle.attention_kv(q, k, v, causal=causal)
    mask = None
    if causal:
        mask = torch.from_numpy(np.arange(Nk)[None, :] <=
                                np.arange(Nq)[:, None] + (Nk - Nq))
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), attn_mask=mask,
        scale=1.0 / math.sqrt(d), enable_gqa=True)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_square_case_matches_attention(causal):
    q, k, v = _rand((1, 2, 33, 8), 7), _rand((1, 2, 33, 8), 8), _rand(
        (1, 2, 33, 8), 9)
    o, lse = oracle.attention_kv(q, k, v, causal=causal)
    o2, lse2 = oracle.attention(q, k, v, causal=causal)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_single_causal_query_is_last_row_of_square():
    """One decode query sees every key under the bottom-right rule: it is the
    last row of square causal attention."""
    q = _rand((1, 2, 40, 8), 10)
    k, v = _rand((1, 2, 40, 8), 11), _rand((1, 2, 40, 8), 12)
    o, lse = oracle.attention_kv(q[:, :, -1:], k, v, causal=True)
    o2, lse2 = oracle.attention(q, k, v, causal=True)
    np.testing.assert_allclose(o[:, :, 0], o2[:, :, -1], atol=1e-13)
    np.testing.assert_allclose(lse[:, :, 0], lse2[:, :, -1], atol=1e-13)


def test_merge_of_a_key_split():
    """Softmax over the union of two key sets from the two partial results:
    LSE = log(e^LSE_1 + e^LSE_2), O = sum_s e^(LSE_s - LSE) O_s."""
    q = _rand((1, 2, 5, 8), 13)
    k, v = _rand((1, 2, 50, 8), 14), _rand((1, 2, 50, 8), 15)
    o, lse = oracle.attention_kv(q, k, v)
    parts = [oracle.attention_kv(q, k[:, :, a:b], v[:, :, a:b])
             for a, b in ((0, 17), (17, 50))]
    l_m = np.logaddexp(parts[0][1], parts[1][1])
    o_m = sum(np.exp(ls - l_m)[..., None] * os for os, ls in parts)
    np.testing.assert_allclose(lse, l_m, atol=1e-12)
    np.testing.assert_allclose(o, o_m, atol=1e-12)
