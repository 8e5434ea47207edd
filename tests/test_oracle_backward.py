"""Pins of the CPU backward oracle against things other than itself.

The gradients are checked against central finite differences of the loss
sum(dO * O) through the (separately pinned) forward oracle, against torch's
float64 autograd of its own attention routine, and against closed forms.  A
dropped scale, a transposed operand, a missing D term, a causal mask on the
wrong side or a wrong GQA reduction fails at least one of them.
"""

import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(q, k, v, do, causal, scale):
    o, _ = oracle.attention(q, k, v, causal=causal, scale=scale)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Hkv,N,d", [(1, 1, 1, 4, 3), (1, 2, 1, 5, 2),
                                         (2, 2, 2, 3, 4)])
def test_finite_differences(B, H, Hkv, N, d, causal):
    """Central differences of sum(dO * O) in every input entry."""
    q, k, v = _rand((B, H, N, d), 1), _rand((B, Hkv, N, d), 2), _rand(
        (B, Hkv, N, d), 3)
    do = _rand((B, H, N, d), 4)
    scale = 0.7
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal=causal,
                                           scale=scale)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            up = _loss(q, k, v, do, causal, scale)
            x[idx] = keep - eps
            dn = _loss(q, k, v, do, causal, scale)
            x[idx] = keep
            num[idx] = (up - dn) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=0, atol=2e-8)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Hkv,N,d", [(2, 4, 2, 33, 16), (1, 4, 1, 70, 32)])
def test_torch_autograd_fp64(B, H, Hkv, N, d, causal):
    """Library routine: autograd of torch's CPU scaled_dot_product_attention
    in float64."""
    q, k, v = _rand((B, H, N, d), 5), _rand((B, Hkv, N, d), 6), _rand(
        (B, Hkv, N, d), 7)
    do = _rand((B, H, N, d), 8)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal=causal,
                                           scale=scale)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True)
                  for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=(H != Hkv))
    o.backward(torch.from_numpy(do))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_gradient_sums_to_zero(causal):
    """Adding one vector to every key shifts each row's scores by a constant,
    which the softmax ignores: the gradients of all keys sum to zero."""
    q = _rand((1, 2, 40, 8), 9)
    k = _rand((1, 2, 40, 8), 10)
    v = _rand((1, 2, 40, 8), 11)
    do = _rand((1, 2, 40, 8), 12)
    _, dk, _ = oracle.attention_backward(q, k, v, do, causal=causal)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v(causal):
    """Constant value rows make O constant whatever the scores: dQ = dK = 0,
    and dV_j = sum_i P_ij dO_i, whose sum over j is sum_i dO_i."""
    q = _rand((1, 2, 30, 8), 13)
    k = _rand((1, 2, 30, 8), 14)
    v = np.broadcast_to(_rand((1, 2, 1, 8), 15), (1, 2, 30, 8)).copy()
    do = _rand((1, 2, 30, 8), 16)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal=causal)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)
    np.testing.assert_allclose(dk, 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_dv_column_sums(causal):
    """Rows of P sum to 1, so the dV rows sum to the dO rows (any V)."""
    q = _rand((2, 4, 25, 8), 17)
    k = _rand((2, 2, 25, 8), 18)
    v = _rand((2, 2, 25, 8), 19)
    do = _rand((2, 4, 25, 8), 20)
    _, _, dv = oracle.attention_backward(q, k, v, do, causal=causal)
    want = do.reshape(2, 2, 2, 25, 8).sum(axis=(2, 3))
    np.testing.assert_allclose(dv.sum(axis=2), want, atol=1e-12)


def test_first_row_causal_dq_is_zero():
    """Under the causal mask query 0 sees only key 0: its softmax weight is
    1 whatever the score, so dQ_0 = 0."""
    q, k, v = _rand((1, 1, 6, 4), 21), _rand((1, 1, 6, 4), 22), _rand(
        (1, 1, 6, 4), 23)
    do = _rand((1, 1, 6, 4), 24)
    dq, _, _ = oracle.attention_backward(q, k, v, do, causal=True)
    np.testing.assert_allclose(dq[0, 0, 0], 0.0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_matches_full(causal):
    B, H, Hkv, N, d = 2, 4, 2, 90, 16
    q, k, v = _rand((B, H, N, d), 25), _rand((B, Hkv, N, d), 26), _rand(
        (B, Hkv, N, d), 27)
    do = _rand((B, H, N, d), 28)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal=causal)
    q_rows = np.array([0, 5, 44, 89])
    k_rows = np.array([0, 1, 60, 89])
    kv_heads = [(0, 1), (1, 0)]
    sq, sk, sv = oracle.attention_backward_sampled(
        q, k, v, do, q_rows, k_rows, kv_heads, causal=causal, chunk=32)
    for t, (b, kvh) in enumerate(kv_heads):
        for g in range(H // Hkv):
            np.testing.assert_allclose(sq[t, g], dq[b, kvh * 2 + g][q_rows],
                                       atol=1e-12)
        np.testing.assert_allclose(sk[t], dk[b, kvh][k_rows], atol=1e-12)
        np.testing.assert_allclose(sv[t], dv[b, kvh][k_rows], atol=1e-12)
