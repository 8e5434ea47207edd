"""Pins of the oracle's variable-length, sliding-window attention against
things other than itself: a scalar brute force, torch's float64 attention
with an explicit mask, the unwindowed decode oracle, and closed forms of the
narrowest windows."""

import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _visible(i, j, off, causal, wl, wr):
    return ((not causal or j <= i + off) and (wl < 0 or j >= i + off - wl)
            and (wr < 0 or j <= i + off + wr))


def _brute(q, k, v, causal, wl, wr, scale):
    H, Nq, d = q.shape
    Hkv, Nk, _ = k.shape
    g = H // Hkv
    o = np.zeros((H, Nq, d))
    lse = np.full((H, Nq), -np.inf)
    for h in range(H):
        for i in range(Nq):
            keys = [j for j in range(Nk)
                    if _visible(i, j, Nk - Nq, causal, wl, wr)]
            if not keys:
                continue
            w = [math.exp(scale * math.fsum(float(q[h, i, t]) * float(
                k[h // g, j, t]) for t in range(d))) for j in keys]
            z = math.fsum(w)
            lse[h, i] = math.log(z)
            for t in range(d):
                o[h, i, t] = math.fsum(wj * float(v[h // g, j, t])
                                       for wj, j in zip(w, keys)) / z
    return o, lse


CASES = [(False, -1, -1), (True, -1, -1), (False, 2, 1), (True, 3, -1),
         (False, 0, 0), (False, -1, 2), (True, 1, 4)]


@pytest.mark.parametrize("causal,wl,wr", CASES)
def test_brute_force(causal, wl, wr):
    lens = [(5, 7), (3, 3), (6, 2)]
    qs = [_rand((4, nq, 3), 10 + i) for i, (nq, _) in enumerate(lens)]
    ks = [_rand((2, nk, 3), 20 + i) for i, (_, nk) in enumerate(lens)]
    vs = [_rand((2, nk, 3), 30 + i) for i, (_, nk) in enumerate(lens)]
    os_, ls_ = oracle.attention_varlen(qs, ks, vs, causal=causal,
                                       window_left=wl, window_right=wr,
                                       scale=0.6)
    for q, k, v, o, lse in zip(qs, ks, vs, os_, ls_):
        ob, lb = _brute(q, k, v, causal, wl, wr, 0.6)
        np.testing.assert_allclose(o, ob, atol=1e-12)
        np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(lb))
        fin = np.isfinite(lb)
        np.testing.assert_allclose(lse[fin], lb[fin], atol=1e-12)


@pytest.mark.parametrize("causal,wl,wr", CASES)
def test_torch_masked_fp64(causal, wl, wr):
    H, Hkv, Nq, Nk, d = 4, 2, 40, 70, 16
    q, k, v = _rand((H, Nq, d), 1), _rand((Hkv, Nk, d), 2), _rand(
        (Hkv, Nk, d), 3)
    (o,), (lse,) = oracle.attention_varlen([q], [k], [v], causal=causal,
                                           window_left=wl, window_right=wr)
    mask = np.array([[_visible(i, j, Nk - Nq, causal, wl, wr)
                      for j in range(Nk)] for i in range(Nq)])
    alive = mask.any(axis=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x[None]) for x in (q, k, v)),
        attn_mask=torch.from_numpy(mask), scale=1.0 / math.sqrt(d),
        enable_gqa=True)[0].numpy()
    np.testing.assert_allclose(o[:, alive], ref[:, alive], atol=1e-12)
    assert np.all(o[:, ~alive] == 0) and np.all(np.isneginf(lse[:, ~alive]))


@pytest.mark.parametrize("causal", [False, True])
def test_unbounded_window_is_plain_attention(causal):
    q, k, v = _rand((1, 4, 9, 8), 4), _rand((1, 2, 30, 8), 5), _rand(
        (1, 2, 30, 8), 6)
    (o,), (lse,) = oracle.attention_varlen([q[0]], [k[0]], [v[0]],
                                           causal=causal)
    o2, lse2 = oracle.attention_kv(q, k, v, causal=causal)
    np.testing.assert_array_equal(o, o2[0])
    np.testing.assert_array_equal(lse, lse2[0])


def test_zero_width_window_picks_one_key():
    """window (0, 0): query i sees only key i + off, so O_i = V_{i+off} and
    LSE_i = scale * q_i . k_{i+off}."""
    q, k, v = _rand((2, 6, 8), 7), _rand((2, 9, 8), 8), _rand((2, 9, 8), 9)
    (o,), (lse,) = oracle.attention_varlen([q], [k], [v], window_left=0,
                                           window_right=0, scale=0.5)
    for i in range(6):
        np.testing.assert_allclose(o[:, i], v[:, i + 3], atol=1e-14)
        np.testing.assert_allclose(lse[:, i],
                                   0.5 * (q[:, i] * k[:, i + 3]).sum(-1),
                                   atol=1e-13)


def test_causal_wins_over_a_wider_right_window():
    q, k, v = _rand((2, 12, 8), 10), _rand((2, 12, 8), 11), _rand((2, 12, 8),
                                                                   12)
    a = oracle.attention_varlen([q], [k], [v], causal=True, window_right=5)
    b = oracle.attention_varlen([q], [k], [v], causal=True)
    np.testing.assert_array_equal(a[0][0], b[0][0])


def test_window_outside_the_keys_gives_empty_rows():
    """Nq > Nk with a narrow causal window: leading rows see no key."""
    q, k, v = _rand((1, 8, 4), 13), _rand((1, 3, 4), 14), _rand((1, 3, 4), 15)
    (o,), (lse,) = oracle.attention_varlen([q], [k], [v], causal=True,
                                           window_left=1)
    assert np.all(np.isneginf(lse[0, :5])) and np.all(o[0, :5] == 0)
    assert np.all(np.isfinite(lse[0, 5:]))
