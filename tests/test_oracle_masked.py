"""Pins of the oracle's attention under an arbitrary boolean mask against
things other than itself: a scalar brute force, torch's float64 attention
with the same boolean mask, the independence of the result from masked
keys' contents, and the causal, windowed and all-visible masks (whose own
paths are pinned elsewhere).  Also the bit packing of masks."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _brute(q, k, v, mask, scale):
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = H // Hkv
    o = np.zeros((B, H, Nq, d))
    lse = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                keys = [j for j in range(Nk) if mask[b, h, i, j]]
                if not keys:
                    continue
                w = [math.exp(scale * math.fsum(
                    float(q[b, h, i, t]) * float(k[b, h // g, j, t])
                    for t in range(d))) for j in keys]
                z = math.fsum(w)
                lse[b, h, i] = math.log(z)
                for t in range(d):
                    o[b, h, i, t] = math.fsum(
                        wj * float(v[b, h // g, j, t])
                        for wj, j in zip(w, keys)) / z
    return o, lse


@pytest.mark.parametrize("p", [0.05, 0.4, 1.0])
def test_brute_force(p):
    B, H, Hkv, Nq, Nk, d = 2, 4, 2, 6, 9, 3
    q, k, v = _rand((B, H, Nq, d), 1), _rand((B, Hkv, Nk, d), 2), _rand(
        (B, Hkv, Nk, d), 3)
    mask = workloads.random_mask((B, H, Nq, Nk), p, 4)
    mask[0, 0, 0] = False                    # one row with no visible key
    o, lse = oracle.attention_masked(q, k, v, mask, scale=0.7)
    ob, lb = _brute(q, k, v, mask, 0.7)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], atol=1e-12)
    assert np.all(o[0, 0, 0] == 0) and np.isneginf(lse[0, 0, 0])


@pytest.mark.parametrize("bcast", [(1, 1), (2, 1), (1, 4), (2, 4)])
def test_torch_masked_fp64(bcast):
    """Masks shared across batches and/or heads broadcast as stated."""
    B, H, Hkv, Nq, Nk, d = 2, 4, 2, 33, 50, 16
    q, k, v = _rand((B, H, Nq, d), 5), _rand((B, Hkv, Nk, d), 6), _rand(
        (B, Hkv, Nk, d), 7)
    mask = workloads.random_mask((bcast[0], bcast[1], Nq, Nk), 0.3, 8)
    o, lse = oracle.attention_masked(q, k, v, mask)
    full = np.broadcast_to(mask, (B, H, Nq, Nk))
    alive = full.any(axis=-1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)),
        attn_mask=torch.from_numpy(full.copy()),
        scale=1.0 / math.sqrt(d), enable_gqa=True).numpy()
    np.testing.assert_allclose(o[alive], ref[alive], atol=1e-12)
    assert np.all(o[~alive] == 0) and np.all(np.isneginf(lse[~alive]))


def test_masked_keys_do_not_matter():
    """Changing K and V wherever no query sees them changes nothing."""
    q, k, v = _rand((1, 2, 10, 8), 9), _rand((1, 2, 20, 8), 10), _rand(
        (1, 2, 20, 8), 11)
    mask = workloads.random_mask((1, 1, 10, 20), 0.5, 12)
    mask[..., 5] = False
    mask[..., 17] = False
    a = oracle.attention_masked(q, k, v, mask)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, [5, 17]] = 1e3
    v2[:, :, [5, 17]] = -7.0
    b = oracle.attention_masked(q, k2, v2, mask)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_causal_window_and_full_masks():
    B, H, Hkv, N, d = 1, 4, 2, 24, 8
    q, k, v = _rand((B, H, N, d), 13), _rand((B, Hkv, N, d), 14), _rand(
        (B, Hkv, N, d), 15)
    i, j = np.arange(N)[:, None], np.arange(N)[None, :]
    o, lse = oracle.attention_masked(q, k, v, (j <= i)[None, None])
    oc, lc = oracle.attention(q, k, v, causal=True)
    np.testing.assert_array_equal(o, oc)
    np.testing.assert_array_equal(lse, lc)
    o, lse = oracle.attention_masked(q, k, v, np.ones((1, 1, N, N), bool))
    of, lf = oracle.attention(q, k, v)
    np.testing.assert_array_equal(o, of)
    np.testing.assert_array_equal(lse, lf)
    win = (j <= i) & (j >= i - 3)
    o, lse = oracle.attention_masked(q, k, v, win[None, None])
    (ow,), (lw,) = oracle.attention_varlen([q[0]], [k[0]], [v[0]],
                                           causal=True, window_left=3)
    np.testing.assert_array_equal(o[0], ow)
    np.testing.assert_array_equal(lse[0], lw)


def test_rows_subset():
    q, k, v = _rand((2, 2, 30, 8), 16), _rand((2, 1, 40, 8), 17), _rand(
        (2, 1, 40, 8), 18)
    mask = workloads.random_mask((2, 1, 30, 40), 0.2, 19)
    o, lse = oracle.attention_masked(q, k, v, mask)
    rows = np.array([0, 7, 29])
    o2, lse2 = oracle.attention_masked(q, k, v, mask, rows=rows)
    np.testing.assert_array_equal(o2, o[:, :, rows])
    np.testing.assert_array_equal(lse2, lse[:, :, rows])


def test_pack_mask_bits():
    m = workloads.random_mask((3, 70), 0.5, 20)
    w = workloads.pack_mask(m)
    assert w.shape == (3, 3) and w.dtype == np.uint32
    for r in range(3):
        for j in range(96):
            bit = (int(w[r, j // 32]) >> (j % 32)) & 1
            assert bit == (int(m[r, j]) if j < 70 else 0)


def test_block_sparse_mask_shape():
    m = workloads.block_sparse_mask(1000, 700, 128, 2, 21)
    assert m.shape == (1000, 700)
    # Every query block sees key block 0 and its own diagonal block.
    assert m[:, :128].all()
    assert m[300, 256:384].all()
