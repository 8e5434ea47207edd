"""Seeded generators: reproducible, right shapes, right outlier rate, and the
bf16 cast is round-to-nearest-even."""

import numpy as np
import torch

import workloads


def test_same_seed_same_bytes():
    a = workloads.qkv(1, 2, 1, 64, 16, 123, outliers=True)
    b = workloads.qkv(1, 2, 1, 64, 16, 123, outliers=True)
    for x, y in zip(a, b):
        assert x.tobytes() == y.tobytes()
    c = workloads.qkv(1, 2, 1, 64, 16, 124, outliers=True)
    assert a[0].tobytes() != c[0].tobytes()


def test_shapes_and_dtype():
    q, k, v = workloads.qkv(2, 8, 2, 33, 64, 7)
    assert q.shape == (2, 8, 33, 64) and k.shape == v.shape == (2, 2, 33, 64)
    assert q.dtype == np.float32 and q.flags.c_contiguous


def test_outlier_fraction():
    n = 4_000_000
    base = workloads.draw((n,), 5, outliers=False)
    x = workloads.draw((n,), 5, outliers=True, outlier_seed=99)
    hit = x != base
    p = 1e-3
    sigma = np.sqrt(n * p * (1 - p))
    assert abs(hit.sum() - n * p) < 5 * sigma
    np.testing.assert_array_equal(x[hit], base[hit] * np.float32(20))


def test_bf16_cast_is_rne():
    x = workloads.draw((100_000,), 11) * np.float32(3.7)
    bits = x.view(np.uint32).astype(np.uint64)
    rne = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    got = workloads.to_bf16(x).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, rne)
    back = workloads.bf16_values(workloads.to_bf16(x))
    np.testing.assert_array_equal(back.view(np.uint32) >> 16, rne.astype(np.uint32))


def test_workload_table():
    w = workloads.WORKLOADS
    assert w["tiny_d64"].N == 256 and w["tiny_d64"].d == 64
    assert w["bf16_causal_gqa_n16384"].H == 32 and w["bf16_causal_gqa_n16384"].Hkv == 8
    # 4 B H N^2 d, halved for causal
    assert w["bf16_n8192"].flops == 4.0 * 4 * 16 * 8192 ** 2 * 128
    assert w["bf16_causal_n8192"].flops == 2.0 * 2 * 32 * 8192 ** 2 * 128
    assert abs(w["bf16_n8192"].flops - 2.199e12) / 2.199e12 < 1e-3
    assert workloads.HEADLINE in w


def test_hadamard_signs():
    s = workloads.hadamard_signs(128, 9)
    assert s.shape == (128,) and set(np.unique(s)) == {-1, 1}
    np.testing.assert_array_equal(s, workloads.hadamard_signs(128, 9))
