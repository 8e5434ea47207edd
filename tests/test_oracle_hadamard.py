"""Pins of the oracle's Sylvester Hadamard matrix and signed rotation."""

import numpy as np
import pytest
import scipy.linalg

import oracle


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128])
def test_sylvester_matches_scipy(d):
    np.testing.assert_array_equal(oracle.sylvester(d), scipy.linalg.hadamard(d))


@pytest.mark.parametrize("d", [2, 64, 128])
def test_orthogonality(d):
    h = oracle.sylvester(d)
    np.testing.assert_array_equal(h @ h.T, d * np.eye(d))


def test_small_matrix_by_hand():
    np.testing.assert_array_equal(oracle.sylvester(2), [[1, 1], [1, -1]])
    np.testing.assert_array_equal(
        oracle.sylvester(4),
        [[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])


def test_rotation_is_orthonormal_and_preserves_scores():
    rng = np.random.default_rng(0)
    d = 128
    s = np.where(rng.random(d) < 0.5, -1, 1)
    q = rng.standard_normal((40, d))
    k = rng.standard_normal((50, d))
    qr, kr = oracle.rotate(q, s), oracle.rotate(k, s)
    np.testing.assert_allclose(np.linalg.norm(qr, axis=1),
                               np.linalg.norm(q, axis=1), rtol=1e-13)
    ref = q @ k.T
    np.testing.assert_allclose(qr @ kr.T, ref, rtol=0,
                               atol=1e-12 * np.abs(ref).max())
    r = oracle.rotate(np.eye(d), s)
    np.testing.assert_allclose(r @ r.T, np.eye(d), atol=1e-14)
    # the inverse rotation R^T = H diag(s) / sqrt(d) recovers x
    back = (qr @ oracle.sylvester(d).T / np.sqrt(d)) * s
    np.testing.assert_allclose(back, q, atol=1e-12)


def test_unit_signs_is_plain_hadamard():
    x = np.arange(8.0)
    np.testing.assert_allclose(oracle.rotate(x, np.ones(8)),
                               x @ scipy.linalg.hadamard(8) / np.sqrt(8),
                               rtol=0, atol=1e-13)


def test_rotation_lowers_outlier_quantisation_error():
    """Direction of the pages' claim (rotation reduces the FP8 error); the
    page's 2.6x factor depends on an unstated distribution and is not
    checked."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2048, 128)).astype(np.float32)
    x[rng.random(x.shape) < 1e-3] *= 20
    s = np.where(rng.random(128) < 0.5, -1, 1)
    c0, d0, _ = oracle.quantize_per_tensor(x)
    e0 = np.linalg.norm(oracle.e4m3_decode(c0) * d0 - x) / np.linalg.norm(x)
    c1, d1, _ = oracle.quantize_per_tensor(x, s)
    xr = oracle.rotate(x, s)
    e1 = np.linalg.norm(oracle.e4m3_decode(c1) * d1 - xr) / np.linalg.norm(xr)
    assert e1 < e0
