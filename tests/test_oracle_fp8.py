"""Pins of the oracle's OCP e4m3 codec and per-tensor quantisation."""

import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3_decode, e4m3_encode


def _torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _torch_encode(x):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = _torch_decode(codes)
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_landmark_values():
    assert e4m3_decode(0x7E) == 448.0
    assert e4m3_decode(0xFE) == -448.0
    assert e4m3_decode(0x08) == 2.0 ** -6          # smallest normal
    assert e4m3_decode(0x01) == 2.0 ** -9          # smallest subnormal
    assert e4m3_decode(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert e4m3_decode(0x38) == 1.0
    assert e4m3_decode(0x00) == 0.0 and np.signbit(e4m3_decode(0x80))


def test_round_trip_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert len(codes) == 254
    np.testing.assert_array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def _tricky_values(n, seed):
    rng = np.random.default_rng(seed)
    mags = np.exp2(rng.uniform(-12, np.log2(448.0), n))
    pos = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2                  # exact ties
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9))])
    vals = np.concatenate([mags, mids, near, pos, [0.0, 2.0 ** -10, 3 * 2.0 ** -11]])
    vals = vals.astype(np.float32)
    sign = np.where(rng.random(vals.shape) < 0.5, -1, 1).astype(np.float32)
    return vals * sign


def test_encode_matches_torch_rne():
    x = _tricky_values(1_000_000, 1)
    assert np.all(np.abs(x) <= 448.0)
    np.testing.assert_array_equal(e4m3_encode(x), _torch_encode(x))


def test_encode_brute_force_nearest_even():
    x = _tricky_values(3000, 2).astype(np.float64)
    table = e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = np.array([c for c in range(256) if not np.isnan(table[c])])
    for xi, c in zip(x, e4m3_encode(x)):
        dist = np.abs(table[finite] - xi)
        best = finite[dist == dist.min()]
        best = [b for b in best if (b >= 0x80) == bool(np.signbit(xi)) or table[b] != 0]
        # among equally near codes take the one with the even mantissa
        best = [b for b in best if b % 2 == 0] or best
        assert table[c] == table[best[0]], (xi, c, best)


def test_saturation_and_nan():
    np.testing.assert_array_equal(e4m3_encode([1000.0, -1000.0, 449.0, 1e30]),
                                  [0x7E, 0xFE, 0x7E, 0x7E])
    assert e4m3_encode([np.nan])[0] == 0x7F


@pytest.mark.parametrize("signs", [None, "random"])
def test_quantize_invariants(signs):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    x[3, 5] = 40.0
    s = None if signs is None else np.where(rng.random(128) < 0.5, -1, 1)
    codes, descale, amax = oracle.quantize_per_tensor(x, s)
    xr = x.astype(np.float64) if s is None else oracle.rotate(x, s)
    assert amax == np.float32(np.max(np.abs(xr.astype(np.float32))))
    assert descale == np.float32(amax / np.float32(448.0))
    vals = e4m3_decode(codes)
    assert np.max(np.abs(vals)) == 448.0
    # each code is within half an e4m3 step (relative 2^-4, or 2^-10 absolute
    # in the subnormal range) of x * inv
    y = xr * (448.0 / float(amax))
    err = np.abs(vals - y)
    bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * 1.0001
    assert np.all(err <= bound)
    # dequantised relative error is small
    deq = vals * float(descale)
    rel = np.linalg.norm(deq - xr) / np.linalg.norm(xr)
    assert rel < 0.05


def test_quantize_zero_tensor():
    codes, descale, amax = oracle.quantize_per_tensor(np.zeros((4, 8), np.float32))
    assert amax == 0 and descale == 1.0 and np.all(codes == 0)
