"""The polynomial of the FMA-pipe exponential (fa_exp2_fma.h), checked on
the CPU against exact 2^x: the header's coefficients are the Remez fit that
exp2_fit.py computes, the fit equioscillates (it is the minimax polynomial,
not merely a close one), and a float32 model of the device code's steps
(range reduction, Horner with fused multiply-adds, exponent add) stays
within the 7.5e-5 relative bound fa.h states for x in [-125, 127]."""

import importlib.util
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_101_amd", "csrc")
BOUND = 7.5e-5


def _fit():
    spec = importlib.util.spec_from_file_location(
        "exp2_fit", os.path.join(CSRC, "exp2_fit.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _header_coefficients():
    text = open(os.path.join(CSRC, "fa_exp2_fma.h")).read()
    found = dict(re.findall(r"EXP2_C(\d) = (0x[0-9a-fp.+-]+)f;", text))
    return np.array([float.fromhex(found[str(i)]) for i in range(4)],
                    dtype=np.float32)


def test_header_holds_the_fit():
    c = _header_coefficients()
    np.testing.assert_array_equal(c, _fit().coefficients(3))


def test_fit_equioscillates():
    """Minimax: the relative error reaches its maximum magnitude, with
    alternating signs, at degree + 2 = 5 points of [-1/2, 1/2]."""
    c = _fit().remez(3)
    f = np.linspace(-0.5, 0.5, 400001)
    err = np.polyval(c[::-1], f) / np.exp2(f) - 1.0
    emax = np.abs(err).max()
    # local extrema of the error, endpoints included
    inner = np.flatnonzero((np.abs(err[1:-1]) >= np.abs(err[:-2])) &
                           (np.abs(err[1:-1]) >= np.abs(err[2:]))) + 1
    ext = np.concatenate(([0], inner, [f.size - 1]))
    big = ext[np.abs(err[ext]) >= 0.999 * emax]
    signs = np.sign(err[big])
    assert big.size >= 5
    assert np.all(signs[1:] != signs[:-1])
    # better than the Taylor polynomial of the same degree about 0
    ln2 = np.log(2.0)
    taylor = [ln2 ** k / np.prod(np.arange(1, k + 1)) for k in range(4)]
    terr = np.abs(np.polyval(taylor[::-1], f) / np.exp2(f) - 1.0).max()
    assert emax < terr / 4


def _device_model(x):
    """The device code's steps in float32 (fa_exp2_fma.h, exp2_fma)."""
    fit = _fit()
    c = _header_coefficients()
    x = np.maximum(x.astype(np.float32), np.float32(-125.0))
    R = np.float32(12582912.0)
    t = (x + R).astype(np.float32)
    n = (t - R).astype(np.float32)
    f = (x - n).astype(np.float32)
    p = fit.eval32(c, f)
    bits = p.view(np.uint32).astype(np.uint64) + \
        ((t.view(np.uint32).astype(np.uint64) << 23) & 0xFFFFFFFF)
    return (bits & 0xFFFFFFFF).astype(np.uint32).view(np.float32)


def test_device_steps_within_bound():
    x = np.concatenate([
        np.linspace(-125.0, 127.0, 2_000_001, dtype=np.float32),
        np.arange(-125, 128, dtype=np.float32),
        np.arange(-125, 127, dtype=np.float32) + 0.5,
    ])
    y = _device_model(x).astype(np.float64)
    rel = np.abs(y / np.exp2(x.astype(np.float64)) - 1.0)
    assert np.all(np.isfinite(y))
    assert rel.max() <= BOUND
    # the reduction is exact: f = x - rint(x) lies in [-1/2, 1/2]
    R = np.float32(12582912.0)
    f = x - ((x + R) - R)
    assert np.abs(f).max() <= 0.5


def test_device_steps_below_range():
    y = _device_model(np.array([-np.inf, -1000.0, -126.0], np.float32))
    assert np.all(y > 0) and np.all(y <= 2.36e-38)
