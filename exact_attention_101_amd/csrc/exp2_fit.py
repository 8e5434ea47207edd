"""Minimax polynomial for 2^f on f in [-1/2, 1/2] (relative error), the
core of the software exp2 the fp8 forward can run on the FMA pipe.

The method: range reduction x = n + f with n = rint(x), which is exact in
binary floating point for base 2 (the two-part constant of Cody and Waite's
reduction is only needed for bases other than 2), then 2^f from a polynomial
whose coefficients come from the Remez exchange algorithm (equioscillation of
the relative error at degree + 2 points), here in float64, then rounded to
float32.  The result is ldexp(p(f), n), done by adding n to the exponent
field.

Usage: python exp2_fit.py [degree]  -- prints the float32 coefficients (c0
first, as hex floats and decimals) and the error of the float32 evaluation
order the kernel uses (Horner with fused multiply-adds).
"""

from __future__ import annotations

import sys

import numpy as np

LO, HI = -0.5, 0.5


def remez(degree: int, iters: int = 40):
    """Coefficients c[0..degree] (float64) minimising max |p(f)/2^f - 1|."""
    n = degree + 2
    # Chebyshev extrema as the first reference.
    k = np.arange(n)
    x = 0.5 * (LO + HI) + 0.5 * (HI - LO) * -np.cos(np.pi * k / (n - 1))
    grid = np.linspace(LO, HI, 200001)
    for _ in range(iters):
        # Solve p(x_i) - (-1)^i E 2^x_i = 2^x_i for c and E.
        A = np.zeros((n, n))
        for j in range(degree + 1):
            A[:, j] = x ** j
        A[:, degree + 1] = -((-1.0) ** k) * np.exp2(x)
        sol = np.linalg.solve(A, np.exp2(x))
        c = sol[:degree + 1]
        err = np.polyval(c[::-1], grid) / np.exp2(grid) - 1.0
        # New reference: the extremum of each sign run of the error.
        sign = np.sign(err)
        runs = np.flatnonzero(np.diff(sign) != 0) + 1
        bounds = np.concatenate(([0], runs, [grid.size]))
        ext = [b0 + int(np.argmax(np.abs(err[b0:b1])))
               for b0, b1 in zip(bounds[:-1], bounds[1:]) if b1 > b0]
        if len(ext) < n:
            break
        # Keep n alternating extrema with the largest errors.
        while len(ext) > n:
            if abs(err[ext[0]]) < abs(err[ext[-1]]):
                ext.pop(0)
            else:
                ext.pop()
        x = grid[ext]
    return c


def fma32(a, b, c):
    """float32 fused multiply-add: a*b is exact in float64, one rounding."""
    return (a.astype(np.float64) * b + c).astype(np.float32)


def eval32(c32, f):
    """Horner in float32 with FMAs, highest coefficient first."""
    acc = np.full_like(f, c32[-1])
    for ci in c32[-2::-1]:
        acc = fma32(acc, f, np.float32(ci))
    return acc


def coefficients(degree: int = 3):
    return np.asarray(remez(degree), dtype=np.float32)


def main():
    degree = int(sys.argv[1]) if len(sys.argv) > 1 else 3
    c32 = coefficients(degree)
    f = np.linspace(LO, HI, 2000001, dtype=np.float32)
    rel = eval32(c32, f).astype(np.float64) / np.exp2(f.astype(np.float64)) - 1
    for i, ci in enumerate(c32):
        print(f"c{i} = {float(ci).hex()}  ({float(ci):.9g})")
    print(f"max relative error in float32: {np.abs(rel).max():.3e}")


if __name__ == "__main__":
    main()
