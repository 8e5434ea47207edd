"""Random-sign Hadamard rotation for "incoherent processing".  TEST
INFRASTRUCTURE ONLY.

The FlashAttention-3 summary (GeekNews), section «Baixa precisão: redução do
erro de quantização com processamento incoerente», says a Hadamard transform
is applied before FP8 quantisation to lower the quantisation error.  The page
gives no further detail; the reading used here:

* H_d is the Sylvester Hadamard matrix of order d (a power of two):
  H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]].  H_d H_d^T = d I.
* The rotation is R = diag(s) H_d / sqrt(d) with a random +-1 vector s of
  length d.  R is orthonormal (R R^T = I), so rotating both Q and K by the
  same R leaves Q K^T, and with it the attention scale and result,
  unchanged.  V is not rotated.
* Rows are rotated independently: x' = x R, i.e. x'_j = sum_i x_i s_i H_ij /
  sqrt(d).

Parity status: pinned against scipy.linalg.hadamard, the identities
H H^T = d I and R R^T = I, norm preservation and (QR)(KR)^T = QK^T
(tests/test_oracle_hadamard.py).
"""

from __future__ import annotations

import numpy as np


def sylvester(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (power of two), float64."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate(x, signs) -> np.ndarray:
    """x [..., d] -> x diag(signs) H_d / sqrt(d), float64, by the dense
    matrix product."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    s = np.asarray(signs, dtype=np.float64).reshape(d)
    if not np.all(np.abs(s) == 1.0):
        raise ValueError("signs must be +-1")
    r = (s[:, None] * sylvester(d)) / np.sqrt(d)
    return x @ r
