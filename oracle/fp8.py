"""OCP FP8 e4m3 codec and per-tensor quantisation.  TEST INFRASTRUCTURE ONLY.

The FlashAttention-3 summary (GeekNews), sections «Principais tecnologias do
FlashAttention-3» and «Novos recursos de hardware da GPU Hopper», names FP8
as the low-precision input format of the fast path.  The pages give neither
the FP8 variant nor a scaling scheme, so this module takes these readings:

* Format: OCP 8-bit floating point E4M3 ("e4m3fn"): 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits.  Exponent field 0 holds the subnormals
  (value = 2^-6 * m/8); exponent fields 1..15 hold normals
  (value = 2^(e-7) * (1 + m/8)), except that e = 15, m = 7 is NaN.  There are
  no infinities.  Largest finite value 448, smallest normal 2^-6, smallest
  subnormal 2^-9.
* Encoding: round to the nearest representable value, ties to the value with
  an even mantissa (the even code), and saturate finite values beyond +-448
  to +-448.  NaN encodes as 0x7F.
* Per-tensor scaling: delta = amax / 448 where amax is the largest magnitude
  in the tensor (after the optional rotation), so the largest entry maps to
  the largest finite code.  Encoding multiplies by inv = 448 / amax in fp32
  and rounds that fp32 product: the same precision the GPU kernel decides
  the code in.  amax = 0 gives delta = inv = 1.

Parity status: the decoder is pinned against torch's float8_e4m3fn for all
256 codes and against the format's landmark values; the encoder against
torch's rounding cast on about a million values (ties and subnormals
included) and a brute-force nearest-value search; quantisation against the
invariants that codes decode to within half a step of x*inv and that amax
maps to 448 (tests/test_oracle_fp8.py).
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _decode_code(c: int) -> float:
    """Value of one e4m3 code, straight from the bit-field definition."""
    sign = -1.0 if (c >> 7) & 1 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (2.0 ** -6) * (m / 8.0)
    return sign * (2.0 ** (e - 7)) * (1.0 + m / 8.0)


def e4m3_table() -> np.ndarray:
    """float64 value of every code 0..255 (index = code)."""
    return np.array([_decode_code(c) for c in range(256)], dtype=np.float64)


_TABLE = e4m3_table()
# Non-negative finite values in code order 0x00..0x7E; strictly increasing.
_POS = _TABLE[:0x7F]


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _TABLE[codes]


def e4m3_encode(x) -> np.ndarray:
    """Float values -> uint8 e4m3 codes (round-to-nearest-even, saturating).

    Works on the exact float64 value of each input.  For |x| <= 448 the two
    neighbouring representable magnitudes are found in the sorted table; the
    nearer one wins, and on a tie the even code wins."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    nan = np.isnan(flat)
    a = np.minimum(np.abs(np.where(nan, 0.0, flat)), E4M3_MAX)  # saturate
    hi = np.searchsorted(_POS, a, side="left")       # _POS[hi] >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == _POS[hi], hi, np.where(pick_hi, hi, lo))
    neg = np.signbit(flat)
    code = code | np.where(neg, 0x80, 0)
    code = np.where(nan, 0x7F, code)
    out[:] = code.astype(np.uint8)
    return out.reshape(x.shape)


def quantize_per_tensor(x, signs=None):
    """Per-tensor e4m3 quantisation with optional random-sign Hadamard
    rotation of the last dimension.

    x: float32 array [..., d].  signs: None or a length-d array of +-1.
    Returns (codes uint8 [..., d], descale np.float32, amax np.float32).
    The dequantised tensor is e4m3_decode(codes) * descale.
    """
    x = np.asarray(x, dtype=np.float32)
    if signs is not None:
        from .hadamard import rotate
        xr = rotate(x, signs).astype(np.float32)     # fp64 rotation, fp32 result
    else:
        xr = x
    amax = np.float32(np.max(np.abs(xr))) if xr.size else np.float32(0.0)
    if amax == 0.0:
        inv = np.float32(1.0)
        descale = np.float32(1.0)
    else:
        inv = np.float32(E4M3_MAX) / amax             # fp32 division
        descale = amax / np.float32(E4M3_MAX)         # fp32 division
    y = (xr * inv).astype(np.float32)                 # fp32 product
    return e4m3_encode(y), np.float32(descale), np.float32(amax)
