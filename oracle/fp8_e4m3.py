"""OCP FP8 E4M3 ("e4m3fn") codec for the oracle: test infrastructure only.

Only tests/, the package entry point's smoke check and the benchmark's CPU
baseline leg may import this module; the product path never does.

The format follows its bit-field definition: sign bit, 4 exponent bits with
bias 7, 3 mantissa bits.  With exponent field e and mantissa field m:
  e = 0      : value = m/8 * 2**-6            (subnormals, step 2**-9)
  e = 1..15  : value = (1 + m/8) * 2**(e-7)
  e = 15, m = 7 is NaN, so the largest finite magnitude is 1.75 * 2**8 = 448.
There are no infinities.

Encoding used by the SLA2 low-bit sparse branch (SLA2 page, section 5,
quantisation-aware training: Q and K are mapped to a low-bit format with a
scale): round to the nearest representable value, ties to the even code
(mantissa LSB 0), and saturate magnitudes above 448 to 448.  Negative values
that round to zero keep their sign (code 0x80).
"""
from __future__ import annotations

import numpy as np

FP8_E4M3_MAX = 448.0


def e4m3_magnitudes() -> np.ndarray:
    """fp64 magnitude of codes 0..126 (127 is NaN), ascending in the code."""
    vals = np.empty(127, dtype=np.float64)
    for c in range(127):
        e, m = c >> 3, c & 7
        if e == 0:
            vals[c] = (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_MAG = e4m3_magnitudes()


def decode(codes: np.ndarray) -> np.ndarray:
    """fp64 values of uint8 codes (NaN for 0x7F / 0xFF)."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag_idx = (codes & 0x7F).astype(np.int64)
    table = np.append(_MAG, np.nan)
    out = table[mag_idx]
    return np.where(codes & 0x80, -out, out)


def encode(y: np.ndarray) -> np.ndarray:
    """uint8 codes of finite values y: round to nearest, ties to even, saturate."""
    y = np.asarray(y, dtype=np.float64)
    if np.isnan(y).any():
        raise ValueError("fp8 encode: NaN input")
    a = np.minimum(np.abs(y), FP8_E4M3_MAX)
    # index of the largest representable magnitude <= a
    lo = np.searchsorted(_MAG, a, side="right") - 1
    lo = np.clip(lo, 0, 126)
    hi = np.minimum(lo + 1, 126)
    d_lo = a - _MAG[lo]
    d_hi = _MAG[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(y)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)
