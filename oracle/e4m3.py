"""OCP FP8 E4M3 ("e4m3fn") codec written from the format definition.

Format (OCP 8-bit floating point spec; the e4m3fn dtype named in the
per_token_group_quant_fp8 reference implementation on the atrex-bench page):
  sign(1) | exponent(4, bias 7) | mantissa(3)
  exponent 0      : subnormal, value = (-1)^s * m/8 * 2^(1-7)
  exponent 1..15  : normal,    value = (-1)^s * (1 + m/8) * 2^(e-7)
  S.1111.111      : NaN (no infinities); largest finite = 0x7E = 448.

Oracle code: used only by tests, smoke() and the bench's CPU baseline.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def decode_one(code: int) -> float:
    """Value of one code, from the bit fields (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    s = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# Table of all 256 code values (float64, exact).
DECODE_TABLE = np.array([decode_one(c) for c in range(256)], dtype=np.float64)

# Non-negative finite codes 0x00..0x7E in increasing value order (code == index).
_POS_VALUES = DECODE_TABLE[:0x7F].copy()
assert np.all(np.diff(_POS_VALUES) > 0)


def decode(codes: np.ndarray) -> np.ndarray:
    """Decode uint8 codes to float64 values."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_rne(y: np.ndarray) -> np.ndarray:
    """Round each float32 value to the nearest e4m3 code, ties to the even code.

    Magnitudes above 448 saturate to 448 (the method clamps before casting,
    so this only matters for callers that skip the clamp). The sign bit is
    always kept: a negative value that rounds to zero gives 0x80. NaN inputs
    are outside the contract and map to the NaN code with their sign.
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    neg = np.signbit(y)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    hi = np.searchsorted(_POS_VALUES, a, side="left")        # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    pick_lo = (dlo < dhi) | ((dlo == dhi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    code = np.where(a == _POS_VALUES[hi], hi, code).astype(np.uint8)   # exact hits
    code = np.where(nan, NAN_CODE, code).astype(np.uint8)
    return (code | np.where(neg, 0x80, 0).astype(np.uint8)).astype(np.uint8)
