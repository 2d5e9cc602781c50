"""OCP E4M3FN (8-bit float, 4 exponent bits, 3 mantissa bits) codec, fp64.

The pages only say that an fp8 KV cache stores one byte per element
([P2] question 1, sub-section 1.3).  The format is read as OCP E4M3FN:
bias 7, no infinities, the all-ones pattern S.1111.111 is NaN, the largest
finite magnitude is 448 and the smallest subnormal 2^-9.

Decode: value(code) * scale.  Encode (cache write): y = fp32(x) / fp32(scale)
as one correctly rounded fp32 division, then round y to the nearest
representable E4M3 value, ties to the code with an even mantissa, magnitudes
past 448 saturate to +-448, NaN stays NaN (sign kept), and the sign of zero
is kept.

Pins (tests/test_oracle_fp8.py): the decode table is compared code by code
with torch's float8_e4m3fn -> float32 conversion and with constants of the
OCP format; the encoder with torch's round-to-nearest-even cast (after
clamping to +-448) over random, boundary and midpoint values.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def decode_table() -> np.ndarray:
    """fp64 value of each of the 256 codes (NaN for the two NaN codes)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_TABLE = decode_table()
# Non-negative finite values, codes 0x00..0x7E, increasing with the code.
_POS = _TABLE[:0x7F].copy()


def decode(codes: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """codes (uint8) -> fp64 values times scale."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)] * float(scale)


def round_to_e4m3(y: np.ndarray) -> np.ndarray:
    """fp32/fp64 values -> uint8 codes: nearest, ties to even, saturating."""
    y = np.asarray(y, dtype=np.float64)
    sign = np.signbit(y)
    a = np.abs(y)
    nan = np.isnan(y)
    a = np.where(nan, 0.0, a)
    # index of the first representable value >= a
    hi = np.searchsorted(_POS, a, side="left")
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = np.abs(_POS[hi] - a)
    d_lo = np.abs(a - _POS[lo])
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    # on a tie take the even code (mantissa LSB clear)
    pick_hi = np.where(tie, (hi % 2) == 0, pick_hi)
    code = np.where(pick_hi, hi, lo).astype(np.int64)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = np.where(nan, NAN_CODE, code)
    code = code | np.where(sign, 0x80, 0)
    return code.astype(np.uint8)


def quantize(x_f32: np.ndarray, scale: float) -> np.ndarray:
    """Cache-write quantiser: one fp32 division by the scale, then rounding."""
    x = np.asarray(x_f32, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        y = x / np.float32(scale)
    return round_to_e4m3(y)
