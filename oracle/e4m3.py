"""OCP FP8 E4M3 codec (test infrastructure only).

The FP8 format the pages use: 1 sign bit, 4 exponent bits, 3 mantissa bits
("FlashAttention 2 & 3" page, "Why FP8 attention is hard"), largest finite
magnitude 448 ("FlashAttention-3: How Warp Specialization ..." page, section
4 "Technique 3: Low-Precision FP8 Attention with Error Mitigation"; the same
448 appears in the first page's fake quantiser). The pages fix neither the
exponent bias, the subnormals, the NaN encoding nor the rounding; this module
takes the OCP E4M3FN reading, which is the only common 1-4-3 format whose
largest finite value is 448:

- exponent bias 7; exponent field 0 encodes subnormals m/8 * 2^-6;
- no infinities; the all-ones pattern S.1111.111 is NaN, so the largest
  finite magnitude is 1.75 * 2^8 = 448 (code 0x7e);
- encoding rounds to nearest, ties to the even code, and saturates magnitudes
  at or above 448 to +-448; NaN encodes to 0x7f; the sign of zero and of values
  that round to zero is kept (0x80 is -0).

The encoder works from the sorted table of the 127 non-negative finite
values: it picks the nearest table entry, and on an exact tie the entry with
an even code. Inputs are compared in float64, so float32 inputs are handled
exactly (every E4M3 value and every midpoint between neighbours is exact in
float32).
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_BIAS = 7


def _decode_magnitude(code7: np.ndarray) -> np.ndarray:
    """Magnitude for the low 7 bits of a code (exponent and mantissa fields)."""
    e = (code7 >> 3) & 0xF
    m = code7 & 0x7
    sub = m.astype(np.float64) / 8.0 * 2.0 ** (1 - _BIAS)
    norm = (1.0 + m.astype(np.float64) / 8.0) * np.exp2(e.astype(np.float64) - _BIAS)
    return np.where(e == 0, sub, norm)


def e4m3_decode(codes) -> np.ndarray:
    """Decode uint8 codes to float64 values (0x7f and 0xff decode to NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = _decode_magnitude(c & 0x7F)
    val = np.where((c & 0x80) != 0, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


# Non-negative finite values, indexed by code 0x00..0x7e (monotonically increasing).
_TABLE = _decode_magnitude(np.arange(0x7F, dtype=np.int64))


def e4m3_encode(x) -> np.ndarray:
    """Encode values to uint8 E4M3 codes: nearest, ties to even code, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # index of the largest table entry <= a (clipped into the table)
    lo = np.clip(np.searchsorted(_TABLE, a, side="right") - 1, 0, len(_TABLE) - 1)
    hi = np.minimum(lo + 1, len(_TABLE) - 1)
    mid = 0.5 * (_TABLE[lo] + _TABLE[hi])
    pick_hi = (a > mid) | ((a == mid) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)               # saturate (covers +inf)
    code = np.where(np.signbit(x), code | 0x80, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)
