"""OCP E4M3FN codec (TEST INFRASTRUCTURE ONLY -- never imported by the product path).

The pages fix the format of every FP8 operand as E4M3 (more mantissa bits than
E5M2), for Fprop, Dgrad and Wgrad alike, with the narrow range recovered by
tile/block scaling ("FP8 mixed precision - где и как DeepSeek снизили точность
вычислений?", section "Использование E4M3 вместо гибридных форматов"). The
pages do not spell out the bit layout; this module uses the OCP 8-bit float
"E4M3FN" definition (sign, 4 exponent bits with bias 7, 3 mantissa bits, no
infinities, only S.1111.111 is NaN, largest finite 448).

Readings where the pages are silent (each pinned in tests/test_oracle_e4m3.py):
    * rounding: round to nearest, ties to the even code;
    * values beyond 448 in magnitude saturate to +-448;
    * the sign of zero and of values that underflow to zero is kept (0x80);
    * non-finite input is rejected (ValueError).
"""

import numpy as np

E4M3_MAX = 448.0
NAN_CODES = (0x7F, 0xFF)


def _decode_one(code: int) -> float:
    """Value of one E4M3FN byte, straight from the field definition."""
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    man_field = code & 0x7
    if exp_field == 0xF and man_field == 0x7:
        return float("nan")
    if exp_field == 0:                      # subnormal: m/8 * 2^(1-7)
        return sign * (man_field / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man_field / 8.0) * 2.0 ** (exp_field - 7)


#: float64 value of every byte 0..255 (NaN at 0x7F and 0xFF).
DECODE_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)

# The 127 non-negative finite magnitudes, codes 0x00..0x7E, strictly increasing.
_MAGNITUDES = DECODE_TABLE[:0x7F].copy()
assert np.all(np.diff(_MAGNITUDES) > 0) and _MAGNITUDES[-1] == E4M3_MAX


def decode(q) -> np.ndarray:
    """Map E4M3FN bytes (uint8 array) to their exact float64 values."""
    q = np.asarray(q)
    if q.dtype != np.uint8:
        raise TypeError("decode expects uint8 codes")
    return DECODE_TABLE[q]


def encode(v) -> np.ndarray:
    """Round finite float32 values to E4M3FN bytes.

    Steps, applied per element:
      1. sign bit = signbit(v) (so -0.0 and negative underflow give 0x80);
      2. magnitude a = min(|v|, 448) (saturation);
      3. the nearest of the 127 finite magnitudes to a; when a lies exactly
         half-way between two neighbours, the one with the even code wins;
      4. the sign bit is OR-ed into the code.
    Every comparison is exact: a float32 magnitude, two E4M3 neighbours and
    their midpoint are all exactly representable in float64.
    """
    v = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("E4M3 encode: non-finite input is not defined")
    sign = np.signbit(v)
    a = np.minimum(np.abs(v).astype(np.float64), E4M3_MAX)
    lo = np.searchsorted(_MAGNITUDES, a, side="right") - 1      # MAG[lo] <= a
    lo = np.clip(lo, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    mid = 0.5 * (_MAGNITUDES[lo] + _MAGNITUDES[hi])
    below = a < mid
    above = a > mid
    tie_pick = np.where(lo % 2 == 0, lo, hi)
    code = np.where(below, lo, np.where(above, hi, tie_pick))
    code = np.where(lo == 0x7E, 0x7E, code)                       # a == 448
    code = code.astype(np.uint8)
    return np.where(sign, code | np.uint8(0x80), code).astype(np.uint8)
