"""The 8-bit floating-point code of fp8 caches -- TEST INFRASTRUCTURE ONLY
(same rule as ``oracle.oracle``).

The pages define no 8-bit floating-point format (their only quantization rule
is the integer one of ``oracle.quant``).  The reading taken for fp8 caches is
the OCP 8-bit floating-point format E4M3 ("e4m3fn"), the fp8 format gfx950
converts natively:

* one sign bit, four exponent bits with bias 7, three mantissa bits;
* exponent field 0 encodes subnormals ``m * 2^-9`` (m = 0..7);
* exponent field e = 1..15 encodes ``(1 + m / 8) * 2^(e - 7)``, except that
  e = 15 with m = 7 is NaN (no infinities), so the largest finite magnitude is
  ``1.75 * 2^8 = 448``.

Codes are handled as uint8 bit patterns.  ``decode`` is the definition above
written out; ``encode`` rounds a value of magnitude at most 448 to the nearest
representable magnitude, ties to the even code (mantissa bit 0 clear), and
copies the sign bit of the value (so negative values that round to zero give
the code of -0).
"""

from __future__ import annotations

import numpy as np

__all__ = ["E4M3_MAX", "decode_e4m3", "encode_e4m3"]

E4M3_MAX = 448.0


def _magnitude(code: int) -> float:
    """Magnitude of a code's low seven bits (NaN for the NaN pattern)."""
    e, m = (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return m * 2.0 ** -9                       # subnormal
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)        # normal


_MAG = np.array([_magnitude(c) for c in range(128)], dtype=np.float64)     # codes 0..127
_FINITE = _MAG[:127]                                                        # 0..126 (127 is NaN)


def decode_e4m3(codes) -> np.ndarray:
    """uint8 codes -> float64 values, exactly."""
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError("fp8 codes are a uint8 array of bit patterns")
    mag = _MAG[c & 0x7F]
    return np.where(c & 0x80, -mag, mag)


def encode_e4m3(x) -> np.ndarray:
    """Values of magnitude <= 448 (any float type) -> uint8 codes: the nearest
    representable magnitude, ties to the even code, the value's sign bit."""
    v = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("encode takes finite values of magnitude at most 448")
    a = np.abs(v).reshape(-1)
    # Candidates: the largest representable magnitude <= a and the next one up.
    lo = np.searchsorted(_FINITE, a, side="right") - 1          # _FINITE[lo] <= a
    hi = np.minimum(lo + 1, len(_FINITE) - 1)
    d_lo = a - _FINITE[lo]
    d_hi = _FINITE[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = np.signbit(v).reshape(-1).astype(np.uint8) << 7
    return (mag | sign).reshape(v.shape).astype(np.uint8)
