"""Number formats the codec stores or rounds to, written from their definitions.

Test infrastructure only: nothing on the product path imports this module.

* bfloat16: 8 significant bits (1 implicit + 7 stored), 8 exponent bits; the
  codec rounds k-means distance operands and bf16 centroids to it
  (round to nearest, ties to even).
* FP8 E4M3FN as defined by the OCP 8-bit floating point specification:
  exponent bias 7, 3 mantissa bits, no infinities, NaN only at S.1111.111,
  largest finite 448, subnormals down to 2^-9.  The pages store the per-group
  scales in this format (163.com article, section 5, implementation details;
  the same format is named in the gist.science summaries, section 2C).
"""
from __future__ import annotations

import numpy as np

__all__ = ["bf16_round", "E4M3_MAX", "e4m3_values", "e4m3_encode", "e4m3_decode"]


def bf16_round(x) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even; returns float64.

    A finite x = m * 2^e with 0.5 <= |m| < 1 lies between consecutive bf16
    values spaced 2^(e-8) apart (2^-133 in the subnormal range), so the result
    is rint(x / spacing) * spacing with rint rounding half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    spacing = np.ldexp(1.0, e - 8)
    return np.rint(x / spacing) * spacing


E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """Value of every non-negative finite E4M3FN code 0x00..0x7E (float64)."""
    codes = np.arange(0x7F)
    E = codes >> 3
    m = codes & 7
    sub = m * 2.0 ** -9
    nor = (1.0 + m / 8.0) * np.ldexp(1.0, E - 7)
    return np.where(E == 0, sub, nor)


_E4M3 = e4m3_values()


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3FN code to each value (ties to the even code), saturating
    magnitudes above 448 to 448.  Returns uint8 codes (sign in bit 7)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_E4M3, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_E4M3) - 1)
    lo = np.where(_E4M3[hi] == a, hi, np.maximum(hi - 1, 0))
    d_lo = a - _E4M3[lo]
    d_hi = _E4M3[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(v) & (code != 0)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    """Value of E4M3FN codes (float64); 0x7F / 0xFF decode to NaN."""
    code = np.asarray(code, dtype=np.int64)
    mag = code & 0x7F
    val = np.where(mag == 0x7F, np.nan, _E4M3[np.minimum(mag, 0x7E)])
    return np.where(code & 0x80, -val, val)
