"""OCP fp8 e4m3 storage of the draft KV, written from the format's definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[VERDICT] forward implications: the window composes with KV quantization (fp8).
The pages name the format family, not its details; the readings taken here:

* the format is OCP 8-bit floating point E4M3 ("e4m3fn"): 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
  m * 2^-9; codes 0x7F / 0xFF are NaN and there is no infinity, so the largest
  finite magnitude is 1.75 * 2^8 = 448 (code 0x7E);
* a bf16 value x is stored as code(x * inv_scale) with one float32 scale per
  cache (K and V each), the product taken in float32 (round to nearest even),
  clamped to [-448, 448], then rounded to the nearest e4m3 value with ties to
  the even code (for e4m3 the even code is the one with an even mantissa);
  the sign of zero is kept;
* the attention reads code values times the scale; since every e4m3 value is
  exactly a bf16 value, the attention over the stored cache is plain attention
  over the dequantized keys and values.
"""

from __future__ import annotations

import numpy as np

MAX_E4M3 = 448.0


def e4m3_positive_values() -> np.ndarray:
    """Magnitudes of codes 0 .. 126 (float64): code c = (E << 3) | m encodes
    m * 2^-9 for E = 0 and (1 + m / 8) * 2^(E - 7) otherwise."""
    vals = np.empty(127)
    for c in range(127):
        E, m = c >> 3, c & 7
        vals[c] = m * 2.0 ** -9 if E == 0 else (1.0 + m / 8.0) * 2.0 ** (E - 7)
    return vals


_VALS = e4m3_positive_values()


def quantize_e4m3(x: np.ndarray, inv_scale: float = 1.0) -> np.ndarray:
    """float32 values -> e4m3 codes (uint8), as the reading above states."""
    with np.errstate(over="ignore"):                         # huge inputs saturate below
        y = np.asarray(x, dtype=np.float32) * np.float32(inv_scale)
    y = np.clip(y, np.float32(-MAX_E4M3), np.float32(MAX_E4M3))
    a = np.abs(y).astype(np.float64)
    hi = np.searchsorted(_VALS, a, side="left")            # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _VALS[lo]
    d_hi = _VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _VALS[hi], hi, code)                # exact hits
    sign = np.signbit(y).astype(np.uint8) << 7
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def dequantize_e4m3(codes: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """e4m3 codes -> float64 values times ``scale`` (NaN codes -> NaN)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = c & 0x7F
    v = np.where(mag == 0x7F, np.nan, _VALS[np.minimum(mag, 126)])
    v = np.where(c & 0x80, -v, v)
    return v * float(scale)


def bf16_to_e4m3(bits: np.ndarray, inv_scale: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) -> e4m3 codes: the stored form of a bf16 K or V."""
    f = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    return quantize_e4m3(f, inv_scale)
