"""Number formats used by the cache, written out from their definitions.

TEST INFRASTRUCTURE ONLY: nothing on the product path imports this module.

Contents
--------
* OCP FP8 E4M3FN (4 exponent bits, bias 7, 3 mantissa bits, no infinities, one
  NaN pattern per sign, largest finite 448, smallest subnormal 2^-9).  The
  cartridge page ("Compress the shared cartridge. Keep the keys.", section
  "What fake quantization does with the other eight bits") rounds each value to
  the nearest E4M3 value; we read "nearest" as round-to-nearest, ties to the
  even code, with saturation at +-448 (there is no infinity to overflow to).
* fp16 rounding toward +infinity for the witness (WitCert, Sec. 4.1, Eq. (2):
  the witness is stored in fp16; rounding up keeps Theorem 2 sound after
  storage).
* Exact IEEE fp32 steps are taken with numpy float32 arithmetic, which is one
  correctly rounded IEEE single operation per numpy operation.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Real value of one E4M3FN byte (NaN for 0x7F / 0xFF)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -9          # subnormal: man/8 * 2^(1-7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e4m3_table() -> np.ndarray:
    """All 256 decoded values as float64 (NaN for the two NaN codes)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


_TABLE = e4m3_table()
# non-negative finite magnitudes in code order 0x00..0x7E (strictly increasing)
_POS = _TABLE[:0x7F].copy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y) -> np.ndarray:
    """Round float32 values to E4M3FN codes: nearest, ties to even code, saturate.

    The sign bit of the code is the sign bit of y (so -0.0 and negative values
    that round to zero give 0x80).  Inputs must be finite.
    """
    y = np.asarray(y, dtype=np.float32)
    if not np.all(np.isfinite(y)):
        raise ValueError("e4m3_encode: non-finite input")
    mag = np.abs(y.astype(np.float64))
    mag = np.minimum(mag, E4M3_MAX)
    # index of the largest representable magnitude <= mag
    lo = np.searchsorted(_POS, mag, side="right") - 1
    lo = np.clip(lo, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    d_lo = mag - _POS[lo]
    d_hi = _POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & ((lo & 1) == 1))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(y)
    return (code | np.where(neg, 0x80, 0).astype(np.uint8)).astype(np.uint8)


def f32(x) -> np.ndarray:
    """Round to the nearest float32 (ties to even), as numpy does."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def fp16_round_up(w) -> np.ndarray:
    """Smallest fp16 value >= w, for finite w >= 0 (returns float16 array).

    Values above the largest fp16 (65504) become +inf, which is still an upper
    bound.  Exact comparisons are done in float64.
    """
    w = np.asarray(w, dtype=np.float64)
    if np.any(w < 0) or not np.all(np.isfinite(w)):
        raise ValueError("fp16_round_up expects finite non-negative values")
    with np.errstate(over="ignore"):
        h = w.astype(np.float16)                  # round to nearest even
    below = h.astype(np.float64) < w
    if np.any(below):
        bits = h.view(np.uint16).copy()
        bits[below] += 1                          # next fp16 toward +inf (w >= 0)
        h = bits.view(np.float16)
    return h


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even) bit patterns.

    Written from the definition: bf16 keeps the upper 16 bits of a float32; the
    value is first rounded to float32 (exact for the inputs used here) and then
    the discarded low half decides the rounding.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    up = u >> 16
    round_up = (low > 0x8000) | ((low == 0x8000) & ((up & 1) == 1))
    return (up + round_up.astype(np.uint64)).astype(np.uint16)
