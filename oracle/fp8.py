"""FP8 E4M3 KV-cache codes for the oracle. TEST INFRASTRUCTURE ONLY.

The pages name an FP8 KV cache ("vLLM PagedAttention explained", section 7:
``--kv-cache-dtype fp8`` halves the bytes of a block) without fixing a format
or a scale. Readings used here:

* Format: the OCP 8-bit floating point E4M3 format ("OCP 8-bit Floating
  Point Specification (OFP8)", E4M3): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 holds subnormals m * 2^-9; no infinities;
  S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
* Scale: one float per pool (``k_scale`` for K, ``v_scale`` for V). A value x
  (bf16 or fp32) is stored as the code of y = fp32(x) / fp32(scale) (an IEEE
  single-precision division), clamped to [-448, 448] and rounded to the
  nearest E4M3 value, ties to even mantissa. A stored code c stands for
  decode(c) * scale.
* Values the format cannot hold (the pages say nothing; reading of this
  library): a quotient beyond +-448, +-infinity included, saturates to the
  largest finite code of its sign (0x7E / 0xFE); a NaN input, whatever its
  sign or payload, is stored as the NaN code 0x7F.

Everything is written from the format definition: the table of the 128
non-negative codes comes from sign/exponent/mantissa, and encoding picks the
nearest entry of that table.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each uint8 code (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


# the finite non-negative magnitudes, code 0 .. 126, increasing
_MAGS = e4m3_decode(np.arange(127, dtype=np.uint8))


def e4m3_encode(y) -> np.ndarray:
    """Nearest E4M3 code of each finite float with |y| <= 448, ties to the code
    with an even mantissa (even code). The sign bit follows the sign of y, so
    -0.0 and negative values that round to zero give 0x80."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    if np.any(a > E4M3_MAX) or not np.all(np.isfinite(a)):
        raise ValueError("e4m3_encode takes finite values with |y| <= 448")
    hi = np.clip(np.searchsorted(_MAGS, a, side="left"), 0, 126)  # first magnitude >= a
    lo = np.clip(hi - 1, 0, 126)
    d_hi = _MAGS[hi] - a
    d_lo = a - _MAGS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    mag = np.where(pick_lo, lo, hi).astype(np.uint8)
    return np.where(np.signbit(y), mag | np.uint8(0x80), mag).astype(np.uint8)


NAN_CODE = 0x7F


def quantize(x, scale: float) -> np.ndarray:
    """Codes of the values x under one pool scale (see the module docstring)."""
    with np.errstate(over="ignore", invalid="ignore"):
        y = np.asarray(x, dtype=np.float32) / np.float32(scale)
    nan = np.isnan(y)
    codes = e4m3_encode(np.clip(np.where(nan, np.float32(0), y), -E4M3_MAX, E4M3_MAX))
    return np.where(nan, np.uint8(NAN_CODE), codes).astype(np.uint8)


def dequantize(codes, scale: float) -> np.ndarray:
    """float64 values the codes stand for."""
    return e4m3_decode(codes) * float(scale)
