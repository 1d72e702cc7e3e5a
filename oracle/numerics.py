"""Rounding helpers of the oracle (float64 throughout).

* ``fp16``: IEEE binary16 round-to-nearest-even of a float64 value (numpy's
  double-to-half conversion rounds correctly from double).
* ``fp16_scale``: the same after clamping to [2^-14, 65504]; STEPQuant stores
  its INT6 baseline scale as FP16 clamped to that range (appendix B.5) and the
  oracle uses the same clamp for every FP16 scale.
* ``rne``: round half to even ("nearest-integer codes", appendix B.5).
* ``qmax(b)``: 2^(b-1) - 1, the largest code magnitude of a symmetric b-bit
  code (INT6 codes live in [-31, 31], appendix B.5).
* ``fp32``: float32 round-to-nearest-even, for values the layout stores as
  float32 (window scales and records).
"""
from __future__ import annotations

import numpy as np

FP16_MIN_NORMAL = 2.0 ** -14
FP16_MAX = 65504.0
PIVOT_BITS = 16


def fp16(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def fp16_scale(x) -> np.ndarray:
    return fp16(np.clip(np.asarray(x, dtype=np.float64), FP16_MIN_NORMAL, FP16_MAX))


def fp32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def rne(x) -> np.ndarray:
    return np.rint(np.asarray(x, dtype=np.float64))


def qmax(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.int64)
    return (np.left_shift(1, b - 1) - 1).astype(np.float64)


def fp16_neighbours(x) -> tuple:
    """The two binary16 values around ``x`` (after the scale clamp):
    (largest value <= x, smallest value >= x)."""
    x = np.clip(np.asarray(x, dtype=np.float64), FP16_MIN_NORMAL, FP16_MAX)
    r = fp16(x)
    lo = np.where(r <= x, r, np.nextafter(r.astype(np.float16), np.float16(-np.inf)).astype(np.float64))
    hi = np.where(r >= x, r, np.nextafter(r.astype(np.float16), np.float16(np.inf)).astype(np.float64))
    return lo, hi
