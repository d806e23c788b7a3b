"""binary16 rounding for the oracle (test infrastructure; see the package docstring).

The pages do not name the storage type of the row factors and column scales;
the oracle stores them as IEEE binary16 (round to nearest, ties to even),
saturated at the largest finite value.  The rounding is written here from the
format's definition (11 significant bits, minimum normal exponent -14, spacing
2^-24 below it) so that it does not depend on how a library converts.
"""
from __future__ import annotations

import numpy as np

FP16_MAX = 65504.0
FP16_MIN_NORMAL = 2.0 ** -14


def fp16_round(x) -> np.ndarray:
    """Nearest binary16 value of float64 x (ties to even), saturating at +-65504; float64 result."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                      # a = m * 2**e with 0.5 <= m < 1
    e = np.where(a > 0, e - 1, -14)         # floor(log2 a)
    e = np.maximum(e, -14)                  # subnormal binade shares the spacing of 2^-14
    ulp = np.ldexp(1.0, e - 10)             # 11 significant bits
    r = np.rint(a / ulp) * ulp              # a / ulp is exact (power-of-two scaling)
    r = np.minimum(r, FP16_MAX)
    return np.copysign(r, x)


def fp16_bits(x) -> np.ndarray:
    """binary16 bit patterns (uint16) of values that are already binary16 values."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def fp16_from_bits(b) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def fp32_round(x) -> np.ndarray:
    """Nearest binary32 value (the storage type of the INT8 comparator's row scales)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
