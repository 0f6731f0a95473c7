"""bfloat16 codec for the oracle (test infrastructure only).

bf16 = 1 sign bit, 8 exponent bits (bias 127), 7 stored mantissa bits: the top
half of an IEEE binary32.  [P2] §3.3 counts it at 2 bytes per element.
Decoding is exact; encoding rounds an fp64 value straight to the nearest bf16
(ties to even), never through fp32, so there is no double rounding.
"""
from __future__ import annotations

import numpy as np


def to_f64(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def from_f64(x) -> np.ndarray:
    """float64 -> nearest bf16 (RNE) bit patterns, uint16.

    A finite nonzero x is m * 2**e with 0.5 <= |m| < 1 (frexp); bf16 keeps 8
    significant bits, so the nearest value is rint(m * 2**8) * 2**(e - 8) with
    rint rounding halves to even.  Below the normal range (|x| < 2**-126) the
    spacing is fixed at 2**-133.  Values beyond the largest finite bf16 after
    rounding become inf (IEEE round-to-nearest overflow).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)                      # subnormal spacing 2**-133
    q = np.rint(np.ldexp(x, 8 - e))              # exact scaling by a power of two
    y = np.ldexp(q, e - 8)
    with np.errstate(over="ignore"):
        y32 = y.astype(np.float32)               # exact: y has <= 8 significant bits
    bits = (y32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    bits[nan] = np.uint16(0x7FC0)
    return bits
