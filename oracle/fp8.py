"""FP8 E4M3 codec and the per-(token, kv head) KV quantiser (test infrastructure only).

[P2] §3.3 names FP8 as a 1-byte-per-element KV-cache format and calls it
nearly lossless; it does not fix the encoding.  The reading taken is the OCP
8-bit floating point specification's E4M3 ("E4M3FN"): sign, 4 exponent bits
with bias 7, 3 mantissa bits; exponent field 0 holds subnormals m/8 * 2**-6;
there is no infinity; S.1111.111 is NaN, so the largest finite magnitude is
S.1111.110 = 1.75 * 2**8 = 448.

The encoder below works from the table of representable values, not from bit
tricks: it finds the two neighbouring table values of |y|, takes the nearer,
and on an exact tie the one whose code is even; magnitudes beyond 448
saturate to 448 (the KV quantiser never produces them, see ``quantize_rows``).

Quantiser (reading of [P2] §3.3 with per-token-per-head absmax scales): for
each row x (one token, one kv head, K or V) with amax = max|x| in fp32:
  scale = fp32(amax / 448)
  inv   = fp32(448 / amax)
  code  = e4m3_rne_sat(fp32(x * inv))
and amax == 0 gives scale 0 and all-zero codes.  All three roundings are
binary32 round-to-nearest, done with numpy float32 arithmetic.
"""
from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0


def decode_table() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for S.1111.111)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def decode(codes) -> np.ndarray:
    return decode_table()[np.asarray(codes, dtype=np.uint8)]


def _positive_table():
    t = decode_table()[:0x7F]              # codes 0x00..0x7E: 0 .. 448, increasing
    assert np.all(np.diff(t) > 0)
    return t


def encode(y) -> np.ndarray:
    """float array -> uint8 E4M3 codes, round to nearest, ties to even code,
    finite overflow saturates to +-448; the sign bit is copied from y (so -0.0
    and negative values that round to zero give 0x80).  NaN maps to 0x7F."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    table = _positive_table()
    hi = np.searchsorted(table, a, side="left")            # table[hi-1] < a <= table[hi]
    hi = np.minimum(hi, len(table) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= table[-1], len(table) - 1, code)  # saturate at 448
    code = np.where(a == 0, 0, code)
    code = code.astype(np.uint8)
    code = code | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)   # sign-magnitude: -0 -> 0x80
    code = np.where(np.isnan(y), 0x7F, code).astype(np.uint8)
    return code


def quantize_rows(x_f32) -> tuple:
    """Quantise each row of a float32 array (rows = (token, kv head) vectors).

    Returns (codes uint8 same shape, scale float32 per row)."""
    x = np.asarray(x_f32, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    lim = np.float32(MAX_FINITE)
    with np.errstate(divide="ignore", invalid="ignore"):
        scale = (amax / lim).astype(np.float32)
        inv = (lim / amax).astype(np.float32)
    inv = np.where(amax == 0, np.float32(0), inv).astype(np.float32)
    y = (x * inv[..., None]).astype(np.float32)
    codes = encode(y)
    return codes, scale.astype(np.float32)


# ---------------------------------------------------------------------------
# Power-of-two row scales (fp8 operands of the attention scores).
#
# [P2] §2.3 lists FP8 inputs with wider accumulation and the softmax kept in
# higher precision; it fixes no scale format.  The reading taken for the
# attention scores: each row (one token, one head) gets a scale that is a
# power of two, 2**e, with e the smallest integer in [-127, 127] for which
# amax * 2**-e <= 448, so the row's largest magnitude lands in (224, 448] and
# nothing saturates; the codes are E4M3 (round to nearest even) of
# y * 2**-e, which is exact scaling.  The scale is stored as the byte e + 127
# (the OCP microscaling E8M0 form: value 2**(byte - 127)).  amax == 0 (or a
# row so small that e would fall below -127) takes e = -127.

def pow2_exponent(amax) -> np.ndarray:
    """Smallest integer e in [-127, 127] with amax * 2**-e <= 448 (array)."""
    a = np.asarray(amax, dtype=np.float64)
    m, E = np.frexp(a)                        # a = m * 2**E, m in [0.5, 1) (0 -> m = 0)
    # 448 = 0.875 * 2**9: m * 2**(E - e) <= 0.875 * 2**9
    e = np.where(m <= 0.875, E - 9, E - 8)
    e = np.where(a == 0, -127, e)
    return np.maximum(e, -127).astype(np.int64)


def quantize_rows_pow2(y_f32) -> tuple:
    """Rows of a float32 array -> (codes uint8, scale bytes uint8 = e + 127)."""
    y = np.asarray(y_f32, dtype=np.float32)
    amax = np.max(np.abs(y), axis=-1).astype(np.float64)
    e = pow2_exponent(amax)
    scaled = y.astype(np.float64) * np.ldexp(1.0, -e)[..., None]     # exact: a power of two
    return encode(scaled), (e + 127).astype(np.uint8)


def decode_rows_pow2(codes, scale_bytes) -> np.ndarray:
    """fp64 values code * 2**(byte - 127), rows along the last axis."""
    e = np.asarray(scale_bytes, dtype=np.int64) - 127
    return decode(codes) * np.ldexp(1.0, e)[..., None]
