"""Causal attention with fp8 (E4M3) score operands (test infrastructure only).

[P2] §2.3 lists FP8 operands with wider accumulation among the prefill
levers, with the softmax kept in higher precision.  Reading taken here for
the attention scores (the P V product and the softmax stay as in
``oracle.attention``):

  * K arrives quantised per (token, kv head) with a power-of-two scale
    (``fp8.quantize_rows_pow2``, on K itself).
  * Q is quantised the same way per (token, head), after being multiplied by
    c = RN32(scale * RN32(log2 e)) in binary32 (one rounding per element), so
    that the dequantised scores are already in log2 units.
  * The scores are the exact products of the dequantised operands, and the
    softmax is taken in base 2: p_c proportional to 2**(s2_c), which is the
    natural-base softmax of s2 * ln 2.  Everything after that is the plain
    definition (explicit causal mask, two-pass softmax, P V), i.e.
    ``oracle.attention.varlen_causal_attention`` on the dequantised Q and K
    with the scale ln 2.
"""
from __future__ import annotations

import numpy as np

from . import attention, bf16, fp8

LOG2E_F32 = np.float32(1.4426950408889634)


def score_factor(scale: float) -> np.float32:
    """c = RN32(RN32(scale) * RN32(log2 e))."""
    return np.float32(np.float32(scale) * LOG2E_F32)


def quantize_q(q_bits, scale: float) -> tuple:
    """q: bf16 bit patterns (T, n_head, hd) -> (codes, scale bytes (T, n_head))."""
    qf = bf16.to_f64(np.asarray(q_bits)).astype(np.float32)
    return fp8.quantize_rows_pow2((qf * score_factor(scale)).astype(np.float32))


def fp8qk_attention(q_bits, k_codes, k_scale_bytes, v, cu_seqlens, scale: float, rows=None) -> np.ndarray:
    """q: bf16 bits (T, n_head, hd); k_codes (T, n_kv, hd) with scale bytes
    (T, n_kv); v (T, n_kv, hd) bf16 bits or fp64.  Returns fp64 (rows or T,
    n_head*hd)."""
    qc, qe = quantize_q(q_bits, scale)
    qd = fp8.decode_rows_pow2(qc, qe)
    kd = fp8.decode_rows_pow2(k_codes, k_scale_bytes)
    return attention.varlen_causal_attention(qd, kd, v, cu_seqlens, scale=float(np.log(2.0)), rows=rows)
