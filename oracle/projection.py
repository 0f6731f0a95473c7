"""Fused QKV projection in fp64 (test infrastructure only).

[P1] §1.2, §2.1 and §4.1: the layer input X (s, h) is multiplied once by the
concatenated weight W_qkv of shape (h, 3h) -- for GQA (h, (n_head + 2*n_kv)*hd)
-- giving (s, N) whose column blocks are Q | K | V.  Here W is taken in that
(h, N) form as drawn; the GPU path receives it pre-transposed to (N, h)
([P1] §5.1), which is a storage choice, not arithmetic.
"""
from __future__ import annotations

import numpy as np

from . import bf16, fp8


def qkv_projection(x_bits, w_bits) -> np.ndarray:
    """Y = X @ W in fp64 from bf16 bit patterns; X (T, h), W (h, N)."""
    return bf16.to_f64(x_bits) @ bf16.to_f64(w_bits)


def projection_entries(x_bits, w_bits, rows, cols) -> np.ndarray:
    """Y[rows][:, cols] only: each sampled entry is one length-h fp64 dot product."""
    x = bf16.to_f64(np.asarray(x_bits)[np.asarray(rows)])
    w = bf16.to_f64(np.asarray(w_bits)[:, np.asarray(cols)])
    return x @ w


def projection_rows(x_bits, w_bits, rows) -> np.ndarray:
    """Whole rows of Y for the sampled token indices."""
    return bf16.to_f64(np.asarray(x_bits)[np.asarray(rows)]) @ bf16.to_f64(w_bits)


def fp8_projection(xq, sx, wq, sw, rows=None) -> np.ndarray:
    """FP8-operand projection ([P2] §2.3: fp8 inputs, wider accumulation) in
    fp64: each operand row is its E4M3 codes decoded times its row scale
    (rows of X are tokens, rows of W^T output features), then Y = Xd @ Wd^T."""
    xq, sx = np.asarray(xq), np.asarray(sx, dtype=np.float64)
    if rows is not None:
        xq, sx = xq[np.asarray(rows)], sx[np.asarray(rows)]
    xd = fp8.decode(xq) * sx[:, None]
    wd = fp8.decode(np.asarray(wq)) * np.asarray(sw, dtype=np.float64)[:, None]
    return xd @ wd.T
