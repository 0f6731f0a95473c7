"""The two ends of the attention unit around the path (test infrastructure only).

[P1] §2.1 writes the decoder layer as: keep the input as the residual,
RMS-normalise it, project to Q, K, V with one fused weight, attend, and add
the attention output back onto the residual; §3.3 flattens the heads back to
(s, h) so the output projection W_o can consume them, and the residual add
follows that projection (the §2.1 sketch folds W_o into "attention").

  * ``rms_norm(x, g, eps)``: x / sqrt(mean_k x[:, k]^2 + eps) * g, per row
    (the usual RMSNorm; the pages name it without a formula, so the plain
    definition is taken, with eps a parameter).
  * ``out_projection_residual(o, w_o, res)``: res + o @ W_o, W_o of shape
    (n_head*hd, h) as drawn.
"""
from __future__ import annotations

import numpy as np

from . import bf16


def rms_norm(x, g, eps: float) -> np.ndarray:
    """fp64 RMSNorm of the rows of x (values or bf16 bit patterns) with gain g."""
    x = bf16.to_f64(x) if np.asarray(x).dtype == np.uint16 else np.asarray(x, dtype=np.float64)
    g = bf16.to_f64(g) if np.asarray(g).dtype == np.uint16 else np.asarray(g, dtype=np.float64)
    r = np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    return x / r * g[None, :]


def out_projection_residual(o_bits, w_bits, res_bits, rows=None) -> np.ndarray:
    """res + O @ W_o in fp64 from bf16 bit patterns; O (T, K), W_o (K, N), res (T, N)."""
    o = np.asarray(o_bits)
    res = np.asarray(res_bits)
    if rows is not None:
        o, res = o[np.asarray(rows)], res[np.asarray(rows)]
    return bf16.to_f64(res) + bf16.to_f64(o) @ bf16.to_f64(w_bits)
