"""Causal GQA attention, the plain definition in fp64 (test infrastructure only).

Follows [P1] §2.3 and §3.1-§3.4 and [P3] §1.1:
  * per query head i, S = Q_i K_g^T / sqrt(head_dim) with g the kv head of i
    (GQA: several consecutive query heads share one kv head, [P1] §3.4,
    [P2] §3.2; the map taken is g = i // (n_head / n_kv_head));
  * the causal rule: a query at position r sees keys c <= r only, built here
    the "data-flow" way, as an explicit additive mask (0 allowed, -inf not;
    [P1] §3.1 prints "1" for allowed entries: a constant per-row shift that
    softmax cancels, so 0 is used);
  * softmax by the naive two-pass method ([P1] §3.2): row max, then exp and
    row sum, then divide;
  * D = P V per head, and the heads flattened back to (s, n_head*head_dim),
    head outer and head_dim inner ([P1] §3.3).
Score rows are materialised whole (full width L); long sequences are handled
a block of whole rows at a time, which changes nothing in the arithmetic.

``online_softmax_attention`` is the blockwise form the pages describe
([P1] §3.2 and §4.3, [P3] §3.1): a double loop over query blocks and kv
blocks, running max m and exp-sum l with rescaling of the old partial
results, and the causal mask as control flow (skip / unmasked / element
mask).  It is an exact rewrite of the plain form; the tests pin the two
together.
"""
from __future__ import annotations

import numpy as np

from . import bf16


def head_split(y, n_head: int, n_kv_head: int, head_dim: int):
    """Split the fused projection output (T, (n_head + 2*n_kv)*hd) into
    Q (T, n_head, hd), K and V (T, n_kv, hd) by explicit column arithmetic
    ([P1] §2.2: columns [Q | K | V], each head a contiguous run of head_dim
    columns, head index outer)."""
    y = np.asarray(y)
    T = y.shape[0]
    q = np.empty((T, n_head, head_dim), dtype=y.dtype)
    k = np.empty((T, n_kv_head, head_dim), dtype=y.dtype)
    v = np.empty((T, n_kv_head, head_dim), dtype=y.dtype)
    k_base = n_head * head_dim
    v_base = (n_head + n_kv_head) * head_dim
    for i in range(n_head):
        q[:, i, :] = y[:, i * head_dim:(i + 1) * head_dim]
    for j in range(n_kv_head):
        k[:, j, :] = y[:, k_base + j * head_dim:k_base + (j + 1) * head_dim]
        v[:, j, :] = y[:, v_base + j * head_dim:v_base + (j + 1) * head_dim]
    return q, k, v


def causal_mask_rows(rows, L: int) -> np.ndarray:
    """Additive mask for the given query rows over all L keys: 0 where
    key c <= row r, -inf where c > r."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.arange(L, dtype=np.int64)
    m = np.zeros((rows.shape[0], L), dtype=np.float64)
    m[cols[None, :] > rows[:, None]] = -np.inf
    return m


def softmax_two_pass(s: np.ndarray) -> np.ndarray:
    """Row softmax, naive: max pass, then exp/sum pass, then divide."""
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    return e / l


def _as_f64(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16.to_f64(x)
    return x.astype(np.float64)


def causal_attention(q, k, v, scale=None, rows=None, row_block: int = 1024) -> np.ndarray:
    """One sequence.  q (L, n_head, hd), k/v (L, n_kv, hd), as fp64 values or
    bf16 bit patterns (uint16).  Returns fp64 (len(rows), n_head*hd); rows
    defaults to all L query positions."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    L, H, D = q.shape
    Hk = k.shape[1]
    assert H % Hk == 0, "n_head must be a multiple of n_kv_head"
    G = H // Hk
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], H * D), dtype=np.float64)
    for i in range(H):
        g = i // G
        kt = k[:, g, :].T
        for a in range(0, rows.shape[0], row_block):
            r = rows[a:a + row_block]
            s = (q[r, i, :] @ kt) * scale
            s = s + causal_mask_rows(r, L)
            p = softmax_two_pass(s)
            out[a:a + row_block, i * D:(i + 1) * D] = p @ v[:, g, :]
    return out


def varlen_causal_attention(q, k, v, cu_seqlens, scale=None, rows=None) -> np.ndarray:
    """Packed sequences: token t of sequence b sits at cu_seqlens[b] + pos.
    Each sequence is attended alone (the causal rule per sequence).  rows, if
    given, are global token indices; returns (len(rows) or T, n_head*hd)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    H, D = np.asarray(q).shape[1], np.asarray(q).shape[2]
    sel = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((sel.shape[0], H * D), dtype=np.float64)
    for b in range(cu.shape[0] - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        pick = np.nonzero((sel >= s0) & (sel < s1))[0]
        if pick.size == 0:
            continue
        out[pick] = causal_attention(np.asarray(q)[s0:s1], np.asarray(k)[s0:s1],
                                     np.asarray(v)[s0:s1], scale, rows=sel[pick] - s0)
    return out


def online_softmax_attention(q, k, v, scale=None, block_q: int = 16, block_k: int = 16) -> np.ndarray:
    """The pages' blockwise algorithm in fp64, one sequence.

    For each query block and head: m = -inf, l = 0, O = 0; then for each kv
    block in order, with the causal rule as control flow ([P1] §4.3, stated
    for unequal block sizes): a kv block whose first key lies after the last
    query of the block is skipped; one whose last key is not after the first
    query is used unmasked; otherwise keys c > r are masked per element.
    Update ([P1] §3.2): m' = max(m, rowmax S); alpha = exp(m - m');
    P = exp(S - m'); l = alpha*l + rowsum P; O = alpha*O + P V_j.  Final O / l.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    L, H, D = q.shape
    G = H // k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((L, H * D), dtype=np.float64)
    for i in range(H):
        g = i // G
        for r0 in range(0, L, block_q):
            r1 = min(L, r0 + block_q)
            qb = q[r0:r1, i, :]
            m = np.full(r1 - r0, -np.inf)
            l = np.zeros(r1 - r0)
            o = np.zeros((r1 - r0, D))
            for c0 in range(0, L, block_k):
                c1 = min(L, c0 + block_k)
                if c0 > r1 - 1:
                    continue                                   # whole block in the future
                s = (qb @ k[c0:c1, g, :].T) * scale
                if c1 - 1 > r0:                                # straddles the diagonal
                    s = s + causal_mask_rows(np.arange(r0, r1), c1)[:, c0:c1]
                m_new = np.maximum(m, np.max(s, axis=1))
                alpha = np.exp(m - m_new)
                p = np.exp(s - m_new[:, None])
                l = alpha * l + np.sum(p, axis=1)
                o = alpha[:, None] * o + p @ v[c0:c1, g, :]
                m = m_new
            out[r0:r1, i * D:(i + 1) * D] = o / l[:, None]
    return out
