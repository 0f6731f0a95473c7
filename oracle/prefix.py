"""Attention of a prefill chunk over a cached prefix (test infrastructure only).

Chunked prefill ([P2] §2.1; [P3] §3.3 runs it with 512-token chunks and
16-token cache blocks): a long prompt is processed a chunk at a time, and the
K/V of the earlier chunks are kept in the paged cache.  A chunk of Lq queries
that follows a prefix of P cached tokens therefore attends, per query head,
to all P + Lq keys of its sequence with the causal rule shifted by P: chunk
row r sits at position P + r and sees keys c <= P + r.  Everything else is the
plain definition of ``oracle.attention`` (scores times 1/sqrt(head_dim),
explicit additive mask, two-pass softmax, P V, heads flattened).

The cached keys are read back through the block table ([P1] §4.2 paged
layout, ``oracle.kvcache.gather``); an fp8 cache is decoded as
code value x its (token, kv head) scale ([P2] §3.3), in fp64.
"""
from __future__ import annotations

import numpy as np

from . import attention, fp8, kvcache


def prefix_causal_attention(q, k, v, prefix_len: int, scale=None, rows=None) -> np.ndarray:
    """One sequence.  q (Lq, n_head, hd): the chunk's queries; k, v
    (prefix_len + Lq, n_kv, hd): every key of the sequence so far (prefix then
    chunk), as fp64 values or bf16 bit patterns.  Row r of the chunk sees keys
    c <= prefix_len + r.  Returns fp64 (len(rows) or Lq, n_head*hd)."""
    q, k, v = attention._as_f64(q), attention._as_f64(k), attention._as_f64(v)
    Lq, H, D = q.shape
    Lk = k.shape[0]
    assert Lk == prefix_len + Lq, "keys must be the prefix followed by the chunk"
    G = H // k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], H * D), dtype=np.float64)
    for i in range(H):
        g = i // G
        s = (q[rows, i, :] @ k[:, g, :].T) * scale
        s = s + attention.causal_mask_rows(rows + prefix_len, Lk)
        p = attention.softmax_two_pass(s)
        out[:, i * D:(i + 1) * D] = p @ v[:, g, :]
    return out


def cached_keys(k_pool, v_pool, block_table, b: int, ctx: int, k_scale=None, v_scale=None, page_size: int = 16):
    """K and V of sequence b, positions 0 .. ctx-1, read through the block
    table.  bf16 pools (uint16 bits) give fp64 values; uint8 pools are E4M3
    codes, decoded and multiplied by their scale in fp64."""
    k = np.empty((ctx,) + k_pool.shape[2:], dtype=k_pool.dtype)
    v = np.empty_like(k)
    ks = vs = None
    if k_scale is not None:
        ks = np.empty((ctx, k_pool.shape[2]), dtype=np.float64)
        vs = np.empty_like(ks)
    for pos in range(ctx):
        page, slot = kvcache._slot(block_table, b, pos, page_size)
        k[pos] = k_pool[page, slot]
        v[pos] = v_pool[page, slot]
        if ks is not None:
            ks[pos] = k_scale[page, slot]
            vs[pos] = v_scale[page, slot]
    if k_pool.dtype == np.uint8:
        kf = fp8.decode(k) * ks[:, :, None]
        vf = fp8.decode(v) * vs[:, :, None]
        return kf, vf
    return attention._as_f64(k), attention._as_f64(v)


def paged_prefix_attention(q, cu_q, ctx_lens, k_pool, v_pool, block_table, scale=None, k_scale=None,
                           v_scale=None, rows=None, page_size: int = 16) -> np.ndarray:
    """Packed chunks: sequence b's queries are rows cu_q[b] .. cu_q[b+1]-1 of q
    (T, n_head, hd) and its keys are the first ctx_lens[b] positions in the
    cache (the prefix, then the chunk itself), so its prefix length is
    ctx_lens[b] - (cu_q[b+1] - cu_q[b]).  rows, if given, are global query
    indices.  Returns fp64 (len(rows) or T, n_head*hd)."""
    cu = np.asarray(cu_q, dtype=np.int64)
    T = int(cu[-1])
    q = np.asarray(q)
    H, D = q.shape[1], q.shape[2]
    sel = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((sel.shape[0], H * D), dtype=np.float64)
    for b in range(cu.shape[0] - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        pick = np.nonzero((sel >= s0) & (sel < s1))[0]
        if pick.size == 0:
            continue
        ctx = int(ctx_lens[b])
        k, v = cached_keys(k_pool, v_pool, block_table, b, ctx, k_scale, v_scale, page_size)
        out[pick] = prefix_causal_attention(q[s0:s1], k, v, ctx - (s1 - s0), scale, rows=sel[pick] - s0)
    return out


def window_mask_rows(rows, L: int, window: int) -> np.ndarray:
    """Additive mask of the sliding-window causal rule ([P3] §4.1: each token
    attends only to a window of W recent positions, O(n W) work instead of
    O(n^2)): row r sees keys c with r - W < c <= r (W keys, itself included);
    window <= 0 means no lower bound."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.arange(L, dtype=np.int64)
    m = np.zeros((rows.shape[0], L), dtype=np.float64)
    hide = cols[None, :] > rows[:, None]
    if window > 0:
        hide |= cols[None, :] <= rows[:, None] - window
    m[hide] = -np.inf
    return m


def window_causal_attention(q, k, v, window: int, prefix_len: int = 0, scale=None, rows=None) -> np.ndarray:
    """prefix_causal_attention with the sliding-window rule: chunk row r at
    position prefix_len + r sees keys c with prefix_len + r - window < c <=
    prefix_len + r."""
    q, k, v = attention._as_f64(q), attention._as_f64(k), attention._as_f64(v)
    Lq, H, D = q.shape
    Lk = k.shape[0]
    assert Lk == prefix_len + Lq, "keys must be the prefix followed by the chunk"
    G = H // k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], H * D), dtype=np.float64)
    for i in range(H):
        g = i // G
        s = (q[rows, i, :] @ k[:, g, :].T) * scale
        s = s + window_mask_rows(rows + prefix_len, Lk, window)
        p = attention.softmax_two_pass(s)
        out[:, i * D:(i + 1) * D] = p @ v[:, g, :]
    return out


def varlen_window_attention(q, k, v, cu_seqlens, window: int, scale=None, rows=None) -> np.ndarray:
    """Packed sequences (no prefix), each attended alone with the window rule."""
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
        out[pick] = window_causal_attention(np.asarray(q)[s0:s1], np.asarray(k)[s0:s1], np.asarray(v)[s0:s1],
                                            window, 0, scale, rows=sel[pick] - s0)
    return out
