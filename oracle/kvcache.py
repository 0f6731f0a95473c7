"""KV-cache accounting and the paged KV write (test infrastructure only).

Byte accounting ([P1] §3.4, [P2] §3.1): per layer and token the cache holds
one K and one V vector per kv head, so 2 * n_kv_head * head_dim * bytes per
element; the whole cache is 2 * layers * kv_heads * head_dim * tokens * bytes.

Paged layout ([P1] §4.2 "per-block contiguous", [P2] §3.4, page size 16 from
[P3] §3.3): fixed-size pages of 16 token slots, each slot holding
[n_kv_head][head_dim]; a block table maps (sequence, logical page) to a
physical page, so token position p of sequence b lands in page
block_table[b][p // 16], slot p % 16.  Two pools, one for K and one for V,
each [num_pages][16][n_kv_head][head_dim].

For the fp8 cache the same slots hold E4M3 codes, and two fp32 scale pools
[num_pages][16][n_kv_head] hold the per-(token, kv head) scales (see
``oracle.fp8``).
"""
from __future__ import annotations

import numpy as np

from . import bf16, fp8

SENTINEL_U16 = 0xA5A5
SENTINEL_U8 = 0xA5
SENTINEL_U32 = 0xA5A5A5A5


def bytes_per_token_layer(n_kv_head: int, head_dim: int, elem_bytes: float) -> float:
    return 2 * n_kv_head * head_dim * elem_bytes


def cache_bytes(layers: int, kv_heads: int, head_dim: int, tokens: int, elem_bytes: float) -> float:
    """[P2] §3.1's formula: 2 (K and V) x layers x heads x head_dim x tokens x bytes."""
    return 2 * layers * kv_heads * head_dim * tokens * elem_bytes


def layout(n_head: int, n_kv_head: int, head_dim: int, page_size: int, elem_bytes: int) -> dict:
    """Offsets of the head split in the fused projection row and the strides of
    the page pools, in elements (except the *_bytes entries)."""
    return {
        "qkv_ld": (n_head + 2 * n_kv_head) * head_dim,
        "q_off": 0,
        "k_off": n_head * head_dim,
        "v_off": (n_head + n_kv_head) * head_dim,
        "head_stride": head_dim,
        "pool_page_stride": page_size * n_kv_head * head_dim,
        "pool_slot_stride": n_kv_head * head_dim,
        "pool_head_stride": head_dim,
        # scale pools exist only for the 1-byte (fp8) cache
        "scale_page_stride": page_size * n_kv_head if elem_bytes == 1 else 0,
        "scale_slot_stride": n_kv_head if elem_bytes == 1 else 0,
        "kv_bytes_per_token_layer": 2 * n_kv_head * head_dim * elem_bytes,
        "scale_bytes_per_token_layer": (2 * n_kv_head * 4) if elem_bytes == 1 else 0,
        "page_bytes": page_size * n_kv_head * head_dim * elem_bytes,
    }


def _slot(block_table, b: int, pos: int, page_size: int):
    return int(block_table[b][pos // page_size]), pos % page_size


def paged_write_bf16(k_bits, v_bits, cu_seqlens, block_table, num_pages: int, page_size: int = 16):
    """k_bits, v_bits: uint16 (T, n_kv, hd).  Returns the two uint16 pools,
    pre-filled with the sentinel so untouched slots can be recognised."""
    k_bits = np.asarray(k_bits, dtype=np.uint16)
    v_bits = np.asarray(v_bits, dtype=np.uint16)
    _, n_kv, hd = k_bits.shape
    kc = np.full((num_pages, page_size, n_kv, hd), SENTINEL_U16, dtype=np.uint16)
    vc = np.full((num_pages, page_size, n_kv, hd), SENTINEL_U16, dtype=np.uint16)
    cu = [int(c) for c in cu_seqlens]
    for b in range(len(cu) - 1):
        for pos in range(cu[b + 1] - cu[b]):
            t = cu[b] + pos
            page, slot = _slot(block_table, b, pos, page_size)
            kc[page, slot] = k_bits[t]
            vc[page, slot] = v_bits[t]
    return kc, vc


def paged_write_fp8(k_bits, v_bits, cu_seqlens, block_table, num_pages: int, page_size: int = 16):
    """Quantise each (token, kv head) row of K and of V to E4M3 with its own
    absmax scale, then place codes and scales in their slots.  Returns
    (k_codes, v_codes, k_scales, v_scales); untouched code slots hold 0xA5 and
    untouched scale slots the bit pattern 0xA5A5A5A5."""
    k = bf16.to_f64(k_bits).astype(np.float32)      # exact: bf16 values are binary32 values
    v = bf16.to_f64(v_bits).astype(np.float32)
    T, n_kv, hd = k.shape
    kq, ks = fp8.quantize_rows(k)
    vq, vs = fp8.quantize_rows(v)
    kc = np.full((num_pages, page_size, n_kv, hd), SENTINEL_U8, dtype=np.uint8)
    vc = np.full((num_pages, page_size, n_kv, hd), SENTINEL_U8, dtype=np.uint8)
    ksc = np.full((num_pages, page_size, n_kv), SENTINEL_U32, dtype=np.uint32)
    vsc = np.full((num_pages, page_size, n_kv), SENTINEL_U32, dtype=np.uint32)
    ks_bits = ks.view(np.uint32)
    vs_bits = vs.view(np.uint32)
    cu = [int(c) for c in cu_seqlens]
    for b in range(len(cu) - 1):
        for pos in range(cu[b + 1] - cu[b]):
            t = cu[b] + pos
            page, slot = _slot(block_table, b, pos, page_size)
            kc[page, slot] = kq[t]
            vc[page, slot] = vq[t]
            ksc[page, slot] = ks_bits[t]
            vsc[page, slot] = vs_bits[t]
    return kc, vc, ksc.view(np.float32), vsc.view(np.float32)


def gather(pool, cu_seqlens, block_table, page_size: int = 16):
    """Read the cache back in token order through the block table."""
    cu = [int(c) for c in cu_seqlens]
    out = np.empty((cu[-1],) + pool.shape[2:], dtype=pool.dtype)
    for b in range(len(cu) - 1):
        for pos in range(cu[b + 1] - cu[b]):
            page, slot = _slot(block_table, b, pos, page_size)
            out[cu[b] + pos] = pool[page, slot]
    return out
