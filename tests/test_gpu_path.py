"""End to end on the GPU: X -> qkv_proj -> head split (strided views) ->
prefill_attention and kv_cache_write, against the oracle's own chain from X
and W in fp64 (no GPU value feeds the oracle)."""
import numpy as np
import pytest
import torch

import prefill_causal_attention_amd as pca
import workloads
from oracle import attention as A
from oracle import bf16 as obf16
from oracle import kvcache, projection

from _gpu_helpers import assert_close, bits, dev, require_gpu, sample_rows, say

pytestmark = pytest.mark.gpu


def _path(w, rows=None):
    x, wq = workloads.projection_inputs(w)
    say(f"path {w.name} T={w.total_tokens} h={w.h} N={w.n_qkv} heads={w.n_head}/{w.n_kv_head}")
    lay = pca.kv_layout(w.n_head, w.n_kv_head, w.head_dim)
    T, nk = w.total_tokens, w.n_kv_head * w.head_dim
    dx, dwt = dev(x), dev(wq.t().contiguous())
    y = torch.empty((T, lay["qkv_ld"]), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((T, w.n_head * w.head_dim), dtype=torch.bfloat16, device="cuda")
    cu = dev(torch.from_numpy(workloads.cu_seqlens(w)))
    bt = workloads.block_table(w)
    d_bt = dev(torch.from_numpy(np.where(bt < 0, 0, bt).astype(np.int32)))
    kc = torch.zeros((w.num_pages, 16, w.n_kv_head, w.head_dim), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    pca.qkv_proj(dx, dwt, y)
    q = y[:, lay["q_off"]:lay["q_off"] + w.n_head * w.head_dim]
    k = y[:, lay["k_off"]:lay["k_off"] + nk]
    v = y[:, lay["v_off"]:lay["v_off"] + nk]
    pca.prefill_attention(q, k, v, o, w.n_head, w.n_kv_head, w.head_dim, cu_seqlens=cu, max_seqlen=w.max_seqlen)
    pca.kv_cache_write(k, v, d_bt, kc, vc, w.n_kv_head, w.head_dim, cu_seqlens=cu)
    torch.cuda.synchronize()

    # oracle chain: fp64 projection, its own RNE to bf16 (the stored precision), attention in fp64
    # (sampled attention rows still need every key before them: project all rows)
    y64 = projection.qkv_projection(bits(x), bits(wq))
    yb = obf16.from_f64(y64)
    qo, ko, vo = A.head_split(yb, w.n_head, w.n_kv_head, w.head_dim)
    want = A.varlen_causal_attention(qo, ko, vo, workloads.cu_seqlens(w), rows=rows)
    got = o.float().cpu().numpy().astype(np.float64)
    assert_close(got if rows is None else got[rows], want, f"{w.name} end-to-end attention")
    # the cache holds exactly the K/V columns the GPU projection produced
    gy = bits(y)
    kb = gy[:, lay["k_off"]:lay["k_off"] + nk].reshape(T, w.n_kv_head, w.head_dim)
    vb = gy[:, lay["v_off"]:lay["v_off"] + nk].reshape(T, w.n_kv_head, w.head_dim)
    cuh = workloads.cu_seqlens(w)
    assert np.array_equal(kvcache.gather(bits(kc), cuh, bt), kb)
    assert np.array_equal(kvcache.gather(bits(vc), cuh, bt), vb)
    # and the projection itself is within tolerance of the oracle's
    assert_close(y.float().cpu().numpy()[:256], y64[:256], f"{w.name} projection")


def test_path_small_gqa():
    require_gpu()
    _path(workloads.custom(61, [77, 300, 5], 8, 2, 128, h=512))


def test_path_gqa_s8192():
    require_gpu()
    w = workloads.WORKLOADS[2]
    _path(w, rows=sample_rows(w.total_tokens, 64, 62))


def _oracle_chain(w, x, wq, rows):
    """The oracle's chain from X and W for the sampled rows: fp64 projection
    rounded once to bf16 (K and V of every token, Q of the sampled rows only),
    head split, per-sequence causal attention in fp64."""
    xb, wb = bits(x), bits(wq)
    nq = w.n_head * w.head_dim
    yb = np.zeros((w.total_tokens, w.n_qkv), dtype=np.uint16)
    yb[:, nq:] = obf16.from_f64(projection.qkv_projection(xb, wb[:, nq:]))
    yb[rows, :nq] = obf16.from_f64(projection.projection_rows(xb, wb[:, :nq], rows))
    q, k, v = A.head_split(yb, w.n_head, w.n_kv_head, w.head_dim)
    return A.varlen_causal_attention(q, k, v, workloads.cu_seqlens(w), rows=rows)


def _edge_rows(w, per_seq, seed):
    """Each sequence's first two and last two rows, its tile edges 63/64, and
    a few random rows of every sequence (global token indices)."""
    cu = workloads.cu_seqlens(w)
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(w.num_seqs):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        for r in (0, 1, 63, 64, s1 - s0 - 2, s1 - s0 - 1):
            if 0 <= r < s1 - s0:
                rows.add(s0 + r)
        rows.update(int(t) for t in rng.integers(s0, s1, per_seq))
    return np.array(sorted(rows), dtype=np.int64)


def test_path_varlen16_gqa():
    """16 packed prompts (lengths uniform in [256, 4096], T = 27 808), GQA 32/8:
    projection -> strided attention -> paged write into a permuted page pool
    with spare pages; sampled rows (every sequence's edges) against the
    oracle chain from X and W, the pools bit for bit, spare pages untouched."""
    require_gpu()
    w = workloads.WORKLOADS[3]
    assert w.total_tokens == 27808
    x, wq = workloads.projection_inputs(w)
    say(f"path {w.name} T={w.total_tokens} lens={list(w.seqlens)} pages={w.num_pages}")
    lay = pca.kv_layout(w.n_head, w.n_kv_head, w.head_dim)
    T, nq, nk = w.total_tokens, w.n_head * w.head_dim, w.n_kv_head * w.head_dim
    y = torch.empty((T, lay["qkv_ld"]), dtype=torch.bfloat16, device="cuda")
    o = torch.full((T, nq + 8), float("nan"), dtype=torch.bfloat16, device="cuda")
    cuh = workloads.cu_seqlens(w)
    cu = dev(torch.from_numpy(cuh))
    bt = workloads.block_table(w)
    d_bt = dev(torch.from_numpy(np.where(bt < 0, 0, bt).astype(np.int32)))
    sentinel = 0xA5A5 - 65536
    kc = torch.full((w.num_pages, 16, w.n_kv_head, w.head_dim), sentinel, dtype=torch.int16, device="cuda")
    vc = torch.full_like(kc, sentinel)
    pca.qkv_proj(dev(x), dev(wq.t().contiguous()), y)
    k = y[:, lay["k_off"]:lay["k_off"] + nk]
    v = y[:, lay["v_off"]:lay["v_off"] + nk]
    pca.prefill_attention(y[:, :nq], k, v, o[:, :nq], w.n_head, w.n_kv_head, w.head_dim, cu_seqlens=cu,
                          max_seqlen=w.max_seqlen)
    pca.kv_cache_write(k, v, d_bt, kc, vc, w.n_kv_head, w.head_dim, cu_seqlens=cu)
    torch.cuda.synchronize()
    assert torch.isnan(o[:, nq:].float()).all(), "wrote outside the heads"
    rows = _edge_rows(w, 6, 4101)
    got = o[:, :nq].float().cpu().numpy()[rows]
    assert_close(got, _oracle_chain(w, x, wq, rows), f"{w.name} end-to-end attention ({len(rows)} rows)")
    gy = bits(y)
    kb = gy[:, lay["k_off"]:lay["k_off"] + nk].reshape(T, w.n_kv_head, w.head_dim)
    vb = gy[:, lay["v_off"]:lay["v_off"] + nk].reshape(T, w.n_kv_head, w.head_dim)
    wk, wv = kvcache.paged_write_bf16(kb, vb, cuh, bt, w.num_pages)
    assert np.array_equal(kc.cpu().numpy().view(np.uint16), wk)     # including 64 untouched spare pages
    assert np.array_equal(vc.cpu().numpy().view(np.uint16), wv)


def test_path_long_gqa_s32768_fp8kv():
    """s = 32768, GQA 40/8 (G = 5), h = 5120: the fused projection writes the
    fp8 E4M3 cache from its epilogue, then strided attention; sampled rows
    against the oracle chain from X and W, the codes and scales bit for bit
    against the oracle's quantising scatter of the projection's K and V."""
    require_gpu()
    w = workloads.WORKLOADS[4]
    x, wq = workloads.projection_inputs(w)
    say(f"path {w.name} T={w.total_tokens} h={w.h} heads={w.n_head}/{w.n_kv_head} fp8 cache (fused write)")
    lay = pca.kv_layout(w.n_head, w.n_kv_head, w.head_dim, 16, "fp8_e4m3")
    T, nq, nk = w.total_tokens, w.n_head * w.head_dim, w.n_kv_head * w.head_dim
    y = torch.empty((T, lay["qkv_ld"]), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((T, nq), dtype=torch.bfloat16, device="cuda")
    bt = workloads.block_table(w)
    d_bt = dev(torch.from_numpy(bt.astype(np.int32)))
    shape = (w.num_pages, 16, w.n_kv_head, w.head_dim)
    kc = torch.full(shape, 0xA5, dtype=torch.uint8, device="cuda")
    vc = torch.full_like(kc, 0xA5)
    ks = torch.full(shape[:3], -1515870811, dtype=torch.int32, device="cuda").view(torch.float32)
    vs = torch.full(shape[:3], -1515870811, dtype=torch.int32, device="cuda").view(torch.float32)
    pca.qkv_proj_kv_write(dev(x), dev(wq.t().contiguous()), y, d_bt, kc, vc, w.n_head, w.n_kv_head, w.head_dim,
                          cache_dtype="fp8_e4m3", k_scale=ks, v_scale=vs)
    pca.prefill_attention(y[:, :nq], y[:, lay["k_off"]:lay["k_off"] + nk], y[:, lay["v_off"]:lay["v_off"] + nk], o,
                          w.n_head, w.n_kv_head, w.head_dim)
    torch.cuda.synchronize()
    rows = sample_rows(T, 96, 5101, must=(0, 1, 15, 16, 63, 64, 127, 128, 4095, 4096, 16383, 16384))
    got = o.float().cpu().numpy()[rows]
    assert_close(got, _oracle_chain(w, x, wq, rows), f"{w.name} end-to-end attention ({len(rows)} rows)")
    gy = bits(y)
    kb = gy[:, lay["k_off"]:lay["k_off"] + nk].reshape(T, w.n_kv_head, w.head_dim)
    vb = gy[:, lay["v_off"]:lay["v_off"] + nk].reshape(T, w.n_kv_head, w.head_dim)
    wkc, wvc, wks, wvs = kvcache.paged_write_fp8(kb, vb, workloads.cu_seqlens(w), bt, w.num_pages)
    assert np.array_equal(kc.cpu().numpy(), wkc) and np.array_equal(vc.cpu().numpy(), wvc)
    assert np.array_equal(ks.cpu().numpy().view(np.uint32), wks.view(np.uint32))
    assert np.array_equal(vs.cpu().numpy().view(np.uint32), wvs.view(np.uint32))
