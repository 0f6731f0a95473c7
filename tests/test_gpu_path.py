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
