"""GPU parity of pca_qkv_proj_kv_write (the KV-cache write done by the QKV
GEMM's epilogue): y must be bit-equal to pca_qkv_proj's, and the page pools
(and fp8 scales) bit-equal to the oracle's scatter / quantiser applied to y's
own K and V columns (the same bf16 values a separate write would read)."""
import numpy as np
import pytest
import torch

import prefill_causal_attention_amd as pca
import workloads
from oracle import kvcache

from _gpu_helpers import bits, dev, require_gpu, say

pytestmark = pytest.mark.gpu

SENT16 = 0xA5A5 - 65536
SENT32 = -1515870811      # 0xA5A5A5A5


def _pools(w, cache):
    shape = (w.num_pages, 16, w.n_kv_head, w.head_dim)
    if cache == "bf16":
        kc = torch.full(shape, SENT16, dtype=torch.int16, device="cuda")
        vc = torch.full(shape, SENT16, dtype=torch.int16, device="cuda")
        return kc, vc, None, None
    kc = torch.full(shape, 0xA5, dtype=torch.uint8, device="cuda")
    vc = torch.full(shape, 0xA5, dtype=torch.uint8, device="cuda")
    ks = torch.full(shape[:3], SENT32, dtype=torch.int32, device="cuda").view(torch.float32)
    vs = torch.full(shape[:3], SENT32, dtype=torch.int32, device="cuda").view(torch.float32)
    return kc, vc, ks, vs


def _run(w, cache):
    x, wq = workloads.projection_inputs(w)
    M, N = w.total_tokens, w.n_qkv
    nk = w.n_kv_head * w.head_dim
    k_off, v_off = w.n_head * w.head_dim, w.n_head * w.head_dim + nk
    cu = workloads.cu_seqlens(w)
    bt = workloads.block_table(w)
    say(f"qkv_proj_kv_write {w.name} M={M} N={N} K={w.h} heads={w.n_head}/{w.n_kv_head} hd={w.head_dim} "
        f"pages={w.num_pages} cache={cache} seeds={w.seed(1)},{w.seed(2)},{w.seed(7)}")
    dx = dev(x)
    dwt = dev(wq.t().contiguous())
    d_cu = dev(torch.from_numpy(cu))
    d_bt = dev(torch.from_numpy(np.where(bt < 0, 0, bt).astype(np.int32)))
    y_ref = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    pca.qkv_proj(dx, dwt, y_ref)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    kc, vc, ks, vs = _pools(w, cache)
    pca.qkv_proj_kv_write(dx, dwt, y, d_bt, kc, vc, w.n_head, w.n_kv_head, w.head_dim, cu_seqlens=d_cu,
                          cache_dtype=cache, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    yb = bits(y)
    assert np.array_equal(yb, bits(y_ref)), "y differs from pca_qkv_proj"
    kb = yb[:, k_off:k_off + nk].reshape(-1, w.n_kv_head, w.head_dim)
    vb = yb[:, v_off:v_off + nk].reshape(-1, w.n_kv_head, w.head_dim)
    if cache == "bf16":
        ek, ev = kvcache.paged_write_bf16(kb, vb, cu, bt, w.num_pages)
        gk = kc.cpu().numpy().view(np.uint16)
        gv = vc.cpu().numpy().view(np.uint16)
        assert np.array_equal(gk, ek), f"K pool mismatch at {np.argwhere(gk != ek)[:5]}"
        assert np.array_equal(gv, ev), f"V pool mismatch at {np.argwhere(gv != ev)[:5]}"
    else:
        ek, ev, eks, evs = kvcache.paged_write_fp8(kb, vb, cu, bt, w.num_pages)
        gk, gv = kc.cpu().numpy(), vc.cpu().numpy()
        assert np.array_equal(gk, ek), f"K codes mismatch at {np.argwhere(gk != ek)[:5]}"
        assert np.array_equal(gv, ev), f"V codes mismatch at {np.argwhere(gv != ev)[:5]}"
        assert np.array_equal(ks.cpu().numpy().view(np.uint32), eks.view(np.uint32)), "K scales mismatch"
        assert np.array_equal(vs.cpu().numpy().view(np.uint32), evs.view(np.uint32)), "V scales mismatch"


@pytest.mark.parametrize("cache", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("lens,H,Hk,hd,h", [
    ([1, 17, 33, 5, 300], 8, 2, 128, 512),   # varlen, ragged tails, a 1-token sequence, M not a tile multiple
    ([70, 190], 8, 4, 64, 256),              # two 64-wide heads per 128-column slab
    ([100, 29], 8, 4, 32, 136),              # four 32-wide heads per slab, K not a multiple of 64
    ([600], 16, 16, 128, 384),               # MHA, one sequence over three M tiles
])
def test_small(cache, lens, H, Hk, hd, h):
    require_gpu()
    _run(workloads.custom(61, lens, H, Hk, hd, h=h, spare_pages=5), cache)


def test_unaligned_heads_bf16():
    """n_head*hd = 192: Q/K and K/V boundaries fall inside 128-column slabs (bf16 only)."""
    require_gpu()
    _run(workloads.custom(62, [77, 40], 3, 1, 64, h=192, spare_pages=3), "bf16")


def test_unaligned_heads_fp8_rejected():
    require_gpu()
    w = workloads.custom(63, [77], 3, 1, 64, h=192)
    x = torch.zeros((77, 192), dtype=torch.bfloat16, device="cuda")
    wt = torch.zeros((w.n_qkv, 192), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((77, w.n_qkv), dtype=torch.bfloat16, device="cuda")
    kc, vc, ks, vs = _pools(w, "fp8_e4m3")
    bt = torch.zeros((1, w.num_pages), dtype=torch.int32, device="cuda")
    with pytest.raises(pca.PcaError) as e:
        pca.qkv_proj_kv_write(x, wt, y, bt, kc, vc, 3, 1, 64, cache_dtype="fp8_e4m3", k_scale=ks, v_scale=vs)
    assert e.value.status == 2


@pytest.mark.parametrize("idx,cache", [(2, "bf16"), (3, "bf16"), (4, "bf16"), (5, "fp8_e4m3")])
def test_full_size(idx, cache):
    require_gpu()
    _run(workloads.WORKLOADS[idx - 1], cache)
