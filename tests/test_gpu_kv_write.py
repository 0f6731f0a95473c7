"""GPU parity of pca_kv_cache_write against the oracle's page scatter (bit-exact)."""
import numpy as np
import pytest
import torch

import prefill_causal_attention_amd as pca
import workloads
from oracle import kvcache

from _gpu_helpers import bits, dev, require_gpu, say

pytestmark = pytest.mark.gpu


def _run(w, ld_pad=0, cache="bf16"):
    """K/V drawn directly into a fused-row buffer (T, ld) -> GPU write and oracle write."""
    buf, _, k_off, v_off = workloads.qkv_inputs(w, ld=w.n_qkv + ld_pad)
    nk = w.n_kv_head * w.head_dim
    cu = workloads.cu_seqlens(w)
    bt = workloads.block_table(w)
    bt_np = np.where(bt < 0, 0, bt).astype(np.int32)       # unused entries never read
    say(f"kv_cache_write {w.name} T={w.total_tokens} n_kv={w.n_kv_head} hd={w.head_dim} "
        f"pages={w.num_pages} cache={cache} seeds={w.seed(4)},{w.seed(5)},{w.seed(7)}")
    d_buf = dev(buf)
    d_cu = dev(torch.from_numpy(cu))
    d_bt = dev(torch.from_numpy(bt_np))
    shape = (w.num_pages, 16, w.n_kv_head, w.head_dim)
    if cache == "bf16":
        kc = torch.full(shape, 0xA5A5 - 65536, dtype=torch.int16, device="cuda")
        vc = torch.full(shape, 0xA5A5 - 65536, dtype=torch.int16, device="cuda")
        ks = vs = None
    else:
        kc = torch.full(shape, 0xA5, dtype=torch.uint8, device="cuda")
        vc = torch.full(shape, 0xA5, dtype=torch.uint8, device="cuda")
        ks = torch.full(shape[:3], -1515870811, dtype=torch.int32, device="cuda").view(torch.float32)
        vs = torch.full(shape[:3], -1515870811, dtype=torch.int32, device="cuda").view(torch.float32)
    pca.kv_cache_write(d_buf[:, k_off:k_off + nk], d_buf[:, v_off:v_off + nk], d_bt, kc, vc,
                       w.n_kv_head, w.head_dim, cu_seqlens=d_cu, cache_dtype=cache,
                       k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    kb = bits(buf[:, k_off:k_off + nk]).reshape(-1, w.n_kv_head, w.head_dim)
    vb = bits(buf[:, v_off:v_off + nk]).reshape(-1, w.n_kv_head, w.head_dim)
    if cache == "bf16":
        ek, ev = kvcache.paged_write_bf16(kb, vb, cu, bt, w.num_pages)
        gk = kc.cpu().numpy().view(np.uint16)
        gv = vc.cpu().numpy().view(np.uint16)
        assert np.array_equal(gk, ek), f"K pool mismatch at {np.argwhere(gk != ek)[:5]}"
        assert np.array_equal(gv, ev), f"V pool mismatch at {np.argwhere(gv != ev)[:5]}"
    else:
        ek, ev, eks, evs = kvcache.paged_write_fp8(kb, vb, cu, bt, w.num_pages)
        gk, gv = kc.cpu().numpy(), vc.cpu().numpy()
        gks = ks.cpu().numpy().view(np.uint32)
        gvs = vs.cpu().numpy().view(np.uint32)
        assert np.array_equal(gk, ek), f"K codes mismatch at {np.argwhere(gk != ek)[:5]}"
        assert np.array_equal(gv, ev), f"V codes mismatch at {np.argwhere(gv != ev)[:5]}"
        assert np.array_equal(gks, eks.view(np.uint32)), "K scales mismatch"
        assert np.array_equal(gvs, evs.view(np.uint32)), "V scales mismatch"


@pytest.mark.parametrize("cache", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("hd", [32, 64, 128])
def test_small_varlen_ragged(cache, hd):
    require_gpu()
    w = workloads.custom(21, [1, 17, 33, 5, 64], 8, 2, hd, spare_pages=5)
    _run(w, ld_pad=8, cache=cache)


def test_identity_table_single_sequence():
    require_gpu()
    _run(workloads.custom(22, [200], 4, 4, 128, block_table="identity"))


@pytest.mark.parametrize("idx", [2, 3, 4])
def test_full_size_bf16(idx):
    require_gpu()
    _run(workloads.WORKLOADS[idx - 1])


def test_full_size_fp8_long_context():
    require_gpu()
    _run(workloads.WORKLOADS[4], cache="fp8_e4m3")


def test_zero_tokens_is_noop():
    require_gpu()
    kc = torch.zeros((2, 16, 1, 32), dtype=torch.int16, device="cuda")
    k = torch.zeros((0, 32), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    pca.kv_cache_write(k, k, bt, kc, kc, 1, 32, total_tokens=0)
    torch.cuda.synchronize()
    assert int(kc.abs().sum()) == 0
