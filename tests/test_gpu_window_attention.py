"""GPU parity of pca_prefill_attention_window (sliding-window causal
attention) against the fp64 oracle, and its special cases on the kernel
itself: a window covering the sequence is pca_prefill_attention bit for bit,
and a window of one key returns each row's own V."""
import numpy as np
import pytest
import torch

import prefill_causal_attention_amd as pca
import workloads
from oracle import attention as A
from oracle import prefix as PX

from _gpu_helpers import assert_close, bits, dev, require_gpu, sample_rows, say

pytestmark = pytest.mark.gpu


def _views(w, buf):
    nq, nk = w.n_head * w.head_dim, w.n_kv_head * w.head_dim
    return buf[:, :nq], buf[:, nq:nq + nk], buf[:, nq + nk:nq + 2 * nk]


def _gpu(w, buf, window, o_pad=8):
    d = dev(buf)
    q, k, v = _views(w, d)
    nq = w.n_head * w.head_dim
    o = torch.full((w.total_tokens, nq + o_pad), float("nan"), dtype=torch.bfloat16, device="cuda")
    cu = dev(torch.from_numpy(workloads.cu_seqlens(w))) if w.num_seqs > 1 else None
    pca.prefill_attention(q, k, v, o[:, :nq], w.n_head, w.n_kv_head, w.head_dim, cu_seqlens=cu,
                          max_seqlen=w.max_seqlen, window=window)
    torch.cuda.synchronize()
    assert torch.isnan(o[:, nq:].float()).all(), "wrote outside the heads"
    return o[:, :nq]


def _oracle(w, buf, window, rows=None):
    q, k, v = A.head_split(bits(buf), w.n_head, w.n_kv_head, w.head_dim)
    return PX.varlen_window_attention(q, k, v, workloads.cu_seqlens(w), window, rows=rows)


@pytest.mark.parametrize("lens,H,Hk,hd,W", [
    ([300], 4, 2, 128, 100),
    ([300], 4, 2, 128, 64),
    ([257, 90, 1], 8, 2, 128, 37),        # varlen, a 1-token sequence
    ([500], 8, 8, 64, 1),
    ([130, 70], 4, 2, 32, 50),             # head_dim 32, varlen
    ([200, 333], 4, 1, 32, 150),
    ([700], 10, 2, 128, 300),              # G = 5
])
def test_parity_small(lens, H, Hk, hd, W):
    require_gpu()
    w = workloads.custom(81, lens, H, Hk, hd)
    buf, *_ = workloads.qkv_inputs(w, ld=w.n_qkv + 8)
    say(f"prefill_attention_window lens={lens} heads={H}/{Hk} hd={hd} W={W} seeds={w.seed(3)}..{w.seed(5)}")
    got = _gpu(w, buf, W).float().cpu().numpy()
    assert_close(got, _oracle(w, buf, W), f"window {W}")


def test_window_covering_sequence_is_plain_causal_bitwise():
    require_gpu()
    w = workloads.custom(82, [400, 130], 8, 2, 128)
    buf, *_ = workloads.qkv_inputs(w)
    got = _gpu(w, buf, 400)
    d = dev(buf)
    q, k, v = _views(w, d)
    o = torch.empty_like(got)
    pca.prefill_attention(q, k, v, o, w.n_head, w.n_kv_head, w.head_dim,
                          cu_seqlens=dev(torch.from_numpy(workloads.cu_seqlens(w))), max_seqlen=400)
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), bits(o))


def test_window_one_returns_own_value_bitwise():
    require_gpu()
    w = workloads.custom(83, [333], 4, 2, 64)
    buf, *_ = workloads.qkv_inputs(w)
    got = bits(_gpu(w, buf, 1))
    vb = bits(_views(w, buf)[2]).reshape(333, 2, 64)
    for i in range(4):
        assert np.array_equal(got[:, i * 64:(i + 1) * 64], vb[:, i // 2, :])


def test_long_gqa_window_sampled():
    """s = 8192 GQA 32/8 hd128 with a 1024-key window."""
    require_gpu()
    w = workloads.custom(84, [8192], 32, 8, 128)
    buf, *_ = workloads.qkv_inputs(w)
    got = _gpu(w, buf, 1024).float().cpu().numpy()
    rows = sample_rows(8192, 48, 85, must=(0, 1, 1023, 1024, 1025, 4096, 8191))
    assert_close(got[rows], _oracle(w, buf, 1024, rows=rows), "window 1024 s=8192")
