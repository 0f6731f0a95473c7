"""GPU parity of pca_rms_norm_qkv_proj (input RMSNorm folded into the QKV
GEMM as a per-row scale) against the fp64 oracle: rms_norm(x, g, eps) @ W."""
import numpy as np
import pytest
import torch

import prefill_causal_attention_amd as pca
import workloads
from oracle import bf16 as obf16
from oracle import layer as LY

from _gpu_helpers import assert_close, bits, dev, require_gpu, sample_rows, say

pytestmark = pytest.mark.gpu


def _inputs(seed, M, K, N):
    """x rows of very different scales, gain g near 1, W ~ N(0, 1/K)."""
    rng = np.random.default_rng(seed)
    x = workloads.normal_bf16(seed + 1, (M, K))
    x = (x.float() * torch.from_numpy(np.exp(rng.uniform(-2.5, 2.5, (M, 1))).astype(np.float32))).to(torch.bfloat16)
    g = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float64)
    w = workloads.normal_bf16(seed + 2, (K, N), std=float(1 / np.sqrt(K)))
    return x, g, w


def _fold(w, g):
    """Load-time transform: W^T with the gain folded along K, rounded once to bf16."""
    wg = obf16.to_f64(bits(w)) * g[:, None]
    return torch.from_numpy(obf16.from_f64(wg.T.copy()).view(np.int16)).view(torch.bfloat16)


def _gpu(x, wtg, eps, pad=8):
    M = x.shape[0]
    N = wtg.shape[0]
    y = torch.full((M, N + pad), float("nan"), dtype=torch.bfloat16, device="cuda")
    inv = torch.full((M + 4,), float("nan"), dtype=torch.float32, device="cuda")
    pca.rms_norm_qkv_proj(dev(x), dev(wtg), y[:, :N], inv, eps=eps)
    torch.cuda.synchronize()
    assert torch.isnan(y[:, N:].float()).all(), "wrote past N"
    assert torch.isnan(inv[M:]).all(), "wrote past M in inv_rms"
    return y[:, :N], inv[:M]


@pytest.mark.parametrize("M,K,N,eps", [(100, 256, 200, 1e-6), (257, 4096, 384, 1e-5), (513, 1032, 1000, 0.0),
                                       (2304, 1032, 8192, 1e-6), (33, 5000, 136, 1e-6)])
def test_parity(M, K, N, eps):
    """(2304, 8192) runs on the mixed grid of 256- and 128-row tiles on 256 CUs.
    K = 5000: the row statistics load a row 4096 elements at a time, so the
    second batch is cut short at the row's end."""
    require_gpu()
    x, g, w = _inputs(101, M, K, N)
    say(f"rms_norm_qkv_proj M={M} K={K} N={N} eps={eps}")
    y, inv = _gpu(x, _fold(w, g), eps)
    xf = obf16.to_f64(bits(x))
    want = LY.rms_norm(xf, g, eps) @ obf16.to_f64(bits(w))
    assert_close(y.float().cpu().numpy(), want, f"rms qkv {M}x{N}x{K}")
    want_inv = 1.0 / np.sqrt(np.mean(xf * xf, axis=1) + eps)
    assert np.max(np.abs(inv.cpu().numpy() / want_inv - 1.0)) < 1e-5


def test_constant_rows_halve_the_plain_product_bitwise():
    """Rows of 2.0 with eps = 0 and g = 1: inv_rms = 0.5 exactly, so y is the
    plain projection halved, bit for bit (scaling by 2^-1 commutes with RNE)."""
    require_gpu()
    M, K, N = 130, 512, 264
    x = torch.full((M, K), 2.0, dtype=torch.bfloat16)
    w = workloads.normal_bf16(102, (K, N), std=float(1 / np.sqrt(K)))
    wt = dev(w.t().contiguous())
    y, inv = _gpu(x, w.t().contiguous(), 0.0)
    assert torch.all(inv == 0.5)
    plain = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    pca.qkv_proj(dev(x), wt, plain)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits((plain.float() * 0.5).to(torch.bfloat16)))


def test_full_size_sampled():
    """s = 8192, h = 4096, N = 6144 (GQA 32/8 hd128), sampled rows."""
    require_gpu()
    M, K, N = 8192, 4096, 6144
    x, g, w = _inputs(103, M, K, N)
    y, _ = _gpu(x, _fold(w, g), 1e-6)
    rows = sample_rows(M, 32, 104, must=(0, 255, 256, M - 1))
    xf = obf16.to_f64(bits(x[rows]))
    want = LY.rms_norm(xf, g, 1e-6) @ obf16.to_f64(bits(w))
    assert_close(y[rows].float().cpu().numpy(), want, "rms qkv s=8192")
