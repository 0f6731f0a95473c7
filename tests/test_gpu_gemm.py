"""GPU parity of pca_qkv_proj against the fp64 oracle projection."""
import numpy as np
import pytest
import torch

import prefill_causal_attention_amd as pca
import workloads
from oracle import bf16 as obf16
from oracle import projection as P

from _gpu_helpers import assert_close, bits, dev, require_gpu, sample_rows, say

pytestmark = pytest.mark.gpu


def _gpu_proj(x, wq, y_pad=0):
    """x (M, K) bf16, wq (K, N) bf16 as drawn; the weight is transposed once
    (untimed, a storage choice) before the call."""
    M, K = x.shape
    N = wq.shape[1]
    dx = dev(x)
    dwt = dev(wq.t().contiguous())
    y = torch.full((M, N + y_pad), float("nan"), dtype=torch.bfloat16, device="cuda")
    pca.qkv_proj(dx, dwt, y[:, :N])
    torch.cuda.synchronize()
    return y


def test_integer_inputs_exact():
    """|x|, |w| <= 4 integers and K = 4096: every fp32 partial sum is an exact
    integer below 2^24, so y must equal RNE_bf16(exact product) bitwise."""
    require_gpu()
    rng = np.random.default_rng(51)
    M, K, N = 300, 4096, 520
    xi = rng.integers(-4, 5, (M, K))
    wi = rng.integers(-4, 5, (K, N))
    x = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16)
    wq = torch.from_numpy(wi.astype(np.float32)).to(torch.bfloat16)
    say(f"qkv_proj integer pin M={M} N={N} K={K}")
    y = _gpu_proj(x, wq)
    exact = xi.astype(np.int64) @ wi.astype(np.int64)
    want = obf16.from_f64(exact.astype(np.float64))
    got = bits(y)
    assert np.array_equal(got, want), f"{np.sum(got != want)} mismatches"


def test_one_hot_columns_copy_x():
    require_gpu()
    rng = np.random.default_rng(52)
    M, K, N = 257, 520, 72
    x = workloads.normal_bf16(53, (M, K))
    picks = rng.integers(0, K, N)
    w = np.zeros((K, N), dtype=np.float32)
    w[picks, np.arange(N)] = 1.0
    y = _gpu_proj(x, torch.from_numpy(w).to(torch.bfloat16))
    assert np.array_equal(bits(y), bits(x)[:, picks])


@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (100, 200, 64), (257, 384, 4096), (513, 1000, 1032), (2048, 6144, 4096)])
def test_normal_inputs_tolerance(M, N, K):
    require_gpu()
    x = workloads.normal_bf16(54, (M, K))
    wq = workloads.normal_bf16(55, (K, N), std=float(1 / np.sqrt(K)))
    say(f"qkv_proj N(0,1) M={M} N={N} K={K}")
    y = _gpu_proj(x, wq, y_pad=8)
    want = P.qkv_projection(bits(x), bits(wq))
    assert_close(y[:, :N].float().cpu().numpy(), want, f"gemm {M}x{N}x{K}")
    assert torch.isnan(y[:, N:].float()).all(), "wrote past N"


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_full_size_sampled(idx):
    require_gpu()
    w = workloads.WORKLOADS[idx - 1]
    x, wq = workloads.projection_inputs(w)
    say(f"qkv_proj {w.name} M={w.total_tokens} N={w.n_qkv} K={w.h} seeds={w.seed(1)},{w.seed(2)}")
    y = _gpu_proj(x, wq)
    rows = sample_rows(w.total_tokens, 64, 200 + idx, must=(0, 255, 256, w.total_tokens - 1))
    want = P.projection_rows(bits(x), bits(wq), rows)
    assert_close(y[rows].float().cpu().numpy(), want, f"{w.name} projection rows")


@pytest.mark.parametrize("short_m,tall_m,N", [(1000, 8192, 6144), (2048, 8192, 12288), (3000, 5120, 6216)])
def test_row_tile_heights_agree_bitwise(short_m, tall_m, N):
    """Every grid plan sums each output's K terms in the same order, so rows
    of a short call equal bitwise those of a tall call.  On 256 CUs the short
    calls run on 128-row tiles (1000 x 6144: 96 tiles of 256 rows would leave
    most CUs idle) or on the mixed grid (2048 x 12288: one round of 256-row
    tiles, then the last 16 column strips as 128-row tiles; 3000 x 6216, also
    ragged in M and N), the tall calls on 256-row tiles throughout."""
    require_gpu()
    K = 1032
    x = workloads.normal_bf16(56, (tall_m, K))
    wq = workloads.normal_bf16(57, (K, N), std=float(1 / np.sqrt(K)))
    say(f"qkv_proj tile plans M={tall_m} and {short_m}, N={N} K={K}")
    tall = _gpu_proj(x, wq)
    short = _gpu_proj(x[:short_m], wq, y_pad=8)
    assert torch.equal(short[:, :N], tall[:short_m]), "grid plans disagree"
    assert torch.isnan(short[:, N:].float()).all(), "wrote past N"
    rows = sample_rows(short_m, 48, 58, must=(0, 127, 128, 255, 256, short_m - 1))
    want = P.projection_rows(bits(x[:short_m]), bits(wq), rows)
    assert_close(short[rows, :N].float().cpu().numpy(), want, "short call vs oracle rows")
