"""GPU parity of the fp8-operand projection: pca_quantize_rows_fp8 bit-exact
against the oracle's row quantiser, and pca_qkv_proj_fp8 against the fp64
product of the same decoded operands (exact on small power-of-two values)."""
import numpy as np
import pytest
import torch

import prefill_causal_attention_amd as pca
import workloads
from oracle import bf16 as obf16
from oracle import fp8 as F
from oracle import projection as PJ

from _gpu_helpers import assert_close, bits, dev, require_gpu, sample_rows, say

pytestmark = pytest.mark.gpu


def _quant_gpu(x, pad=16):
    M, K = x.shape
    q = torch.full((M, K + pad), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((M + 4,), float("nan"), dtype=torch.float32, device="cuda")
    pca.quantize_rows_fp8(dev(x), q[:, :K], s)
    torch.cuda.synchronize()
    assert torch.all(q[:, K:] == 0xA5), "wrote past K"
    assert torch.isnan(s[M:]).all(), "wrote past M"
    return q[:, :K], s[:M]


@pytest.mark.parametrize("M,K", [(5, 16), (77, 4096), (300, 1040), (40, 8192), (17, 6160), (9, 12288)])   # 12288: the two-pass loop
def test_quantize_rows_bit_exact(M, K):
    require_gpu()
    x = workloads.normal_bf16(111, (M, K))
    x[0] = 0                                  # amax 0: scale 0, codes +-0
    x[1] = x[1] * 1000                        # large range
    q, s = _quant_gpu(x)
    eq, es = F.quantize_rows(obf16.to_f64(bits(x)).astype(np.float32))
    assert np.array_equal(q.cpu().numpy(), eq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), es.view(np.uint32))


def _gemm_gpu(xq, sx, wq, sw, pad=8):
    M, N = xq.shape[0], wq.shape[0]
    y = torch.full((M, N + pad), float("nan"), dtype=torch.bfloat16, device="cuda")
    pca.qkv_proj_fp8(xq, sx, wq, sw, y[:, :N])
    torch.cuda.synchronize()
    assert torch.isnan(y[:, N:].float()).all(), "wrote past N"
    return y[:, :N]


def test_small_values_exact():
    """Codes of 0, +-1, 2, 1/2 with power-of-two scales, K = 4096: every fp32
    partial sum is exact, so y is RNE_bf16 of the exact product, bit for bit."""
    require_gpu()
    rng = np.random.default_rng(112)
    codes = np.array([0x38, 0x40, 0x30, 0xB8, 0x00], dtype=np.uint8)
    M, N, K = 300, 520, 4096
    xq = rng.choice(codes, (M, K))
    wq = rng.choice(codes, (N, K))
    sx = (2.0 ** rng.integers(-3, 4, M)).astype(np.float32)
    sw = (2.0 ** rng.integers(-3, 4, N)).astype(np.float32)
    say(f"qkv_proj_fp8 exact pin M={M} N={N} K={K}")
    y = _gemm_gpu(dev(torch.from_numpy(xq)), dev(torch.from_numpy(sx)), dev(torch.from_numpy(wq)),
                  dev(torch.from_numpy(sw)))
    want = obf16.from_f64(PJ.fp8_projection(xq, sx, wq, sw))
    got = bits(y)
    assert np.array_equal(got, want), f"{np.sum(got != want)} mismatches"


@pytest.mark.parametrize("M,N,K", [(100, 200, 64), (257, 384, 4096), (513, 1000, 1040)])
def test_quantised_normal_inputs(M, N, K):
    require_gpu()
    x = workloads.normal_bf16(113, (M, K))
    w = workloads.normal_bf16(114, (K, N), std=float(1 / np.sqrt(K)))
    xq, sx = _quant_gpu(x)
    wq, sw = _quant_gpu(w.t().contiguous())
    say(f"qkv_proj_fp8 N(0,1) M={M} N={N} K={K}")
    y = _gemm_gpu(xq, sx, wq, sw)
    want = PJ.fp8_projection(xq.cpu().numpy(), sx.cpu().numpy(), wq.cpu().numpy(), sw.cpu().numpy())
    assert_close(y.float().cpu().numpy(), want, f"fp8 gemm {M}x{N}x{K}")
    # for information: the error the fp8 operands add against the bf16 inputs
    exact = obf16.to_f64(bits(x)) @ obf16.to_f64(bits(w))
    err = np.abs(y.float().cpu().numpy() - exact)
    say(f"  vs unquantised fp64: max_abs={err.max():.3e} mean_abs={err.mean():.3e}")


def test_full_size_sampled():
    """s = 8192, h = 4096, N = 6144 (GQA 32/8 hd128): quantise X and W^T on the
    GPU (sampled rows bit-exact), GEMM on sampled rows against the oracle."""
    require_gpu()
    w_ = workloads.BY_NAME["gqa_s8192"]
    x, w = workloads.projection_inputs(w_)
    xq, sx = _quant_gpu(x)
    wq, sw = _quant_gpu(w.t().contiguous())
    rows = sample_rows(w_.total_tokens, 32, 115, must=(0, 255, 256, w_.total_tokens - 1))
    eq, es = F.quantize_rows(obf16.to_f64(bits(x[rows])).astype(np.float32))
    assert np.array_equal(xq[rows].cpu().numpy(), eq)
    y = _gemm_gpu(xq, sx, wq, sw)
    want = PJ.fp8_projection(xq.cpu().numpy(), sx.cpu().numpy(), wq.cpu().numpy(), sw.cpu().numpy(), rows=rows)
    assert_close(y[rows].float().cpu().numpy(), want, "fp8 gemm s=8192")


@pytest.mark.parametrize("tall_m,short_m,N", [(12288, 1000, 6144), (12288, 2048, 12288), (12288, 3000, 6216)])
def test_grid_plans_agree(tall_m, short_m, N):
    """As for the bf16 GEMM: every grid plan sums each output's K terms in the
    same order, so rows of a short call (128-row tiles, or the mixed grid of
    256-row tiles then 128-row ones) equal bitwise those of a tall call on
    256-row tiles throughout."""
    require_gpu()
    K = 1040                                            # a ragged last K step
    x = workloads.normal_bf16(116, (tall_m, K))
    w = workloads.normal_bf16(117, (N, K), std=float(1 / np.sqrt(K)))
    say(f"qkv_proj_fp8 tile plans M={tall_m} and {short_m}, N={N} K={K}")
    xq, sx = _quant_gpu(x)
    wq, sw = _quant_gpu(w)
    tall = _gemm_gpu(xq, sx, wq, sw)
    short = _gemm_gpu(xq[:short_m], sx[:short_m], wq, sw)
    assert torch.equal(short, tall[:short_m]), "grid plans disagree"
    rows = sample_rows(short_m, 24, 118, must=(0, 127, 128, 255, 256, short_m - 1))
    want = PJ.fp8_projection(xq.cpu().numpy(), sx.cpu().numpy(), wq.cpu().numpy(), sw.cpu().numpy(), rows=rows)
    assert_close(short[rows].float().cpu().numpy(), want, "short fp8 call vs oracle rows")
