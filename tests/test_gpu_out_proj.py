"""GPU parity of pca_out_proj_residual (out = res + o W_o, one rounding)
against the fp64 oracle: exact integer and zero-weight pins, tolerance on
N(0,1)-scaled inputs, in-place update, ragged shapes."""
import numpy as np
import pytest
import torch

import prefill_causal_attention_amd as pca
import workloads
from oracle import bf16 as obf16
from oracle import layer as LY

from _gpu_helpers import assert_close, bits, dev, require_gpu, sample_rows, say

pytestmark = pytest.mark.gpu


def _run(o, w, res, in_place=False, pad=8):
    """o (M, K), w (K, N) as drawn, res (M, N): bf16 CPU tensors."""
    M, K = o.shape
    N = w.shape[1]
    do, dwt = dev(o), dev(w.t().contiguous())
    out = torch.full((M, N + pad), float("nan"), dtype=torch.bfloat16, device="cuda")
    if in_place:
        out[:, :N] = dev(res)
        pca.out_proj_residual(do, dwt, out[:, :N], out[:, :N])
    else:
        pca.out_proj_residual(do, dwt, dev(res), out[:, :N])
    torch.cuda.synchronize()
    assert torch.isnan(out[:, N:].float()).all(), "wrote past N"
    return out[:, :N]


def _bf(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def test_integer_inputs_exact():
    require_gpu()
    rng = np.random.default_rng(91)
    M, K, N = 300, 4096, 520
    oi, wi, ri = rng.integers(-4, 5, (M, K)), rng.integers(-4, 5, (K, N)), rng.integers(-100, 101, (M, N))
    say(f"out_proj_residual integer pin M={M} N={N} K={K}")
    got = bits(_run(_bf(oi), _bf(wi), _bf(ri)))
    want = obf16.from_f64((ri + oi @ wi).astype(np.float64))
    assert np.array_equal(got, want), f"{np.sum(got != want)} mismatches"


def test_zero_weight_returns_residual():
    require_gpu()
    o = workloads.normal_bf16(92, (77, 136))
    res = workloads.normal_bf16(93, (77, 200))
    got = _run(o, torch.zeros((136, 200), dtype=torch.bfloat16), res)
    assert np.array_equal(bits(got), bits(res))


@pytest.mark.parametrize("M,N,K,in_place", [(100, 200, 64, False), (257, 384, 4096, True), (513, 1000, 1032, False),
                                            (2048, 4096, 4096, True)])
def test_normal_inputs_tolerance(M, N, K, in_place):
    """(2048, 4096) runs on 128-row tiles on 256 CUs, the others on 256-row tiles."""
    require_gpu()
    o = workloads.normal_bf16(94, (M, K))
    w = workloads.normal_bf16(95, (K, N), std=float(1 / np.sqrt(K)))
    res = workloads.normal_bf16(96, (M, N))
    say(f"out_proj_residual N(0,1) M={M} N={N} K={K} in_place={in_place}")
    got = _run(o, w, res, in_place)
    want = LY.out_projection_residual(bits(o), bits(w), bits(res))
    assert_close(got.float().cpu().numpy(), want, f"out_proj {M}x{N}x{K}")


def test_full_size_sampled():
    """s = 8192, h = 4096: o (8192, 4096) @ W_o (4096, 4096) + residual, sampled rows."""
    require_gpu()
    M, K, N = 8192, 4096, 4096
    o = workloads.normal_bf16(97, (M, K))
    w = workloads.normal_bf16(98, (K, N), std=float(1 / np.sqrt(K)))
    res = workloads.normal_bf16(99, (M, N))
    got = _run(o, w, res, in_place=True)
    rows = sample_rows(M, 48, 100, must=(0, 255, 256, M - 1))
    want = LY.out_projection_residual(bits(o), bits(w), bits(res), rows=rows)
    assert_close(got[rows].float().cpu().numpy(), want, "out_proj s=8192")


def test_mixed_grid_rows_equal_a_tall_call_bitwise():
    """2304 x 8192 runs on the mixed grid on 256 CUs (one round of 256-row
    tiles, the last four column strips in 128-row tiles); 8192 x 8192 on
    256-row tiles throughout.  Each output sums its K terms and adds its
    residual in the same order either way, so the first 2304 rows agree bit
    for bit; sampled rows are also checked against the oracle.  The residual
    is drawn at half scale: y is then about N(0, 1.25), and no output reaches
    8, where bf16 rounding alone would exceed the 2e-2 bound."""
    require_gpu()
    M, N, K = 2304, 8192, 1032
    o = workloads.normal_bf16(91, (8192, K))
    w = workloads.normal_bf16(92, (K, N), std=float(1 / np.sqrt(K)))
    res = workloads.normal_bf16(93, (8192, N), std=0.5)
    say(f"out_proj_residual mixed grid M={M} and 8192, N={N} K={K}")
    tall = _run(o, w, res, in_place=False)
    short = _run(o[:M], w, res[:M], in_place=False)
    assert torch.equal(short, tall[:M]), "grid plans disagree"
    rows = sample_rows(M, 48, 90, must=(0, 127, 128, 255, 256, M - 1))
    want = LY.out_projection_residual(bits(o[:M]), bits(w), bits(res[:M]), rows=rows)
    assert_close(short[rows].float().cpu().numpy(), want, "out_proj mixed grid rows")
