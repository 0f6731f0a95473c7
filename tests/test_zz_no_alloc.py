"""GPU check of pca_rms_norm_qkv_proj_noalloc, the RMSNorm-folded projection
whose 1/rms workspace is the library's static device array (for callers that
cannot allocate): called through the C ABI twice in a row, the second time
with fewer rows, its output must equal pca_rms_norm_qkv_proj's (the same
kernels on a caller-owned workspace) bit for bit, and the oracle's fp64
rms_norm(x, g, eps) @ W within the projection tolerance; a row count past the
static array is refused before any launch."""
import numpy as np
import pytest
import torch

import prefill_causal_attention_amd as pca
import workloads
from oracle import bf16 as obf16
from oracle import layer as LY

from _gpu_helpers import assert_close, bits, dev, require_gpu, say

pytestmark = pytest.mark.gpu


def _inputs(seed, M, K, N):
    """Rows of very different scales, gain near 1 folded into W^T, W ~ N(0, 1/K)."""
    rng = np.random.default_rng(seed)
    x = workloads.normal_bf16(seed + 1, (M, K))
    x = (x.float() * torch.from_numpy(np.exp(rng.uniform(-2.5, 2.5, (M, 1))).astype(np.float32))).to(torch.bfloat16)
    g = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float64)
    w = workloads.normal_bf16(seed + 2, (K, N), std=float(1 / np.sqrt(K)))
    wg = obf16.to_f64(bits(w)) * g[:, None]
    wtg = torch.from_numpy(obf16.from_f64(wg.T.copy()).view(np.int16)).view(torch.bfloat16)
    return x, g, w, wtg


@pytest.mark.parametrize("first,second", [((3000, 1024, 1536), (700, 1024, 1536)),
                                          ((1000, 512, 384), (33, 256, 200))])
def test_noalloc_matches_workspace_call_twice_shrinking(first, second):
    require_gpu()
    for i, (M, K, N) in enumerate((first, second)):
        eps = 1e-6 if i == 0 else 1e-5
        say(f"rms_norm_qkv_proj_noalloc call {i + 1}: M={M} K={K} N={N} eps={eps}")
        x, g, w, wtg = _inputs(900 + 10 * i + M, M, K, N)
        dx, dw = dev(x), dev(wtg)
        y = torch.full((M, N + 8), float("nan"), dtype=torch.bfloat16, device="cuda")
        pca.rms_norm_qkv_proj_noalloc(dx, dw, y[:, :N], eps=eps)
        ref = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        inv = torch.empty((M,), dtype=torch.float32, device="cuda")
        pca.rms_norm_qkv_proj(dx, dw, ref, inv, eps=eps)
        torch.cuda.synchronize()
        assert torch.isnan(y[:, N:].float()).all(), "wrote past N"
        assert np.array_equal(bits(y[:, :N]), bits(ref)), "differs from the workspace call"
        want = LY.rms_norm(bits(x), g, eps) @ obf16.to_f64(bits(w))
        assert_close(y[:, :N].float().cpu().numpy(), want, f"noalloc call {i + 1} vs oracle")


def test_noalloc_refuses_rows_beyond_the_static_workspace():
    require_gpu()
    M, K, N = pca.NOALLOC_MAX_ROWS + 1, 64, 64
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pca.PcaError) as e:
        pca.rms_norm_qkv_proj_noalloc(x, w, y)
    assert e.value.status == 2 and "static workspace" in str(e.value)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "a refused call wrote to y"
