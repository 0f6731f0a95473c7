"""Shared plumbing for the GPU tests: device copies, bit views, error stats.

Inputs come from ``workloads`` (seeded draws); expected values only from
``oracle``.  Nothing here computes any part of the method.
"""
import sys

import numpy as np
import pytest
import torch

import prefill_causal_attention_amd as pca

# bound for bf16 attention output and projection versus fp64 on N(0,1)-scaled inputs
MAX_ABS_TOL = 2e-2
MEAN_ABS_TOL = 2e-3


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pca.load()   # fails loudly when the HIP library is missing


def say(*args):
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda")


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 storage bits of a bf16 tensor (device or host)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().double().numpy()


def err_stats(got: np.ndarray, want: np.ndarray):
    d = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64))
    return float(d.max()), float(d.mean())


def assert_close(got, want, what, max_tol=MAX_ABS_TOL, mean_tol=MEAN_ABS_TOL):
    mx, mn = err_stats(got, want)
    say(f"{what}: max_abs={mx:.3e} mean_abs={mn:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert mx <= max_tol, f"{what}: max-abs {mx} > {max_tol}"
    assert mn <= mean_tol, f"{what}: mean-abs {mn} > {mean_tol}"


def sample_rows(L: int, n: int, seed: int, must=(0, 1, 15, 16, 31, 32, 63, 64, 127, 128)):
    rng = np.random.default_rng(seed)
    rows = set(int(r) for r in must if r < L)
    rows.add(L - 1)
    rows.update(int(r) for r in rng.integers(0, L, n))
    return np.array(sorted(rows), dtype=np.int64)
