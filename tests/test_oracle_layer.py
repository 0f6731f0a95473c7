"""Pins for oracle.layer: RMSNorm by its defining properties and a closed
form, the residual output projection by exact and special cases.  CPU only."""
import numpy as np

from oracle import bf16
from oracle import layer as LY


def test_rms_norm_unit_rms_and_gain():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 64)) * 3.0
    y = LY.rms_norm(x, np.ones(64), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=0, atol=1e-14)
    g = rng.standard_normal(64)
    assert np.allclose(LY.rms_norm(x, g, 0.0), y * g, rtol=0, atol=1e-14)


def test_rms_norm_closed_form_and_eps():
    # a row of four 2s has rms 2: it normalises to ones; eps enters under the root
    x = np.full((1, 4), 2.0)
    assert np.array_equal(LY.rms_norm(x, np.ones(4), 0.0), np.ones((1, 4)))
    assert np.allclose(LY.rms_norm(x, np.ones(4), 5.0), np.full((1, 4), 2.0 / 3.0), rtol=0, atol=1e-15)
    # scale invariance for eps = 0
    assert np.allclose(LY.rms_norm(x * 7.5, np.ones(4), 0.0), np.ones((1, 4)), rtol=0, atol=1e-15)


def test_out_projection_zero_weight_is_residual():
    rng = np.random.default_rng(2)
    res = bf16.from_f64(rng.standard_normal((5, 8)))
    o = bf16.from_f64(rng.standard_normal((5, 16)))
    w = bf16.from_f64(np.zeros((16, 8)))
    assert np.array_equal(LY.out_projection_residual(o, w, res), bf16.to_f64(res))


def test_out_projection_integer_exact():
    rng = np.random.default_rng(3)
    oi, wi, ri = rng.integers(-4, 5, (6, 32)), rng.integers(-4, 5, (32, 5)), rng.integers(-50, 50, (6, 5))
    got = LY.out_projection_residual(bf16.from_f64(oi.astype(float)), bf16.from_f64(wi.astype(float)),
                                     bf16.from_f64(ri.astype(float)))
    assert np.array_equal(got, (ri + oi @ wi).astype(float))
