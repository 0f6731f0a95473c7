"""Pins of the oracle's power-of-two fp8 quantiser and its fp8-score attention.

The quantiser is checked against its definition (the smallest exponent that
keeps the row's amax at or below 448, found by brute force over exact
power-of-two multiplications), against hand-worked rows, and by its round-trip
bound; the attention against a pure-Python base-2 softmax on tiny inputs and
the causal closed forms (row 0 is V's row 0; Q = 0 gives the prefix mean).
"""
import math

import numpy as np

from oracle import bf16, fp8, fp8_attention


def test_pow2_exponent_is_the_smallest_that_fits():
    rng = np.random.default_rng(70)
    amax = np.concatenate([2.0 ** rng.uniform(-135, 127, 4000),
                           [448.0, 449.0, 224.0, 224.0 + 2 ** -20, 1.0, 1.75, 1.75 + 2 ** -20, 2.0 ** -126,
                            2.0 ** -140, 0.0, 3.0e38]])
    e = fp8.pow2_exponent(amax)
    for a, ei in zip(amax, e):
        ei = int(ei)
        assert -127 <= ei <= 127
        assert math.ldexp(a, -ei) <= 448.0, (a, ei)
        if ei > -127:
            assert math.ldexp(a, -(ei - 1)) > 448.0, (a, ei)     # one less would overflow 448


def test_quantize_rows_pow2_hand_worked():
    # amax 448: e = 0 (byte 127); 448 -> 0x7E, -1 -> 0xB8, 0.5 -> 0x30, 3 = 1.5 * 2**1 -> 0x44
    codes, b = fp8.quantize_rows_pow2(np.array([[448.0, -1.0, 0.5, 3.0]], dtype=np.float32))
    assert codes.tolist() == [[0x7E, 0xB8, 0x30, 0x44]] and b.tolist() == [127]
    # amax 0.002 = 0.512 * 2**-8: e = -17 (0.002 * 2**17 = 262.1 <= 448, twice that is not);
    # 0.001 * 2**17 = 131.07 -> 128 (0x70), -0.002 * 2**17 = -262.1 -> -256 (0xF8); byte 110
    codes, b = fp8.quantize_rows_pow2(np.array([[0.001, -0.002]], dtype=np.float32))
    assert codes.tolist() == [[0x70, 0xF8]] and b.tolist() == [110]
    # an all-zero row: byte 0 (2**-127), codes +0 / -0
    codes, b = fp8.quantize_rows_pow2(np.array([[0.0, -0.0]], dtype=np.float32))
    assert codes.tolist() == [[0x00, 0x80]] and b.tolist() == [0]


def test_quantize_rows_pow2_round_trip_bound():
    rng = np.random.default_rng(71)
    y = (rng.standard_normal((300, 128)) * 2.0 ** rng.uniform(-20, 20, (300, 1))).astype(np.float32)
    codes, b = fp8.quantize_rows_pow2(y)
    d = fp8.decode_rows_pow2(codes, b)
    e = b.astype(np.int64) - 127
    amax = np.max(np.abs(y), axis=1)
    top = np.abs(d[np.arange(300), np.argmax(np.abs(y), axis=1)]) * np.ldexp(1.0, -e)
    pre = amax * np.ldexp(1.0, -e)
    assert np.all((pre > 224) & (pre <= 448))                  # the scaled amax lands in (224, 448]
    assert np.all((top >= 224) & (top <= 448))                 # and its code decodes within [224, 448]
    normal = np.abs(y) * np.ldexp(1.0, -e)[:, None] >= 2.0 ** -6
    rel = np.abs(d - y) / np.abs(y)
    assert np.all(rel[normal] <= 2.0 ** -4)                    # half an E4M3 step
    sub = ~normal
    assert np.all(np.abs(d - y)[sub] <= np.ldexp(2.0 ** -10, e)[:, None].repeat(128, 1)[sub])
    assert np.all(amax > 0)


def _brute(qd, kd, v, G):
    """Pure-Python causal attention with a base-2 softmax of the given scores."""
    L, H, D = qd.shape
    out = np.zeros((L, H * D))
    for r in range(L):
        for i in range(H):
            g = i // G
            s = [sum(qd[r, i, d] * kd[c, g, d] for d in range(D)) for c in range(r + 1)]
            m = max(s)
            w = [math.pow(2.0, x - m) for x in s]
            tot = sum(w)
            for d in range(D):
                out[r, i * D + d] = sum(w[c] * v[c, g, d] for c in range(r + 1)) / tot
    return out


def test_fp8qk_attention_matches_base2_brute_force():
    rng = np.random.default_rng(72)
    for L, H, Hk, D in [(9, 2, 1, 8), (6, 4, 2, 4), (5, 2, 2, 16)]:
        q = bf16.from_f64(rng.standard_normal((L, H, D)))
        k = rng.standard_normal((L, Hk, D)).astype(np.float32)
        v = rng.standard_normal((L, Hk, D))
        kc, kb = fp8.quantize_rows_pow2(k)
        scale = 1.0 / math.sqrt(D)
        got = fp8_attention.fp8qk_attention(q, kc, kb, v, [0, L], scale)
        qc, qb = fp8_attention.quantize_q(q, scale)
        want = _brute(fp8.decode_rows_pow2(qc, qb), fp8.decode_rows_pow2(kc, kb), v, H // Hk)
        assert np.max(np.abs(got - want)) < 1e-12


def test_fp8qk_attention_closed_forms():
    rng = np.random.default_rng(73)
    L, H, Hk, D = 40, 4, 2, 16
    v = rng.standard_normal((L, Hk, D))
    kc, kb = fp8.quantize_rows_pow2(rng.standard_normal((L, Hk, D)).astype(np.float32))
    q = bf16.from_f64(rng.standard_normal((L, H, D)))
    o = fp8_attention.fp8qk_attention(q, kc, kb, v, [0, L], 0.25)
    for i in range(H):
        assert np.array_equal(o[0, i * D:(i + 1) * D], v[0, i // 2])          # row 0 sees only key 0
    o0 = fp8_attention.fp8qk_attention(bf16.from_f64(np.zeros((L, H, D))), kc, kb, v, [0, L], 0.25)
    for r in (1, 7, 39):
        for i in range(H):
            assert np.allclose(o0[r, i * D:(i + 1) * D], v[:r + 1, i // 2].mean(axis=0), atol=1e-14)


def test_score_factor_is_two_binary32_roundings():
    assert fp8_attention.score_factor(0.125) == np.float32(np.float32(0.125) * np.float32(math.log2(math.e)))
    assert fp8_attention.score_factor(1.0) == np.float32(math.log2(math.e))
