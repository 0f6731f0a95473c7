"""Pins of the oracle's power-of-two fp8 quantiser and its fp8-score attention.

The quantiser is checked against its definition (the smallest exponent that
keeps the row's amax at or below 448, found by brute force over exact
power-of-two multiplications), against hand-worked rows, and by its round-trip
bound; the attention against a pure-Python base-2 softmax on tiny inputs and
the causal closed forms (row 0 is V's row 0; Q = 0 gives the prefix mean).
"""
import math

import numpy as np

from oracle import attention, bf16, fp8, fp8_attention


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


def _f32(bits_hex: int) -> np.float32:
    return np.array([bits_hex], dtype=np.uint32).view(np.float32)[0]


def test_score_factor_hand_worked():
    """c = RN32(RN32(scale) * RN32(log2 e)), checked against bit patterns worked
    out by hand.  RN32(log2 e) = 0x3FB8AA3B (significand 0xB8AA3B).
      * scale 1/8: a power of two, so the product is exact: the exponent of
        log2 e drops by 3, 0x3FB8AA3B -> 0x3E38AA3B.
      * scale 1/sqrt(128) = sqrt(2) * 2^-4: RN32(sqrt 2) = 0x3FB504F3
        (significand 0xB504F3); 0xB504F3 * 0xB8AA3B = 0x8293EDA98201 (48 bits),
        whose low 24 bits 0xA98201 exceed half an ulp (0x800000), so the
        significand rounds up to 0x8293EE; the product is 2.0403 (exponent
        field 128) and the 2^-4 takes it to exponent field 124: 0x3E0293EE.
      * scale 1: RN32(log2 e) itself.
      * scale RN32(1/sqrt(160)) = 0x3DA1E89B (significand 0xA1E89B, 2^-4):
        0xA1E89B * 0xB8AA3B = 0x74CAD92F89B9 (47 bits, a significand product
        in [1, 2)), low 23 bits 0x2F89B9 below half (0x400000): rounds down
        to 0xE995B2, so c = 0x3DE995B2.  Rounding log2 e only once, with the
        product, would give 0x3DE995B3: this case tells the two apart."""
    assert fp8_attention.score_factor(0.125).view(np.uint32) == 0x3E38AA3B
    assert fp8_attention.score_factor(1 / math.sqrt(128)).view(np.uint32) == 0x3E0293EE
    assert fp8_attention.score_factor(1.0).view(np.uint32) == 0x3FB8AA3B
    assert fp8_attention.score_factor(1 / math.sqrt(128)) == _f32(0x3E0293EE)
    assert fp8_attention.score_factor(float(_f32(0x3DA1E89B))).view(np.uint32) == 0x3DE995B2


def test_quantize_q_hand_worked():
    """Q is quantised after the factor c.  Scale 1/8 gives c = 0.18033688
    (0x3E38AA3B).  Row [8, 1] (exact in bf16):
      y = [8c, c] = [1.44269502, 0.18033688] in binary32 (power-of-two
      multiples of c, so exact); amax 1.4427: 1.4427 * 2^8 = 369.3 <= 448
      but 2^9 would give 738.7, so e = -8 (byte 119);
      369.33 lies between the E4M3 values 352 and 384 and is nearer 384 =
      1.5 * 2^8: exponent field 15, mantissa 100 -> 0x7C;
      0.18034 * 256 = 46.17 lies between 44 and 48, nearer 48 = 1.5 * 2^5:
      exponent field 12, mantissa 100 -> 0x64.
    Quantising Q first and applying c afterwards would give other codes:
    amax 8 -> e = -5, codes 256 -> 0x78 and 32 -> 0x60 (byte 122)."""
    q = bf16.from_f64(np.array([[[8.0, 1.0]]]))
    codes, b = fp8_attention.quantize_q(q, 0.125)
    assert codes.tolist() == [[[0x7C, 0x64]]] and b.tolist() == [[119]]
    # a negative row, and a row whose scaled amax sits exactly on 448 * 2^k
    q = bf16.from_f64(np.array([[[-8.0, 1.0], [0.0, 0.0]]]))
    codes, b = fp8_attention.quantize_q(q, 0.125)
    assert codes.tolist() == [[[0xFC, 0x64], [0x00, 0x00]]] and b.tolist() == [[119, 0]]
    # scale = RN32(1 / log2 e) makes c exactly 1: Q is quantised as it is;
    # 7 = 448 * 2^-6 (e = -6, code 0x7E) and 2^-15 = 2^-9 * 2^-6 (the smallest subnormal, 0x01)
    s1 = float(np.float32(1 / 1.4426950408889634))
    assert fp8_attention.score_factor(s1) == np.float32(1.0)
    q = bf16.from_f64(np.array([[[7.0, 2.0 ** -15, -3.5]]]))
    codes, b = fp8_attention.quantize_q(q, s1)
    assert codes.tolist() == [[[0x7E, 0x01, 0xF6]]] and b.tolist() == [[121]]


# Bound of the fp8-score attention against the plain fp64 attention on the
# unquantised operands.  E4M3 keeps 3 mantissa bits, so each quantised operand
# element is within a relative 2^-4 of its input (normals; the power-of-two
# row scale is exact).  On unit-variance rows with head_dim 128 that is a
# score error of RMS ~0.05 (natural units); through the softmax the output
# moves by that times the spread of the visible V rows, the most for early
# rows with few keys.  Measured on N(0,1) inputs: max-abs ~0.07, mean-abs
# ~0.004.  The bound (5 sigma of the worst row class, and the mean with
# margin) still fails any systematic mistake (a Q exponent one off rescales
# every score by 2, a dropped factor changes them by 1/c).
FP8_SCORE_MAX_ABS = 0.25
FP8_SCORE_MEAN_ABS = 1e-2


def test_fp8qk_attention_within_quantisation_bound_of_plain_attention():
    rng = np.random.default_rng(74)
    L, H, Hk, D = 512, 4, 2, 128
    q = bf16.from_f64(rng.standard_normal((L, H, D)))
    k = bf16.from_f64(rng.standard_normal((L, Hk, D)))
    v = bf16.from_f64(rng.standard_normal((L, Hk, D)))
    kc, kb = fp8.quantize_rows_pow2(bf16.to_f64(k).astype(np.float32))
    rows = np.concatenate([np.arange(8), np.sort(rng.choice(np.arange(8, L), 120, replace=False))])
    got = fp8_attention.fp8qk_attention(q, kc, kb, v, [0, L], 1 / math.sqrt(D), rows=rows)
    want = attention.varlen_causal_attention(q, k, v, np.array([0, L]), rows=rows)
    d = np.abs(got - want)
    assert d.max() <= FP8_SCORE_MAX_ABS and d.mean() <= FP8_SCORE_MEAN_ABS, (d.max(), d.mean())
    assert d.max() > 1e-3                      # the operands really are quantised
    # the bound does reject a Q exponent one off (every score doubled)
    bad = fp8_attention.fp8qk_attention(q, kc, kb, v, [0, L], 2 / math.sqrt(D), rows=rows)
    assert np.abs(bad - want).mean() > FP8_SCORE_MEAN_ABS
