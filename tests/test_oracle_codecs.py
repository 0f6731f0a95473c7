"""Pins for the oracle's bf16 and E4M3 codecs and the fp8 quantiser.  CPU only."""
import numpy as np
import pytest
import torch

from oracle import bf16, fp8


# ---------------------------------------------------------------- bf16
def test_bf16_known_patterns():
    cases = {1.0: 0x3F80, -2.0: 0xC000, 0.0: 0x0000, 0.5: 0x3F00, 3.0: 0x4040,
             2.0 ** -126: 0x0080, 2.0 ** -133: 0x0001, 65280.0: 0x477F}
    for x, bits in cases.items():
        assert int(bf16.from_f64(np.array([x]))[0]) == bits, x
        assert bf16.to_f64(np.array([bits], dtype=np.uint16))[0] == x


def test_bf16_ties_to_even_and_no_double_rounding():
    one = 1.0
    assert bf16.from_f64(np.array([one + 2 ** -8]))[0] == 0x3F80          # tie -> even (1.0)
    assert bf16.from_f64(np.array([one + 3 * 2 ** -8]))[0] == 0x3F82      # tie -> even (1+2^-6)
    # just above the tie: via fp32 this would first round to the tie, then to 1.0
    assert bf16.from_f64(np.array([one + 2 ** -8 + 2 ** -40]))[0] == 0x3F81
    assert bf16.from_f64(np.array([-(one + 2 ** -8 + 2 ** -40)]))[0] == 0xBF81


def test_bf16_matches_torch_on_fp32_values():
    x = np.random.default_rng(0).standard_normal(200000).astype(np.float32) * 10
    x[:5] = [0.1, -0.1, 1e-39, 3.0e38, -7.5]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16.from_f64(x.astype(np.float64)), want)
    assert np.array_equal(bf16.to_f64(want), torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).double().numpy())


# ---------------------------------------------------------------- e4m3
def test_e4m3_decode_known_codes():
    t = fp8.decode_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6
    assert t[0x01] == 2.0 ** -9
    assert t[0x07] == 7 * 2.0 ** -9
    assert t[0x38] == 1.0 and t[0x40] == 2.0 and t[0x39] == 1.125
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    want = codes.view(torch.float8_e4m3fn).double().numpy()
    got = fp8.decode_table()
    nan = np.isnan(want)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], want[~nan])


def test_e4m3_encode_midpoints_ties_to_even():
    t = fp8.decode_table()[:0x7F]
    for c in range(0x7E):
        lo, hi = t[c], t[c + 1]
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2                       # midpoints are binary32-exact
        want_tie = c if c % 2 == 0 else c + 1
        assert fp8.encode(np.array([mid]))[0] == want_tie
        assert fp8.encode(np.array([-mid]))[0] == want_tie | 0x80
        below = np.nextafter(mid, np.float32(-np.inf))
        above = np.nextafter(mid, np.float32(np.inf))
        assert fp8.encode(np.array([below]))[0] == c
        assert fp8.encode(np.array([above]))[0] == c + 1
        assert fp8.encode(np.array([lo]))[0] == c


def test_e4m3_saturates_and_signs():
    enc = fp8.encode(np.array([448.0, 463.9, 464.0, 500.0, 1e30, -1e6, -0.0, 0.0, 1e-10, -1e-10]))
    assert list(enc) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x00, 0x80]


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-448, 448, 100000),
                        rng.standard_normal(100000) * 0.01,
                        rng.standard_normal(100000)]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.encode(x), want)


def test_quantize_rows_properties():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((300, 128)).astype(np.float32)
    x[5] = 0.0
    codes, scale = fp8.quantize_rows(x)
    assert scale.dtype == np.float32
    assert scale[5] == 0 and np.all(codes[5] == 0)
    amax_idx = np.argmax(np.abs(x), axis=1)
    for r in range(300):
        if r == 5:
            continue
        c = codes[r, amax_idx[r]]
        assert c == (0xFE if x[r, amax_idx[r]] < 0 else 0x7E)
        assert scale[r] == np.float32(np.max(np.abs(x[r])) / np.float32(448))
    deq = fp8.decode(codes) * scale[:, None].astype(np.float64)
    normal = np.abs(fp8.decode(codes)) >= 2.0 ** -6
    rel = np.abs(deq - x)[normal] / np.abs(x)[normal]
    assert rel.max() <= 2.0 ** -4


def test_quantize_rows_reference_steps():
    # one row by hand: amax 3.5 -> inv = fp32(448/3.5) = 128 exactly; codes of x*128
    x = np.array([[3.5, -1.0, 0.25, 0.0078125]], dtype=np.float32)
    codes, scale = fp8.quantize_rows(x)
    assert scale[0] == np.float32(3.5 / 448)
    # 448 -> 0x7E, -128 -> 1.0*2^7 -> e=14 -> 0xF0, 32 -> e=12 -> 0x60, 1.0 -> 0x38
    assert list(codes[0]) == [0x7E, 0xF0, 0x60, 0x38]
