"""Host side of pca_clock_stamp: shader_clock_mhz pairs the two stamps per CU.

Synthetic stamps: on XCD 0 the CUs of two shader engines run counters that
differ by a large constant offset, as the cycle counters of different shader
engines do on the chip; each CU's counter advances at the XCD's clock.  Pairing
per CU recovers that clock exactly; pairing XCD-wide medians would not."""
import numpy as np

import prefill_causal_attention_amd as pca


def _stamp(t_real_ticks, clocks_mhz, offsets, cus, rng):
    """One stamp: all 1024 blocks, spread round-robin over the (xcd, se, cu)
    in `cus`, in shuffled order."""
    rows = []
    for i in range(pca.CLOCK_STAMP_WORDS // 4):
        x, se, cu = cus[i % len(cus)]
        cyc = offsets[(x, se)] + int(t_real_ticks / 100e6 * clocks_mhz[x] * 1e6)
        hw_id = (se << 13) | (cu << 8) | 0x3          # wave/simd bits set, ignored
        rows.append((x, hw_id, cyc, t_real_ticks))
    rows = [rows[i] for i in rng.permutation(len(rows))]
    return np.array(rows, dtype=np.int64).reshape(-1)


def test_pairs_per_cu_not_per_xcd():
    rng = np.random.default_rng(3)
    clocks = {0: 1750.0, 1: 2100.0}
    offsets = {(0, 0): 10**9, (0, 1): 5 * 10**12, (1, 0): 7 * 10**11, (1, 1): 7 * 10**11 + 12345}
    cus = [(x, se, cu) for x in (0, 1) for se in (0, 1) for cu in range(4)]
    a = _stamp(1_000_000, clocks, offsets, cus, rng)
    b = _stamp(1_000_000 + 5_000_000, clocks, offsets, cus[:-3], rng)   # a few CUs missing the second time
    got = pca.shader_clock_mhz(a, b)
    assert sorted(got) == [0, 1]
    for x, f in clocks.items():
        assert abs(got[x] - f) < 1e-3, (x, got[x], f)


def test_no_common_cu_gives_no_clock():
    rng = np.random.default_rng(4)
    a = _stamp(0, {0: 2000.0}, {(0, 0): 0, (0, 1): 0}, [(0, 0, 1)], rng)
    b = _stamp(10**6, {0: 2000.0}, {(0, 0): 0, (0, 1): 0}, [(0, 1, 1)], rng)
    assert pca.shader_clock_mhz(a, b) == {}
