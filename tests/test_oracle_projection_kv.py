"""Pins for oracle.projection and oracle.kvcache.  CPU only."""
import numpy as np

import workloads
from oracle import bf16, kvcache, projection


def _bits_of_ints(a):
    return bf16.from_f64(np.asarray(a, dtype=np.float64))


def test_projection_integer_inputs_exact():
    rng = np.random.default_rng(3)
    x = rng.integers(-4, 5, (16, 96))
    w = rng.integers(-4, 5, (96, 40))
    y = projection.qkv_projection(_bits_of_ints(x), _bits_of_ints(w))
    assert np.array_equal(y, (x.astype(np.int64) @ w.astype(np.int64)).astype(np.float64))


def test_projection_one_hot_columns_copy_x():
    rng = np.random.default_rng(4)
    xb = bf16.from_f64(rng.standard_normal((10, 12)))
    w = np.zeros((12, 5))
    picks = [3, 0, 11, 3, 7]
    for n, kk in enumerate(picks):
        w[kk, n] = 1.0
    y = projection.qkv_projection(xb, bf16.from_f64(w))
    assert np.array_equal(y, bf16.to_f64(xb)[:, picks])


def test_projection_entries_pure_python_dot():
    rng = np.random.default_rng(5)
    xb = bf16.from_f64(rng.standard_normal((6, 50)))
    wb = bf16.from_f64(rng.standard_normal((50, 9)))
    xv, wv = bf16.to_f64(xb), bf16.to_f64(wb)
    rows, cols = np.array([0, 5, 2]), np.array([8, 1, 4])
    got = projection.projection_entries(xb, wb, rows, cols)
    for a, r in enumerate(rows):
        for b, c in enumerate(cols):
            want = sum(float(xv[r, kk]) * float(wv[kk, c]) for kk in range(50))
            assert abs(got[a, b] - want) < 1e-12
    assert np.array_equal(projection.projection_rows(xb, wb, rows), projection.qkv_projection(xb, wb)[rows])


def test_kv_bytes_match_page_figures(golden):
    for name, n_kv, hd, eb, layers, tokens, expected, _src in golden("kv_bytes_pages.txt"):
        n_kv, hd, eb, layers, tokens = int(n_kv), int(hd), int(eb), int(layers), int(tokens)
        if layers == 1 and tokens == 1:
            assert kvcache.bytes_per_token_layer(n_kv, hd, eb) == int(expected), name
            assert kvcache.layout(32, n_kv, hd, 16, eb)["kv_bytes_per_token_layer"] == int(expected)
        assert kvcache.cache_bytes(layers, n_kv, hd, tokens, eb) == int(expected), name
    # GQA 32 -> 8 kv heads is a quarter of the cache ([P2] §3.2)
    assert kvcache.bytes_per_token_layer(8, 128, 2) * 4 == kvcache.bytes_per_token_layer(32, 128, 2)


def test_activation_and_block_figures(golden):
    rows = {r[0]: r for r in golden("sizes_pages.txt")}
    assert 8192 * 3 * 4096 * 2 == int(rows["qkv_activation_fp16_s8192_h4096"][2])
    assert 3 * 128 * 128 * 2 == int(rows["flash_blocks_fp16_128x128_hd128"][2])


def test_layout_offsets():
    lay = kvcache.layout(32, 8, 128, 16, 2)
    assert lay["qkv_ld"] == 6144 and lay["k_off"] == 4096 and lay["v_off"] == 5120
    assert lay["pool_page_stride"] == 16 * 8 * 128 and lay["pool_slot_stride"] == 1024
    assert kvcache.layout(40, 8, 128, 16, 1)["scale_bytes_per_token_layer"] == 64


def test_paged_slots_hand_worked(golden):
    cu = [0, 3, 21]
    bt = np.array([[5, -1], [2, 7]], dtype=np.int32)
    T, n_kv, hd = 21, 2, 4
    k = np.arange(T * n_kv * hd, dtype=np.uint16).reshape(T, n_kv, hd)
    v = (k + 1000).astype(np.uint16)
    kc, vc = kvcache.paged_write_bf16(k, v, cu, bt, num_pages=8)
    for tok, seq, pos, page, slot in golden("page_slots_small.txt"):
        tok, page, slot = int(tok), int(page), int(slot)
        assert np.array_equal(kc[page, slot], k[tok])
        assert np.array_equal(vc[page, slot], v[tok])
    written = np.any(kc != kvcache.SENTINEL_U16, axis=(2, 3))
    assert written.sum() == T
    assert np.all(kc[[0, 1, 3, 4, 6]] == kvcache.SENTINEL_U16)


def test_identity_table_is_contiguous_copy():
    w = workloads.custom(9, [50], 4, 2, 8, block_table="identity")
    bt = workloads.block_table(w)
    rng = np.random.default_rng(6)
    k = rng.integers(0, 65535, (50, 2, 8)).astype(np.uint16)
    v = rng.integers(0, 65535, (50, 2, 8)).astype(np.uint16)
    kc, vc = kvcache.paged_write_bf16(k, v, workloads.cu_seqlens(w), bt, w.num_pages)
    assert np.array_equal(kc.reshape(-1, 2, 8)[:50], k)
    assert np.array_equal(vc.reshape(-1, 2, 8)[:50], v)
    assert np.all(kc.reshape(-1, 2, 8)[50:] == kvcache.SENTINEL_U16)


def test_permuted_table_round_trip_and_sentinels():
    w = workloads.custom(9, [33, 1, 16, 47], 4, 2, 8, spare_pages=3)
    bt = workloads.block_table(w)
    cu = workloads.cu_seqlens(w)
    rng = np.random.default_rng(7)
    k = rng.integers(0, 65535, (w.total_tokens, 2, 8)).astype(np.uint16)
    v = rng.integers(0, 65535, (w.total_tokens, 2, 8)).astype(np.uint16)
    kc, vc = kvcache.paged_write_bf16(k, v, cu, bt, w.num_pages)
    assert np.array_equal(kvcache.gather(kc, cu, bt), k)
    assert np.array_equal(kvcache.gather(vc, cu, bt), v)
    used = set(int(p) for p in bt.ravel() if p >= 0)
    for p in range(w.num_pages):
        if p not in used:
            assert np.all(kc[p] == kvcache.SENTINEL_U16)


def test_fp8_paged_write_round_trip():
    w = workloads.custom(9, [40, 9], 8, 2, 16)
    bt, cu = workloads.block_table(w), workloads.cu_seqlens(w)
    rng = np.random.default_rng(8)
    kb = bf16.from_f64(rng.standard_normal((w.total_tokens, 2, 16)))
    vb = bf16.from_f64(rng.standard_normal((w.total_tokens, 2, 16)) * 3)
    kc, vc, ks, vs = kvcache.paged_write_fp8(kb, vb, cu, bt, w.num_pages)
    from oracle import fp8
    kq = fp8.decode(kvcache.gather(kc, cu, bt)) * kvcache.gather(ks, cu, bt)[..., None]
    k = bf16.to_f64(kb)
    assert np.max(np.abs(kq - k) / np.maximum(np.abs(k), 2.0 ** -6 * kvcache.gather(ks, cu, bt)[..., None])) <= 2.0 ** -4 + 1e-12
    assert kc.dtype == np.uint8 and ks.dtype == np.float32


def test_workload_recipes():
    w4 = workloads.WORKLOADS[3]
    assert list(w4.seqlens) == [910, 2001, 1254, 2865, 1079, 1880, 3113, 1241, 1271, 3871,
                                1617, 1452, 1882, 1404, 1559, 409]
    assert w4.total_tokens == 27808 and sum(w4.pages_per_seq) == 1746
    assert w4.attention_flops() == 491325931520.0
    w3 = workloads.WORKLOADS[2]
    assert w3.attention_flops() == 2 * 8192 ** 2 * 128 * 32
    assert w3.n_qkv == 6144 and w3.num_pages == 512
    assert sorted(workloads.block_table(w3)[0].tolist()) == list(range(512))


def test_fp8_projection_exact_small_values():
    """Codes of small powers of two with power-of-two scales: the fp8 product is
    the exact integer-like product of the decoded values."""
    from oracle import fp8 as F
    from oracle import projection as PJ
    rng = np.random.default_rng(61)
    table = {0x38: 1.0, 0x40: 2.0, 0x30: 0.5, 0xB8: -1.0, 0x00: 0.0}
    codes = np.array(list(table), dtype=np.uint8)
    xq = rng.choice(codes, (5, 32))
    wq = rng.choice(codes, (7, 32))
    sx = np.array([1, 2, 4, 0.5, 1], dtype=np.float32)
    sw = np.array([1, 1, 2, 8, 0.25, 1, 1], dtype=np.float32)
    xv = np.vectorize(table.get)(xq) * sx[:, None]
    wv = np.vectorize(table.get)(wq) * sw[:, None]
    assert np.array_equal(PJ.fp8_projection(xq, sx, wq, sw), xv @ wv.T)
    assert np.array_equal(F.decode(codes), np.array(list(table.values())))


def test_fp8_quantised_projection_close_to_exact():
    """Row-quantised operands reproduce the fp64 product within the E4M3 step."""
    from oracle import fp8 as F
    from oracle import projection as PJ
    rng = np.random.default_rng(62)
    x = rng.standard_normal((16, 256)).astype(np.float32)
    w = rng.standard_normal((24, 256)).astype(np.float32) / 16
    xq, sx = F.quantize_rows(x)
    wq, sw = F.quantize_rows(w)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    got = PJ.fp8_projection(xq, sx, wq, sw)
    # each operand carries a relative error <= 2^-4 per element; the dot
    # products of random signs average it down: a loose bound
    assert np.max(np.abs(got - exact)) < 0.15 * np.max(np.abs(exact))
