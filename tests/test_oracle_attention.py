"""Pins for oracle.attention: brute force, closed forms, invariants and the
pages' blockwise algorithm.  CPU only."""
import math

import numpy as np
import pytest

from oracle import attention as A


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def brute_force(q, k, v, scale):
    """Pure-Python loops with math.exp: for each head and row, weights over the
    keys c <= r only (no mask array), normalised by their sum."""
    L, H, D = len(q), len(q[0]), len(q[0][0])
    G = H // len(k[0])
    out = [[0.0] * (H * D) for _ in range(L)]
    for i in range(H):
        g = i // G
        for r in range(L):
            sc = []
            for c in range(r + 1):
                sc.append(sum(q[r][i][d] * k[c][g][d] for d in range(D)) * scale)
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            tot = sum(w)
            for d in range(D):
                out[r][i * D + d] = sum(w[c] * v[c][g][d] for c in range(r + 1)) / tot
    return np.array(out)


@pytest.mark.parametrize("L,H,Hk,D", [(7, 2, 2, 4), (9, 4, 2, 3), (12, 4, 1, 5), (5, 8, 2, 2)])
def test_brute_force_matches(L, H, Hk, D):
    q, k, v = _rand(1, L, H, D), _rand(2, L, Hk, D), _rand(3, L, Hk, D)
    scale = 1.0 / math.sqrt(D)
    ref = brute_force(q.tolist(), k.tolist(), v.tolist(), scale)
    got = A.causal_attention(q, k, v)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_brute_force_tiny_mha_shape():
    # the tiny MHA workload's shape (s=64, 2 heads, head_dim 32), on a 24-row prefix
    q, k, v = _rand(11, 24, 2, 32), _rand(12, 24, 2, 32), _rand(13, 24, 2, 32)
    ref = brute_force(q.tolist(), k.tolist(), v.tolist(), 1 / math.sqrt(32))
    assert np.max(np.abs(A.causal_attention(q, k, v) - ref)) < 1e-12


def test_two_token_closed_form():
    # L=2, one head: row 1 = (e^a v0 + e^b v1) / (e^a + e^b), a = q1.k0*s, b = q1.k1*s
    q, k, v = _rand(4, 2, 1, 3), _rand(5, 2, 1, 3), _rand(6, 2, 1, 3)
    s = 1 / math.sqrt(3)
    a = float(q[1, 0] @ k[0, 0]) * s
    b = float(q[1, 0] @ k[1, 0]) * s
    want = (math.exp(a) * v[0, 0] + math.exp(b) * v[1, 0]) / (math.exp(a) + math.exp(b))
    got = A.causal_attention(q, k, v)
    assert np.allclose(got[1], want, rtol=0, atol=1e-14)
    assert np.array_equal(got[0], v[0, 0])


def test_softmax_rows_sum_to_one_and_causal_zero():
    L = 40
    s = _rand(7, L, L) * 3
    p = A.softmax_two_pass(s + A.causal_mask_rows(np.arange(L), L))
    assert np.max(np.abs(p.sum(axis=1) - 1)) < 1e-12
    assert np.all(p[np.triu_indices(L, 1)] == 0.0)
    assert np.all(p[np.tril_indices(L)] > 0.0)


def test_row0_is_v0_exactly():
    q, k, v = _rand(8, 33, 4, 16), _rand(9, 33, 2, 16), _rand(10, 33, 2, 16)
    o = A.causal_attention(q, k, v)
    for i in range(4):
        assert np.array_equal(o[0, i * 16:(i + 1) * 16], v[0, i // 2])


def test_zero_q_gives_causal_prefix_mean():
    L, H, Hk, D = 50, 4, 2, 8
    q = np.zeros((L, H, D))
    k, v = _rand(14, L, Hk, D), _rand(15, L, Hk, D)
    o = A.causal_attention(q, k, v)
    for i in range(H):
        g = i // 2
        want = np.cumsum(v[:, g, :], axis=0) / np.arange(1, L + 1)[:, None]
        assert np.max(np.abs(o[:, i * D:(i + 1) * D] - want)) < 1e-13


def test_constant_v_gives_constant_output():
    L, H, D = 37, 2, 8
    q, k = _rand(16, L, H, D) * 4, _rand(17, L, H, D) * 4
    v = np.full((L, H, D), 1.0)
    assert np.max(np.abs(A.causal_attention(q, k, v) - 1.0)) < 1e-14


def test_gqa_equals_mha_on_repeated_kv():
    L, H, Hk, D = 29, 8, 2, 6
    q, k, v = _rand(18, L, H, D), _rand(19, L, Hk, D), _rand(20, L, Hk, D)
    g = A.causal_attention(q, k, v)
    m = A.causal_attention(q, np.repeat(k, H // Hk, axis=1), np.repeat(v, H // Hk, axis=1))
    assert np.array_equal(g, m)


def test_future_perturbation_does_not_leak():
    L, H, D = 31, 2, 4
    q, k, v = _rand(21, L, H, D), _rand(22, L, H, D), _rand(23, L, H, D)
    base = A.causal_attention(q, k, v)
    r = 13
    k2, v2 = k.copy(), v.copy()
    k2[r + 1:] = 1e4
    v2[r + 1:] = -1e4
    pert = A.causal_attention(q, k2, v2)
    assert np.array_equal(base[:r + 1], pert[:r + 1])
    assert not np.allclose(base[r + 1:], pert[r + 1:])


@pytest.mark.parametrize("bq,bk", [(16, 16), (16, 32), (32, 16), (7, 5), (64, 64)])
def test_online_softmax_blockwise_equals_two_pass(bq, bk):
    L, H, Hk, D = 77, 4, 2, 8
    q, k, v = _rand(24, L, H, D) * 2, _rand(25, L, Hk, D) * 2, _rand(26, L, Hk, D)
    a = A.causal_attention(q, k, v)
    b = A.online_softmax_attention(q, k, v, block_q=bq, block_k=bk)
    assert np.max(np.abs(a - b)) < 1e-12


def test_sampled_rows_equal_full():
    L, H, Hk, D = 90, 4, 1, 8
    q, k, v = _rand(27, L, H, D), _rand(28, L, Hk, D), _rand(29, L, Hk, D)
    full = A.causal_attention(q, k, v)
    rows = np.array([0, 1, 15, 16, 47, 89])
    part = A.causal_attention(q, k, v, rows=rows, row_block=4)
    assert np.max(np.abs(full[rows] - part)) < 1e-13


def test_varlen_equals_each_sequence_alone():
    lens = [5, 17, 1, 30]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, Hk, D = cu[-1], 4, 2, 4
    q, k, v = _rand(30, T, H, D), _rand(31, T, Hk, D), _rand(32, T, Hk, D)
    packed = A.varlen_causal_attention(q, k, v, cu)
    for b in range(len(lens)):
        s0, s1 = cu[b], cu[b + 1]
        assert np.array_equal(packed[s0:s1], A.causal_attention(q[s0:s1], k[s0:s1], v[s0:s1]))
    rows = np.array([0, 4, 5, 21, 22, T - 1])
    # a different row subset changes the BLAS blocking, hence rounding order only
    assert np.max(np.abs(A.varlen_causal_attention(q, k, v, cu, rows=rows) - packed[rows])) < 1e-13


def test_default_scale_matches_page_figure(golden):
    row = {r[0]: r for r in golden("sizes_pages.txt")}["scale_hd128"]
    assert abs(math.sqrt(128) - float(row[2])) < 1e-4
    # the oracle divides by sqrt(head_dim): one key, one query, value = score weight 1
    q = np.ones((2, 1, 128))
    k = np.zeros((2, 1, 128))
    k[1, 0, 0] = math.sqrt(128) * math.log(3.0)      # score q1.k1/sqrt(128) = ln 3
    v = np.zeros((2, 1, 128))
    v[1, 0, 0] = 1.0
    o = A.causal_attention(q, k, v)
    assert abs(o[1, 0] - 3.0 / 4.0) < 1e-14           # e^{ln3} / (e^0 + e^{ln3})


def test_head_split_columns():
    n_head, n_kv, hd, T = 4, 2, 3, 5
    N = (n_head + 2 * n_kv) * hd
    y = np.arange(T * N).reshape(T, N)
    q, k, v = A.head_split(y, n_head, n_kv, hd)
    for t in range(T):
        for i in range(n_head):
            for d in range(hd):
                assert q[t, i, d] == t * N + i * hd + d
        for j in range(n_kv):
            for d in range(hd):
                assert k[t, j, d] == t * N + n_head * hd + j * hd + d
                assert v[t, j, d] == t * N + (n_head + n_kv) * hd + j * hd + d


def test_scores_size_figure(golden):
    row = {r[0]: r for r in golden("sizes_pages.txt")}["scores_fp16_s8192_32heads"]
    assert 8192 * 8192 * 32 * 2 == int(row[2])
