"""Pins for oracle.prefix (a chunk attending over a cached prefix): brute
force with the shifted causal rule, the chunking invariant against the plain
causal attention, the prefix-0 special case, the paged read-back, and the fp8
decode.  CPU only."""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import fp8, kvcache
from oracle import prefix as PX


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def brute_force_prefix(q, k, v, P, scale):
    """Pure-Python loops: chunk row r (position P + r) weighs keys 0 .. P + r
    with math.exp, normalised by their sum."""
    Lq, H, D = len(q), len(q[0]), len(q[0][0])
    G = H // len(k[0])
    out = [[0.0] * (H * D) for _ in range(Lq)]
    for i in range(H):
        g = i // G
        for r in range(Lq):
            sc = [sum(q[r][i][d] * k[c][g][d] for d in range(D)) * scale for c in range(P + r + 1)]
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            tot = sum(w)
            for d in range(D):
                out[r][i * D + d] = sum(w[c] * v[c][g][d] for c in range(P + r + 1)) / tot
    return np.array(out)


@pytest.mark.parametrize("P,Lq,H,Hk,D", [(0, 5, 2, 2, 3), (3, 4, 4, 2, 3), (9, 6, 4, 1, 4), (1, 1, 2, 1, 2)])
def test_brute_force(P, Lq, H, Hk, D):
    q, k, v = _rand(1, Lq, H, D), _rand(2, P + Lq, Hk, D), _rand(3, P + Lq, Hk, D)
    ref = brute_force_prefix(q.tolist(), k.tolist(), v.tolist(), P, 1 / math.sqrt(D))
    got = PX.prefix_causal_attention(q, k, v, P)
    assert np.max(np.abs(got - ref)) < 1e-12


@pytest.mark.parametrize("L,P", [(40, 0), (40, 17), (40, 39), (33, 32)])
def test_chunk_rows_equal_whole_sequence_rows(L, P):
    """Processing positions P .. L-1 as a chunk over the cached prefix gives
    exactly the rows P .. L-1 of attention over the whole sequence."""
    q, k, v = _rand(4, L, 4, 8), _rand(5, L, 2, 8), _rand(6, L, 2, 8)
    whole = A.causal_attention(q, k, v)
    chunk = PX.prefix_causal_attention(q[P:], k, v, P)
    assert np.max(np.abs(chunk - whole[P:])) < 1e-12


def test_first_chunk_row_with_long_prefix_sees_whole_prefix():
    # one key dominating the prefix: row 0 of the chunk returns (almost) its value
    P, D = 20, 4
    q = np.zeros((1, 1, D)); q[0, 0, 0] = 40.0
    k = np.zeros((P + 1, 1, D)); k[7, 0, 0] = 1.0
    v = _rand(7, P + 1, 1, D)
    got = PX.prefix_causal_attention(q, k, v, P, scale=1.0)
    assert np.max(np.abs(got[0] - v[7, 0])) < 1e-12


def _pools(seed, lens, ctxs, Hk, D, pages, fp8_cache=False):
    """Write each sequence's ctx keys through a permuted block table."""
    rng = np.random.default_rng(seed)
    mp = max((c + 15) // 16 for c in ctxs)
    order = rng.permutation(pages)
    bt = np.full((len(ctxs), mp), -1, dtype=np.int64)
    at = 0
    for b, c in enumerate(ctxs):
        n = (c + 15) // 16
        bt[b, :n] = order[at:at + n]
        at += n
    cu_k = np.concatenate([[0], np.cumsum(ctxs)])
    kk = _rand(seed + 1, int(cu_k[-1]), Hk, D).astype(np.float32)
    vv = _rand(seed + 2, int(cu_k[-1]), Hk, D).astype(np.float32)
    from oracle import bf16
    kb, vb = bf16.from_f64(kk.astype(np.float64)), bf16.from_f64(vv.astype(np.float64))
    if fp8_cache:
        kc, vc, ks, vs = kvcache.paged_write_fp8(kb, vb, cu_k, bt, pages)
        return kb, vb, cu_k, bt, kc, vc, ks, vs
    kc, vc = kvcache.paged_write_bf16(kb, vb, cu_k, bt, pages)
    return kb, vb, cu_k, bt, kc, vc, None, None


def test_paged_read_back_bf16():
    lens, ctxs = [5, 9], [21, 9]
    kb, vb, cu_k, bt, kc, vc, _, _ = _pools(31, lens, ctxs, 2, 8, 6)
    cu_q = np.concatenate([[0], np.cumsum(lens)])
    q = _rand(32, int(cu_q[-1]), 4, 8)
    got = PX.paged_prefix_attention(q, cu_q, ctxs, kc, vc, bt)
    for b in range(2):
        k = kb[cu_k[b]:cu_k[b + 1]]
        v = vb[cu_k[b]:cu_k[b + 1]]
        want = PX.prefix_causal_attention(q[cu_q[b]:cu_q[b + 1]], k, v, ctxs[b] - lens[b])
        assert np.array_equal(got[cu_q[b]:cu_q[b + 1]], want)


def test_paged_read_back_fp8_decodes_with_scales():
    lens, ctxs = [4], [37]
    kb, vb, cu_k, bt, kc, vc, ks, vs = _pools(41, lens, ctxs, 2, 16, 4, fp8_cache=True)
    k, v = PX.cached_keys(kc, vc, bt, 0, 37, ks, vs)
    # decoded values match the stored codes times scales, and sit within the E4M3 step of the bf16 input
    kf = A._as_f64(kb)
    assert np.max(np.abs(k - kf) / np.maximum(np.abs(kf).max(axis=2, keepdims=True), 1e-30)) <= 2.0 ** -4
    page, slot = bt[0, 2], 3          # position 35: page 2, slot 3
    pos = 2 * 16 + slot
    assert np.array_equal(k[pos], fp8.decode(kc[page, slot]) * ks[page, slot][:, None])


def brute_force_window(q, k, v, W, scale):
    """Pure-Python loops: row r weighs keys max(0, r - W + 1) .. r."""
    L, H, D = len(q), len(q[0]), len(q[0][0])
    G = H // len(k[0])
    out = [[0.0] * (H * D) for _ in range(L)]
    for i in range(H):
        g = i // G
        for r in range(L):
            keys = range(max(0, r - W + 1), r + 1)
            sc = [sum(q[r][i][d] * k[c][g][d] for d in range(D)) * scale for c in keys]
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            tot = sum(w)
            for d in range(D):
                out[r][i * D + d] = sum(wi * v[c][g][d] for wi, c in zip(w, keys)) / tot
    return np.array(out)


@pytest.mark.parametrize("L,W,H,Hk,D", [(9, 3, 2, 1, 3), (12, 5, 4, 2, 2), (6, 1, 2, 2, 4)])
def test_window_brute_force(L, W, H, Hk, D):
    q, k, v = _rand(21, L, H, D), _rand(22, L, Hk, D), _rand(23, L, Hk, D)
    ref = brute_force_window(q.tolist(), k.tolist(), v.tolist(), W, 1 / math.sqrt(D))
    got = PX.window_causal_attention(q, k, v, W)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_window_covering_everything_is_causal():
    q, k, v = _rand(24, 30, 4, 8), _rand(25, 30, 2, 8), _rand(26, 30, 2, 8)
    full = A.causal_attention(q, k, v)
    assert np.max(np.abs(PX.window_causal_attention(q, k, v, 30) - full)) < 1e-12
    assert np.max(np.abs(PX.window_causal_attention(q, k, v, 0) - full)) < 1e-12


def test_window_one_returns_own_value():
    # W = 1: each row sees only itself, so the output is its own V row
    q, k, v = _rand(27, 10, 2, 4), _rand(28, 10, 1, 4), _rand(29, 10, 1, 4)
    got = PX.window_causal_attention(q, k, v, 1)
    for i in range(2):
        assert np.array_equal(got[:, i * 4:(i + 1) * 4], v[:, 0, :])


def test_window_chunk_rows_equal_whole_rows():
    L, P, W = 50, 23, 7
    q, k, v = _rand(30, L, 4, 8), _rand(31, L, 2, 8), _rand(32, L, 2, 8)
    whole = PX.window_causal_attention(q, k, v, W)
    chunk = PX.window_causal_attention(q[P:], k, v, W, prefix_len=P)
    assert np.max(np.abs(chunk - whole[P:])) < 1e-12


def brute_force_varlen_window(q, k, v, cu, W, scale, rows):
    """Pure-Python loops over a packed batch: global row t of sequence b
    (tokens cu[b] .. cu[b+1]-1) weighs the keys of its own sequence at global
    positions max(cu[b], t - W + 1) .. t."""
    H, D = len(q[0]), len(q[0][0])
    G = H // len(k[0])
    out = []
    for t in rows:
        b = max(i for i in range(len(cu) - 1) if cu[i] <= t)
        keys = range(max(cu[b], t - W + 1), t + 1)
        o = [0.0] * (H * D)
        for i in range(H):
            g = i // G
            sc = [sum(q[t][i][d] * k[c][g][d] for d in range(D)) * scale for c in keys]
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            tot = sum(w)
            for d in range(D):
                o[i * D + d] = sum(wi * v[c][g][d] for wi, c in zip(w, keys)) / tot
        out.append(o)
    return np.array(out)


@pytest.mark.parametrize("lens,W", [([7, 1, 9], 3), ([5, 12], 4), ([3, 3, 3], 1), ([10, 2], 20)])
def test_varlen_window_brute_force(lens, W):
    """Packed sequences: the window never reaches into the previous sequence,
    and the rows= selection (global indices) picks the right rows."""
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, Hk, D = int(cu[-1]), 4, 2, 3
    q, k, v = _rand(40, T, H, D), _rand(41, T, Hk, D), _rand(42, T, Hk, D)
    rows = [0, T - 1] + [int(c) for c in cu[1:-1]] + [int(c) - 1 for c in cu[1:-1]] + [T // 2]
    rows = sorted(set(rows))
    ref = brute_force_varlen_window(q.tolist(), k.tolist(), v.tolist(), cu.tolist(), W, 1 / math.sqrt(D), rows)
    assert np.max(np.abs(PX.varlen_window_attention(q, k, v, cu, W, rows=np.array(rows)) - ref)) < 1e-12
    full = brute_force_varlen_window(q.tolist(), k.tolist(), v.tolist(), cu.tolist(), W, 1 / math.sqrt(D), range(T))
    assert np.max(np.abs(PX.varlen_window_attention(q, k, v, cu, W) - full)) < 1e-12


def test_varlen_window_limits():
    """W at least the longest sequence is the plain packed causal attention;
    W = 1 returns every row's own V."""
    lens = [13, 1, 30, 8]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v = _rand(43, T, 6, 8), _rand(44, T, 3, 8), _rand(45, T, 3, 8)
    plain = A.varlen_causal_attention(q, k, v, cu)
    assert np.max(np.abs(PX.varlen_window_attention(q, k, v, cu, 30) - plain)) < 1e-12
    assert np.max(np.abs(PX.varlen_window_attention(q, k, v, cu, 10 ** 6) - plain)) < 1e-12
    own = PX.varlen_window_attention(q, k, v, cu, 1)
    for i in range(6):
        assert np.array_equal(own[:, i * 8:(i + 1) * 8], v[:, i // 2, :])
