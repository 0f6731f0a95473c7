"""GPU parity of pca_prefill_attention against the fp64 oracle, plus the
closed-form and invariant pins run on the kernel itself."""
import math

import numpy as np
import pytest
import torch

import prefill_causal_attention_amd as pca
import workloads
from oracle import attention as A
from oracle import bf16 as obf16

from _gpu_helpers import assert_close, bits, dev, require_gpu, sample_rows, say

pytestmark = pytest.mark.gpu


def _views(w, buf):
    nq, nk = w.n_head * w.head_dim, w.n_kv_head * w.head_dim
    return buf[:, :nq], buf[:, nq:nq + nk], buf[:, nq + nk:nq + 2 * nk]


def _gpu_attention(w, buf_host, o_pad=0):
    d_buf = dev(buf_host)
    q, k, v = _views(w, d_buf)
    T = w.total_tokens
    o = torch.full((T, w.n_head * w.head_dim + o_pad), float("nan"), dtype=torch.bfloat16, device="cuda")
    cu = dev(torch.from_numpy(workloads.cu_seqlens(w))) if w.num_seqs > 1 else None
    pca.prefill_attention(q, k, v, o[:, :w.n_head * w.head_dim], w.n_head, w.n_kv_head, w.head_dim,
                          cu_seqlens=cu, max_seqlen=w.max_seqlen)
    torch.cuda.synchronize()
    return o


def _oracle_inputs(w, buf_host):
    b = bits(buf_host)
    T, hd = w.total_tokens, w.head_dim
    q, k, v = A.head_split(b, w.n_head, w.n_kv_head, hd)
    return q, k, v


def _check_parity(w, rows=None, ld_pad=0, o_pad=0):
    buf, *_ = workloads.qkv_inputs(w, ld=w.n_qkv + ld_pad)
    say(f"prefill_attention {w.name} lens={list(w.seqlens)[:8]}{'...' if w.num_seqs > 8 else ''} "
        f"T={w.total_tokens} heads={w.n_head}/{w.n_kv_head} hd={w.head_dim} seeds={w.seed(3)}..{w.seed(5)}")
    o = _gpu_attention(w, buf, o_pad)
    q, k, v = _oracle_inputs(w, buf)
    cu = workloads.cu_seqlens(w)
    want = A.varlen_causal_attention(q, k, v, cu, rows=rows)
    got = o[:, :w.n_head * w.head_dim].float().cpu().numpy().astype(np.float64)
    got = got if rows is None else got[rows]
    assert_close(got, want, w.name)
    if o_pad:
        assert torch.isnan(o[:, w.n_head * w.head_dim:].float()).all(), "wrote outside the heads"
    return o


@pytest.mark.parametrize("lens,H,Hk,hd", [
    ([64], 2, 2, 32),
    ([100], 4, 2, 64),
    ([129], 8, 2, 128),
    ([300], 4, 4, 128),
    ([257], 10, 2, 128),                   # G = 5, tasks straddle query blocks
    ([1, 2, 63, 64, 65, 190], 8, 2, 128),  # varlen with ragged tails and a 1-token sequence
    ([33, 7, 200], 4, 1, 64),
])
def test_parity_small(lens, H, Hk, hd):
    require_gpu()
    _check_parity(workloads.custom(31, lens, H, Hk, hd), ld_pad=8, o_pad=8)


def test_parity_tiny_mha_workload():
    """The tiny MHA workload (s=64, 2 heads, hd 32): fp32 Q/K/V drawn and rounded to
    bf16 once; both sides consume those values."""
    require_gpu()
    w = workloads.WORKLOADS[0]
    o = _check_parity(w)
    # for information: error against the unrounded fp32 draw
    rng_q = np.random.default_rng(w.seed(3)).standard_normal((64, 64), dtype=np.float32)
    rng_k = np.random.default_rng(w.seed(4)).standard_normal((64, 64), dtype=np.float32)
    rng_v = np.random.default_rng(w.seed(5)).standard_normal((64, 64), dtype=np.float32)
    ref32 = A.causal_attention(rng_q.reshape(64, 2, 32), rng_k.reshape(64, 2, 32), rng_v.reshape(64, 2, 32))
    d = np.abs(o.float().cpu().numpy() - ref32)
    say(f"tiny MHA vs unrounded fp32 inputs: max_abs={d.max():.3e} mean_abs={d.mean():.3e}")


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_parity_full_size_sampled_rows(idx):
    require_gpu()
    w = workloads.WORKLOADS[idx - 1]
    rows = []
    cu = workloads.cu_seqlens(w)
    for b in range(w.num_seqs):
        L = w.seqlens[b]
        # the longest sequence: 512 sampled query rows (all heads) plus the edges
        n = 500 if L >= 32768 else (96 if w.num_seqs == 1 else 12)
        rows.extend((cu[b] + sample_rows(L, n, 100 + b)).tolist())
    _check_parity(w, rows=np.array(rows))


def _mk(T, H, Hk, hd, seed):
    w = workloads.custom(seed, [T], H, Hk, hd)
    buf, *_ = workloads.qkv_inputs(w)
    return w, buf


def test_row0_equals_v0_bitwise():
    require_gpu()
    w, buf = _mk(200, 8, 2, 128, 41)
    o = _gpu_attention(w, buf)
    q, k, v = _views(w, buf)
    for i in range(w.n_head):
        g = i // w.group
        assert torch.equal(o[0, i * 128:(i + 1) * 128].cpu(), v[0, g * 128:(g + 1) * 128]), f"head {i}"


def test_zero_q_gives_prefix_mean():
    require_gpu()
    w, buf = _mk(256, 4, 2, 64, 42)
    buf[:, :4 * 64] = 0
    o = _gpu_attention(w, buf)
    v = obf16.to_f64(bits(buf[:, 4 * 64 + 2 * 64:]).reshape(256, 2, 64))
    got = o.float().cpu().numpy().astype(np.float64)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(got), 1e-30))) - 7)
    for i in range(4):
        mean = np.cumsum(v[:, i // 2, :], axis=0) / np.arange(1, 257)[:, None]
        err = np.abs(got[:, i * 64:(i + 1) * 64] - mean)
        # within one bf16 ulp of the exact prefix mean (P is exactly 1 everywhere)
        assert np.all(err <= 1.01 * ulp[:, i * 64:(i + 1) * 64] + 1e-6), float(err.max())


def test_constant_v_gives_one():
    require_gpu()
    w, buf = _mk(300, 4, 1, 128, 43)
    buf[:, 4 * 128 + 128:] = 1.0
    buf[:, :4 * 128] *= 4
    o = _gpu_attention(w, buf)
    assert float((o.float() - 1).abs().max()) <= 4e-3


def test_gqa_equals_mha_on_repeated_kv():
    require_gpu()
    T, H, Hk, hd = 333, 8, 2, 128
    wg, buf = _mk(T, H, Hk, hd, 44)
    og = _gpu_attention(wg, buf)
    q, k, v = _views(wg, buf)
    wm = workloads.custom(44, [T], H, H, hd)
    rep = lambda t: t.reshape(T, Hk, 1, hd).expand(T, Hk, H // Hk, hd).reshape(T, H * hd)
    bm = torch.cat([q, rep(k), rep(v)], dim=1).contiguous()
    om = _gpu_attention(wm, bm)
    d = (og.float() - om.float()).abs().max().item()
    say(f"GQA vs repeated-MHA max diff {d}")
    assert d == 0.0


def test_future_perturbation_bitwise():
    require_gpu()
    T, H, Hk, hd = 400, 4, 2, 128
    w, buf = _mk(T, H, Hk, hd, 45)
    base = _gpu_attention(w, buf)
    r = 150
    pert = buf.clone()
    pert[r + 1:, H * hd:] = 1e4
    out = _gpu_attention(w, pert)
    assert torch.equal(base[:r + 1], out[:r + 1])
    assert not torch.equal(base[r + 1:], out[r + 1:])


def test_varlen_equals_each_sequence_alone_bitwise():
    require_gpu()
    lens = [70, 1, 128, 259]
    w = workloads.custom(46, lens, 8, 2, 128)
    buf, *_ = workloads.qkv_inputs(w)
    packed = _gpu_attention(w, buf)
    cu = workloads.cu_seqlens(w)
    for b, L in enumerate(lens):
        wb = workloads.custom(46, [L], 8, 2, 128)
        alone = _gpu_attention(wb, buf[cu[b]:cu[b + 1]].clone())
        assert torch.equal(packed[cu[b]:cu[b + 1]], alone), f"sequence {b}"


@pytest.mark.parametrize("lens,H,Hk", [
    # deep enough for the one-workgroup-per-CU walk, with empty virtual
    # workgroups (short sequences next to long ones): ranked batch slots
    ([1500, 40, 700, 2100, 300, 1, 900, 64], 32, 8),
    ([1200, 2600, 33, 800], 16, 4),
    # more than 64 sequences: batch slots in packing order
    ([97 * (1 + (i * 37) % 11) for i in range(72)], 16, 8),
])
def test_deep_varlen_batch_equals_each_sequence_alone_bitwise(lens, H, Hk):
    require_gpu()
    w = workloads.custom(49, lens, H, Hk, 128)
    buf, *_ = workloads.qkv_inputs(w)
    say(f"prefill_attention deep varlen: {len(lens)} seqs T={w.total_tokens} heads={H}/{Hk}")
    packed = _gpu_attention(w, buf)
    cu = workloads.cu_seqlens(w)
    for b, L in enumerate(lens):
        wb = workloads.custom(49, [L], H, Hk, 128)
        alone = _gpu_attention(wb, buf[cu[b]:cu[b + 1]].clone())
        assert torch.equal(packed[cu[b]:cu[b + 1]], alone), f"sequence {b} (length {L})"
    # and the batch against the oracle on sampled rows
    q, k, v = _oracle_inputs(w, buf)
    rows = sample_rows(w.total_tokens, 64, seed=49)
    want = A.varlen_causal_attention(q, k, v, cu, rows=rows)
    got = packed[:, :H * 128].float().cpu().numpy().astype(np.float64)[rows]
    assert_close(got, want, "deep varlen")


def test_growing_scores_move_the_reference_on_every_tile():
    """Keys whose magnitude steps up every 64 positions raise a row's scores by
    about 16 (in log2 units) from one kv tile to the next, far past the
    2^12 tile-sum limit of the lazy softmax: every row moves its reference on
    every new tile it sees, so O and l are rescaled mid-sequence many times
    (with N(0,1) inputs a row's reference practically never moves after its
    first tile).  The output must still match the oracle."""
    require_gpu()
    T, H, Hk, hd = 520, 4, 2, 128
    w, buf = _mk(T, H, Hk, hd, 50)
    rng = np.random.default_rng(50)
    q = 0.25 + 0.05 * rng.standard_normal((T, H * hd))
    # q.k grows by 128 * 0.25 * 4 = 128 per tile: 128 / sqrt(128) * log2(e) = 16.3
    kmag = 4.0 * (np.arange(T) // 64)[:, None] + 0.1 * rng.standard_normal((T, Hk * hd))
    buf[:, :H * hd] = torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16)
    buf[:, H * hd:(H + Hk) * hd] = torch.from_numpy(kmag.astype(np.float32)).to(torch.bfloat16)
    say(f"prefill_attention growing scores T={T} heads={H}/{Hk} hd={hd} seed=50")
    o = _gpu_attention(w, buf)
    qq, kk, vv = _oracle_inputs(w, buf)
    want = A.causal_attention(qq, kk, vv)
    assert_close(o.float().cpu().numpy(), want, "growing scores")


def test_deterministic_bitwise():
    require_gpu()
    w, buf = _mk(1000, 8, 2, 128, 47)
    a = _gpu_attention(w, buf)
    b = _gpu_attention(w, buf)
    assert torch.equal(a, b)


def test_scale_argument_is_used():
    require_gpu()
    w, buf = _mk(96, 2, 2, 64, 48)
    d_buf = dev(buf)
    q, k, v = _views(w, d_buf)
    o = torch.empty((96, 128), dtype=torch.bfloat16, device="cuda")
    pca.prefill_attention(q, k, v, o, 2, 2, 64, scale=0.3)
    torch.cuda.synchronize()
    qq, kk, vv = _oracle_inputs(w, buf)
    want = A.causal_attention(qq, kk, vv, scale=0.3)
    assert_close(o.float().cpu().numpy(), want, "scale=0.3")


def test_invalid_arguments_rejected():
    require_gpu()
    x = torch.zeros((16, 256), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((16, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pca.PcaError):
        pca.prefill_attention(x[:, :128], x[:, :96], x[:, :96], o[:, :128], 4, 3, 32)   # 4 % 3 != 0
    with pytest.raises(pca.PcaError):
        pca.prefill_attention(x, x, x, o, 1, 1, 256)                                     # head_dim 256
    assert float(o.abs().sum()) == 0.0
