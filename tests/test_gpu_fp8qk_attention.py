"""GPU parity of the fp8 score operands: pca_quantize_heads_fp8 (bit-exact
against the oracle's power-of-two quantiser) and pca_prefill_attention_fp8qk
(against the oracle's attention on the dequantised Q and K, with the same
tolerance as the bf16 kernel), plus a crafted case that pins the kernel's own
Q quantisation exactly."""
import math

import numpy as np
import pytest
import torch

import prefill_causal_attention_amd as pca
import workloads
from oracle import attention as A
from oracle import bf16 as obf16
from oracle import fp8, fp8_attention

from _gpu_helpers import assert_close, bits, dev, require_gpu, sample_rows, say
from test_oracle_fp8_attention import FP8_SCORE_MAX_ABS, FP8_SCORE_MEAN_ABS

pytestmark = pytest.mark.gpu


def _quantize(d_x, T, H, hd, prescale=1.0):
    """GPU codes (T, H*hd) and scale bytes (T, H) in padded buffers (pad = 0xA5)."""
    w = H * hd
    codes = torch.full((T, w + 16), 0xA5, dtype=torch.uint8, device="cuda")
    lde = (H + 3) // 4 * 4 + 4
    exps = torch.full((T, lde), 0xA5, dtype=torch.uint8, device="cuda")
    pca.quantize_heads_fp8(d_x, codes[:, :w], exps[:, :H], H, hd, prescale)
    torch.cuda.synchronize()
    return codes, exps


def _oracle_quantize(x_bits, T, H, hd, prescale=1.0):
    y = obf16.to_f64(np.asarray(x_bits)).astype(np.float32).reshape(T, H, hd)
    return fp8.quantize_rows_pow2((y * np.float32(prescale)).astype(np.float32))


@pytest.mark.parametrize("T,H,hd", [(1, 8, 128), (37, 8, 128), (100, 3, 64), (65, 5, 32)])
@pytest.mark.parametrize("prescale", [1.0, float(fp8_attention.score_factor(1 / math.sqrt(128)))])
def test_quantize_heads_bit_exact(T, H, hd, prescale):
    require_gpu()
    say(f"quantize_heads_fp8 T={T} H={H} hd={hd} prescale={prescale}")
    rng = np.random.default_rng(501 + T)
    x = torch.from_numpy((rng.standard_normal((T, H * hd + 24)) *
                          2.0 ** rng.integers(-30, 30, (T, 1))).astype(np.float32)).to(torch.bfloat16)
    x[0, 8:8 + hd] = 0                                              # an all-zero row
    d = dev(x)
    codes, exps = _quantize(d[:, 8:8 + H * hd], T, H, hd, prescale)
    wc, we = _oracle_quantize(bits(x[:, 8:8 + H * hd]), T, H, hd, prescale)
    got_c = codes.cpu().numpy()
    assert np.array_equal(got_c[:, :H * hd].reshape(T, H, hd), wc)
    assert np.array_equal(exps.cpu().numpy()[:, :H], we)
    assert np.all(got_c[:, H * hd:] == 0xA5) and np.all(exps.cpu().numpy()[:, H:] == 0xA5)


def _run(w, q_off=None, rows=None, scale=None):
    """GPU fp8-score attention of a workload's Q/K/V draw and the oracle's."""
    buf, qo, ko, vo = workloads.qkv_inputs(w)
    T, hd, H, Hk = w.total_tokens, w.head_dim, w.n_head, w.n_kv_head
    nq, nk = H * hd, Hk * hd
    scale = 1 / math.sqrt(hd) if scale is None else scale
    say(f"prefill_attention_fp8qk {w.name} lens={list(w.seqlens)[:8]} T={T} heads={H}/{Hk} seeds={w.seed(3)}..")
    d = dev(buf)
    codes, exps = _quantize(d[:, ko:ko + nk], T, Hk, hd)
    o = torch.full((T, nq), float("nan"), dtype=torch.bfloat16, device="cuda")
    cu = dev(torch.from_numpy(workloads.cu_seqlens(w))) if w.num_seqs > 1 else None
    pca.prefill_attention_fp8qk(d[:, qo:qo + nq], codes[:, :nk], exps[:, :Hk], d[:, vo:vo + nk], o, H, Hk, hd,
                                cu_seqlens=cu, max_seqlen=w.max_seqlen, scale=scale)
    torch.cuda.synchronize()
    b = bits(buf)
    q, k, v = A.head_split(b, H, Hk, hd)
    kc, ke = fp8.quantize_rows_pow2(obf16.to_f64(k).astype(np.float32))
    assert np.array_equal(codes.cpu().numpy()[:, :nk].reshape(T, Hk, hd), kc)
    want = fp8_attention.fp8qk_attention(q, kc, ke, v, workloads.cu_seqlens(w), scale, rows=rows)
    got = o.float().cpu().numpy().astype(np.float64)
    return (got if rows is None else got[rows]), want, o, v


@pytest.mark.parametrize("lens,H,Hk", [([64], 2, 1), ([129], 8, 2), ([300], 4, 4), ([257], 10, 2),
                                       ([1, 2, 63, 64, 65, 190], 8, 2)])
def test_parity_small(lens, H, Hk):
    require_gpu()
    got, want, _, _ = _run(workloads.custom(41, lens, H, Hk, 128))
    assert_close(got, want, f"fp8qk {lens} {H}/{Hk}")


def test_parity_full_size_sampled():
    require_gpu()
    w = workloads.WORKLOADS[2]                       # s=8192, 32 q / 8 kv heads, hd 128
    rows = sample_rows(w.total_tokens, 48, 4242)
    got, want, o, v = _run(w, rows=rows)
    assert_close(got, want, "fp8qk gqa_s8192 sampled")
    # row 0 sees only key 0: its output is V's row 0 exactly
    v0 = np.repeat(np.asarray(v)[0], w.n_head // w.n_kv_head, axis=0).reshape(-1)
    assert np.array_equal(bits(o[0].cpu()), v0)


def test_full_size_within_quantisation_bound_of_plain_attention():
    """Against the plain definition on the unquantised bf16 Q and K (fp64, no
    fp8 anywhere): the fp8 score operands may only add the E4M3 quantisation
    error, bounded as derived for the oracle's fp8-score attention."""
    require_gpu()
    w = workloads.WORKLOADS[2]                       # s=8192, 32 q / 8 kv heads, hd 128
    rows = sample_rows(w.total_tokens, 48, 4243)
    got, _, _, _ = _run(w, rows=rows)
    buf, _, _, _ = workloads.qkv_inputs(w)
    q, k, v = A.head_split(bits(buf), w.n_head, w.n_kv_head, w.head_dim)
    plain = A.varlen_causal_attention(q, k, v, workloads.cu_seqlens(w), rows=rows)
    assert_close(got, plain, "fp8qk vs plain bf16-operand attention", max_tol=FP8_SCORE_MAX_ABS,
                 mean_tol=FP8_SCORE_MEAN_ABS)


def test_zero_q_gives_prefix_mean():
    require_gpu()
    w = workloads.custom(43, [200], 4, 2, 128)
    buf, qo, ko, vo = workloads.qkv_inputs(w)
    buf[:, qo:qo + 4 * 128] = 0
    d = dev(buf)
    codes, exps = _quantize(d[:, ko:ko + 256], 200, 2, 128)
    o = torch.empty((200, 512), dtype=torch.bfloat16, device="cuda")
    say("prefill_attention_fp8qk Q = 0")
    pca.prefill_attention_fp8qk(d[:, :512], codes[:, :256], exps[:, :2], d[:, vo:vo + 256], o, 4, 2, 128)
    torch.cuda.synchronize()
    v = obf16.to_f64(bits(buf[:, vo:vo + 256])).reshape(200, 2, 128)
    got = o.float().cpu().numpy().reshape(200, 4, 128)
    for r in (0, 1, 7, 63, 64, 199):
        for i in range(4):
            m = v[:r + 1, i // 2].mean(axis=0)
            assert np.all(np.abs(got[r, i] - m) <= 2.0 ** -8 * np.abs(m) + 1e-6), (r, i)


def test_q_quantisation_exponent_pinned():
    """scale = RN32(1 / log2 e) makes c = 1 exactly, so Q enters unchanged.
    Q rows hold 7 = 448 * 2^-6 (their amax: e = -6, code 0x7E) and 2^-15 =
    2^-9 * 2^-6 (code 0x01); both are exact only at e = -6: at e = -5 the small
    one is a tie that rounds to 0, at e = -7 the large one saturates.  Keys
    give them weight through exact K codes (0.125 on every third key, 8192 on
    odd keys), so either mistake moves the output far more than the tolerance."""
    require_gpu()
    L, hd = 96, 128
    scale = float(np.float32(1 / 1.4426950408889634))
    assert fp8_attention.score_factor(scale) == np.float32(1.0)
    q = np.zeros((L, 1, hd)); q[:, 0, 0] = 7.0; q[:, 0, 1] = 2.0 ** -15
    k = np.zeros((L, 1, hd)); k[::3, 0, 0] = 0.125; k[1::2, 0, 1] = 8192.0
    rng = np.random.default_rng(77)
    v = rng.standard_normal((L, 1, hd))
    qb, kb, vb = obf16.from_f64(q), obf16.from_f64(k), obf16.from_f64(v)
    to_t = lambda a: torch.from_numpy(a.reshape(L, hd).view(np.int16)).view(torch.bfloat16)
    dq, dk, dv = dev(to_t(qb)), dev(to_t(kb)), dev(to_t(vb))
    codes, exps = _quantize(dk, L, 1, hd)
    o = torch.empty((L, hd), dtype=torch.bfloat16, device="cuda")
    say("prefill_attention_fp8qk exact-Q pin")
    pca.prefill_attention_fp8qk(dq, codes[:, :hd], exps[:, :1], dv, o, 1, 1, hd, scale=scale)
    torch.cuda.synchronize()
    kc, ke = fp8.quantize_rows_pow2(k.astype(np.float32))
    want = fp8_attention.fp8qk_attention(qb, kc, ke, vb, [0, L], scale)
    got = o.float().cpu().numpy().astype(np.float64)
    vv = obf16.to_f64(vb)
    wrong_small = A.causal_attention(q * np.array([1.0, 0.0] + [1.0] * (hd - 2)), k, vv, scale=math.log(2.0))
    wrong_big = A.causal_attention(q * np.array([0.5] + [1.0] * (hd - 1)), k, vv, scale=math.log(2.0))
    err = np.max(np.abs(got - want))
    say(f"exact-Q pin: err={err:.3e} vs e+1 {np.max(np.abs(want - wrong_small)):.3e}, "
        f"e-1 {np.max(np.abs(want - wrong_big)):.3e}")
    assert err < 0.2 * np.max(np.abs(want - wrong_small))
    assert err < 0.2 * np.max(np.abs(want - wrong_big))
    assert_close(got, want, "fp8qk exact-Q pin", max_tol=1e-2, mean_tol=1e-3)
