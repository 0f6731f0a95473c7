"""GPU parity of pca_prefill_attention_paged (a prefill chunk over its cached
prefix, bf16 or fp8 pages) against the fp64 oracle, plus invariants run on the kernel itself:
with no prefix it equals pca_prefill_attention bit for bit, and a chunk's rows
equal the same rows of the whole sequence attended in one piece."""
import numpy as np
import pytest
import torch

import prefill_causal_attention_amd as pca
import workloads
from oracle import attention as A
from oracle import kvcache
from oracle import prefix as PX

from _gpu_helpers import assert_close, bits, dev, require_gpu, sample_rows, say

pytestmark = pytest.mark.gpu


def _case(seed, chunks, prefixes, H, Hk, hd, spare=3):
    """Seeded draws: per sequence b, prefix P_b + chunk L_b keys (N(0,1) bf16),
    placed in permuted pages by the oracle's scatter; chunk queries N(0,1)."""
    ctx = [p + l for p, l in zip(prefixes, chunks)]
    rng = np.random.default_rng(seed)
    npg = [(c + 15) // 16 for c in ctx]
    pages = sum(npg) + spare
    order = rng.permutation(pages)
    bt = np.full((len(ctx), max(npg)), -1, dtype=np.int64)
    at = 0
    for b, n in enumerate(npg):
        bt[b, :n] = order[at:at + n]
        at += n
    cu_k = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int64)
    kb = bits(workloads.normal_bf16(seed + 1, (int(cu_k[-1]), Hk * hd))).reshape(-1, Hk, hd)
    vb = bits(workloads.normal_bf16(seed + 2, (int(cu_k[-1]), Hk * hd))).reshape(-1, Hk, hd)
    kc, vc = kvcache.paged_write_bf16(kb, vb, cu_k, bt, pages)
    cu_q = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = workloads.normal_bf16(seed + 3, (int(cu_q[-1]), H * hd))
    return dict(ctx=np.array(ctx, dtype=np.int32), bt=bt, kb=kb, vb=vb, cu_k=cu_k, kc=kc, vc=vc, cu_q=cu_q, q=q,
                H=H, Hk=Hk, hd=hd)


def _gpu(c, o_pad=8, window=0):
    T = int(c["cu_q"][-1])
    nq = c["H"] * c["hd"]
    o = torch.full((T, nq + o_pad), float("nan"), dtype=torch.bfloat16, device="cuda")
    d_bt = dev(torch.from_numpy(np.where(c["bt"] < 0, 0, c["bt"]).astype(np.int32)))
    kc = dev(torch.from_numpy(c["kc"].view(np.int16)))
    vc = dev(torch.from_numpy(c["vc"].view(np.int16)))
    cu = dev(torch.from_numpy(c["cu_q"])) if len(c["ctx"]) > 1 else None
    pca.prefill_attention_paged(dev(c["q"]), o[:, :nq], kc, vc, d_bt, dev(torch.from_numpy(c["ctx"])),
                                c["H"], c["Hk"], c["hd"], cu_seqlens=cu,
                                max_seqlen=int(np.diff(c["cu_q"]).max()), max_ctx=int(c["ctx"].max()),
                                window=window)
    torch.cuda.synchronize()
    assert torch.isnan(o[:, nq:].float()).all(), "wrote outside the heads"
    return o[:, :nq]


def _oracle(c, rows=None):
    qb = bits(c["q"]).reshape(-1, c["H"], c["hd"])
    return PX.paged_prefix_attention(qb, c["cu_q"], c["ctx"], c["kc"], c["vc"], c["bt"], rows=rows)


@pytest.mark.parametrize("chunks,prefixes,H,Hk,hd", [
    ([37], [100], 4, 2, 128),               # prefix and chunk not tile multiples
    ([64], [64], 8, 2, 64),
    ([129, 1, 50], [0, 300, 17], 8, 2, 128),  # varlen: no prefix, a 1-row chunk, ragged
    ([200], [333], 4, 4, 32),
    ([96, 40], [512, 1], 10, 2, 128),       # G = 5
])
def test_parity_small(chunks, prefixes, H, Hk, hd):
    require_gpu()
    c = _case(71, chunks, prefixes, H, Hk, hd)
    say(f"prefill_attention_paged chunks={chunks} prefixes={prefixes} heads={H}/{Hk} hd={hd} seed=71")
    got = _gpu(c).float().cpu().numpy()
    assert_close(got, _oracle(c), "paged")


def test_no_prefix_equals_contiguous_kernel_bitwise():
    """ctx = chunk: the paged kernel reads the same keys through the pages and
    must give exactly pca_prefill_attention's output."""
    require_gpu()
    c = _case(72, [300, 77], [0, 0], 8, 2, 128)
    got = _gpu(c)
    kv = np.concatenate([c["kb"].reshape(c["kb"].shape[0], -1), c["vb"].reshape(c["vb"].shape[0], -1)], axis=1)
    kvt = dev(torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16))
    nk = c["Hk"] * c["hd"]
    o = torch.empty_like(got)
    pca.prefill_attention(dev(c["q"]), kvt[:, :nk], kvt[:, nk:], o, c["H"], c["Hk"], c["hd"],
                          cu_seqlens=dev(torch.from_numpy(c["cu_q"])), max_seqlen=300)
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), bits(o))


@pytest.mark.parametrize("P", [64, 200, 512])
def test_chunk_rows_equal_whole_sequence_rows_bitwise(P):
    """The chunk's rows (positions P ..) equal rows P .. of the whole sequence
    attended at once: every row sees the same kv tiles in the same order."""
    require_gpu()
    L, H, Hk, hd = 700, 8, 2, 128
    c = _case(73, [L - P], [P], H, Hk, hd)
    got = _gpu(c)
    kv = np.concatenate([c["kb"].reshape(L, -1), c["vb"].reshape(L, -1)], axis=1)
    kvt = dev(torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16))
    qfull = dev(workloads.normal_bf16(74, (L, H * hd)))
    qfull[P:] = dev(c["q"])
    o = torch.empty((L, H * hd), dtype=torch.bfloat16, device="cuda")
    nk = Hk * hd
    pca.prefill_attention(qfull, kvt[:, :nk], kvt[:, nk:], o, H, Hk, hd)
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), bits(o[P:]))


def test_long_prefix_gqa_sampled():
    """s = 8192 GQA 32/8 hd128 processed as a last 512-row chunk over a 7680-key prefix."""
    require_gpu()
    c = _case(75, [512], [7680], 32, 8, 128, spare=64)
    got = _gpu(c).float().cpu().numpy()
    rows = sample_rows(512, 48, 76, must=(0, 1, 63, 64, 511))
    assert_close(got[rows], _oracle(c, rows=rows), "paged s=8192 chunk")


def test_growing_scores_move_the_reference_on_every_tile():
    """Paged keys whose magnitude steps up every 64 positions raise the chunk
    rows' scores by about 16 (log2 units) per kv tile, so every row moves its
    softmax reference on every tile of the prefix and of the chunk (O and l
    rescaled many times); the output must still match the oracle."""
    require_gpu()
    H, Hk, hd = 4, 2, 128
    c = _case(77, [100], [300], H, Hk, hd)
    ctx = int(c["ctx"][0])
    rng = np.random.default_rng(77)
    kmag = 4.0 * (np.arange(ctx) // 64)[:, None] + 0.1 * rng.standard_normal((ctx, Hk * hd))
    c["kb"] = bits(torch.from_numpy(kmag.astype(np.float32)).to(torch.bfloat16)).reshape(-1, Hk, hd)
    c["kc"], c["vc"] = kvcache.paged_write_bf16(c["kb"], c["vb"], c["cu_k"], c["bt"], c["kc"].shape[0])
    q = 0.25 + 0.05 * rng.standard_normal((100, H * hd))
    c["q"] = torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16)
    say(f"prefill_attention_paged growing scores: chunk 100 over prefix 300, heads {H}/{Hk}, seed 77")
    assert_close(_gpu(c).float().cpu().numpy(), _oracle(c), "paged growing scores")


def _case_fp8(seed, chunks, prefixes, H, Hk, hd, spare=3):
    """As _case, with the keys quantised into fp8 pools (codes + scales) by the oracle."""
    c = _case(seed, chunks, prefixes, H, Hk, hd, spare)
    pages = c["kc"].shape[0]
    kc, vc, ks, vs = kvcache.paged_write_fp8(c["kb"], c["vb"], c["cu_k"], c["bt"], pages)
    c.update(kc=kc, vc=vc, ks=ks, vs=vs)
    return c


def _gpu_fp8(c, o_pad=8):
    T = int(c["cu_q"][-1])
    nq = c["H"] * c["hd"]
    o = torch.full((T, nq + o_pad), float("nan"), dtype=torch.bfloat16, device="cuda")
    d_bt = dev(torch.from_numpy(np.where(c["bt"] < 0, 0, c["bt"]).astype(np.int32)))
    cu = dev(torch.from_numpy(c["cu_q"])) if len(c["ctx"]) > 1 else None
    pca.prefill_attention_paged(dev(c["q"]), o[:, :nq], dev(torch.from_numpy(c["kc"])), dev(torch.from_numpy(c["vc"])),
                                d_bt, dev(torch.from_numpy(c["ctx"])), c["H"], c["Hk"], c["hd"], cu_seqlens=cu,
                                max_seqlen=int(np.diff(c["cu_q"]).max()), max_ctx=int(c["ctx"].max()),
                                cache_dtype="fp8_e4m3", k_scale=dev(torch.from_numpy(c["ks"])),
                                v_scale=dev(torch.from_numpy(c["vs"])))
    torch.cuda.synchronize()
    assert torch.isnan(o[:, nq:].float()).all(), "wrote outside the heads"
    return o[:, :nq]


def _oracle_fp8(c, rows=None):
    qb = bits(c["q"]).reshape(-1, c["H"], c["hd"])
    return PX.paged_prefix_attention(qb, c["cu_q"], c["ctx"], c["kc"], c["vc"], c["bt"], rows=rows,
                                     k_scale=c["ks"], v_scale=c["vs"])


@pytest.mark.parametrize("chunks,prefixes,H,Hk,hd", [
    ([37], [100], 4, 2, 128),
    ([129, 1, 50], [0, 300, 17], 8, 2, 128),
    ([64], [64], 8, 2, 64),
    ([200], [333], 4, 4, 32),
    ([96, 40], [512, 1], 10, 2, 128),
])
def test_fp8_pages_parity(chunks, prefixes, H, Hk, hd):
    """E4M3 pages dequantised on load (code x scale, bf16 on chip) against the
    oracle's fp64 decode of the same codes and scales."""
    require_gpu()
    c = _case_fp8(77, chunks, prefixes, H, Hk, hd)
    say(f"prefill_attention_paged fp8 chunks={chunks} prefixes={prefixes} heads={H}/{Hk} hd={hd} seed=77")
    got = _gpu_fp8(c).float().cpu().numpy()
    assert_close(got, _oracle_fp8(c), "paged fp8")


def test_fp8_pages_long_prefix_sampled():
    """s = 32768-style long context: a 512-row chunk over a 16384-key fp8 prefix, GQA 40/8 hd128."""
    require_gpu()
    c = _case_fp8(78, [512], [16384], 40, 8, 128, spare=16)
    got = _gpu_fp8(c).float().cpu().numpy()
    rows = sample_rows(512, 32, 79, must=(0, 1, 63, 64, 511))
    assert_close(got[rows], _oracle_fp8(c, rows=rows), "paged fp8 16k prefix")


def _run_table(c, bt, fp8):
    """The paged kernel with the given raw block table (entries passed as they are)."""
    T = int(c["cu_q"][-1])
    nq = c["H"] * c["hd"]
    o = torch.full((T, nq + 8), float("nan"), dtype=torch.bfloat16, device="cuda")
    cu = dev(torch.from_numpy(c["cu_q"])) if len(c["ctx"]) > 1 else None
    kc = c["kc"] if fp8 else c["kc"].view(np.int16)
    vc = c["vc"] if fp8 else c["vc"].view(np.int16)
    extra = dict(cache_dtype="fp8_e4m3", k_scale=dev(torch.from_numpy(c["ks"])),
                 v_scale=dev(torch.from_numpy(c["vs"]))) if fp8 else {}
    pca.prefill_attention_paged(dev(c["q"]), o[:, :nq], dev(torch.from_numpy(kc)), dev(torch.from_numpy(vc)),
                                dev(torch.from_numpy(bt.astype(np.int32))), dev(torch.from_numpy(c["ctx"])),
                                c["H"], c["Hk"], c["hd"], cu_seqlens=cu, max_seqlen=int(np.diff(c["cu_q"]).max()),
                                max_ctx=int(c["ctx"].max()), **extra)
    torch.cuda.synchronize()
    assert torch.isnan(o[:, nq:].float()).all(), "wrote outside the heads"
    return o[:, :nq]


@pytest.mark.parametrize("fp8", [False, True])
def test_table_entries_outside_the_pool(fp8):
    """Block-table entries outside [0, num_pages) read as zeros (keys, values
    and, for fp8, scales) and never leave the pools.  Unused entries (past a
    sequence's pages) set to -1 and num_pages + k change nothing, bit for bit;
    used entries set out of range give the attention over a zero page."""
    require_gpu()
    H, Hk, hd = 8, 2, 128
    c = (_case_fp8 if fp8 else _case)(91, [70, 33, 5], [300, 0, 650], H, Hk, hd, spare=2)
    pages = c["kc"].shape[0]
    clean = np.where(c["bt"] < 0, 0, c["bt"])
    say(f"prefill_attention_paged fp8={fp8}: table entries outside the pool ({pages} pages), seed 91")
    ref = _run_table(c, clean, fp8)
    unused = c["bt"].copy()
    holes = np.argwhere(unused < 0)
    for n, (b, j) in enumerate(holes):
        unused[b, j] = -1 if n % 2 == 0 else pages + 1000 * n
    assert len(holes) > 0
    assert np.array_equal(bits(_run_table(c, unused, fp8)), bits(ref))

    # used entries out of range: sequence 0's page 3 -> -7, sequence 2's page 10 -> pages + 5
    bad = clean.copy()
    bad[0, 3] = -7
    bad[2, 10] = pages + 5
    got = _run_table(c, bad, fp8).float().cpu().numpy()
    assert np.all(np.isfinite(got))
    # expected: the same pools with one more, all-zero page that the bad entries point at
    zc = dict(c)
    zc["kc"] = np.concatenate([c["kc"], np.zeros_like(c["kc"][:1])])
    zc["vc"] = np.concatenate([c["vc"], np.zeros_like(c["vc"][:1])])
    if fp8:
        zc["ks"] = np.concatenate([c["ks"], np.zeros_like(c["ks"][:1])])
        zc["vs"] = np.concatenate([c["vs"], np.zeros_like(c["vs"][:1])])
    zbt = c["bt"].copy()
    zbt[0, 3] = pages
    zbt[2, 10] = pages
    zc["bt"] = zbt
    want = _oracle_fp8(zc) if fp8 else _oracle(zc)
    assert_close(got, want, f"paged {'fp8' if fp8 else 'bf16'} zero page")


def _oracle_window(c, window, kc, vc, ks=None, vs=None):
    """Each sequence's cached keys gathered through the table, then the
    window rule over key positions (oracle.prefix.window_causal_attention)."""
    qb = bits(c["q"]).reshape(-1, c["H"], c["hd"])
    cu, out = c["cu_q"], []
    for b in range(len(c["ctx"])):
        s0, s1, ctx = int(cu[b]), int(cu[b + 1]), int(c["ctx"][b])
        k, v = PX.cached_keys(kc, vc, c["bt"], b, ctx, ks, vs)
        out.append(PX.window_causal_attention(qb[s0:s1], k, v, window, prefix_len=ctx - (s1 - s0)))
    return np.concatenate(out)


@pytest.mark.parametrize("chunks,prefixes,H,Hk,hd,W", [
    ([37], [100], 4, 2, 128, 48),                 # window inside the chunk's own span for late rows
    ([129, 1, 50], [0, 300, 17], 8, 2, 128, 70),  # varlen, a 1-row chunk
    ([200], [333], 4, 4, 32, 1),                  # W = 1: each row its own value
    ([96, 40], [512, 1], 10, 2, 128, 300),        # G = 5, window reaching into the prefix
])
def test_window_over_pages_parity(chunks, prefixes, H, Hk, hd, W):
    """pca_prefill_attention_paged_window (bf16 pages) against the window rule
    over the gathered keys."""
    require_gpu()
    c = _case(81, chunks, prefixes, H, Hk, hd)
    say(f"prefill_attention_paged_window chunks={chunks} prefixes={prefixes} heads={H}/{Hk} hd={hd} W={W}")
    got = _gpu(c, window=W).float().cpu().numpy()
    assert_close(got, _oracle_window(c, W, c["kc"], c["vc"]), f"paged window W={W}")


def test_window_over_pages_wide_equals_plain_bitwise():
    """A window covering every key is exactly the paged call without one."""
    require_gpu()
    c = _case(82, [129, 50], [300, 17], 8, 2, 128)
    assert torch.equal(_gpu(c, window=100000), _gpu(c))


def test_window_over_fp8_pages_parity():
    """fp8 pages with a window: dequantised on load, against the oracle's
    decode of the same codes and scales."""
    require_gpu()
    c = _case_fp8(83, [96, 40], [512, 1], 10, 2, 128)
    W = 200
    T, nq = int(c["cu_q"][-1]), c["H"] * c["hd"]
    o = torch.full((T, nq), float("nan"), dtype=torch.bfloat16, device="cuda")
    d_bt = dev(torch.from_numpy(np.where(c["bt"] < 0, 0, c["bt"]).astype(np.int32)))
    pca.prefill_attention_paged(dev(c["q"]), o, dev(torch.from_numpy(c["kc"])), dev(torch.from_numpy(c["vc"])), d_bt,
                                dev(torch.from_numpy(c["ctx"])), c["H"], c["Hk"], c["hd"],
                                cu_seqlens=dev(torch.from_numpy(c["cu_q"])), max_seqlen=int(np.diff(c["cu_q"]).max()),
                                max_ctx=int(c["ctx"].max()), cache_dtype="fp8_e4m3", k_scale=dev(torch.from_numpy(c["ks"])),
                                v_scale=dev(torch.from_numpy(c["vs"])), window=W)
    torch.cuda.synchronize()
    want = _oracle_window(c, W, c["kc"], c["vc"], c["ks"], c["vs"])
    assert_close(o.float().cpu().numpy(), want, f"paged fp8 window W={W}")
