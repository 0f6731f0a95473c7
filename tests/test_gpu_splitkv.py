"""GPU parity of pca_prefill_attention_splitkv (key ranges of long query
blocks split over two workgroups on shallow grids) against the fp64 oracle;
its determinism across calls that reuse one workspace (the arrival counters
must come back to zero); and its fallback on deep grids, which is bitwise
pca_prefill_attention."""
import numpy as np
import pytest
import torch

import prefill_causal_attention_amd as pca
import workloads
from oracle import attention as A

from _gpu_helpers import assert_close, bits, dev, require_gpu, sample_rows, say

pytestmark = pytest.mark.gpu


def _workspace(w):
    n = pca.prefill_attention_splitkv_workspace(w.num_seqs, w.max_seqlen, w.n_head, w.n_kv_head, w.head_dim)
    return torch.zeros(n, dtype=torch.uint8, device="cuda")     # zeroed once, as the header asks


def _run(w, d_buf, ws=None):
    nq, nk = w.n_head * w.head_dim, w.n_kv_head * w.head_dim
    q, k, v = d_buf[:, :nq], d_buf[:, nq:nq + nk], d_buf[:, nq + nk:nq + 2 * nk]
    o = torch.full((w.total_tokens, nq), float("nan"), dtype=torch.bfloat16, device="cuda")
    cu = dev(torch.from_numpy(workloads.cu_seqlens(w))) if w.num_seqs > 1 else None
    if ws is None:
        pca.prefill_attention(q, k, v, o, w.n_head, w.n_kv_head, w.head_dim, cu_seqlens=cu, max_seqlen=w.max_seqlen)
    else:
        pca.prefill_attention_splitkv(q, k, v, o, ws, w.n_head, w.n_kv_head, w.head_dim, cu_seqlens=cu,
                                      max_seqlen=w.max_seqlen)
    torch.cuda.synchronize()
    return o


# shallow grids (at most one task group per workgroup slot, units a multiple of
# 8, at least 8 kv tiles in the longest sequence): the split is active
SHALLOW = [
    ([600], 8, 8, 64),                 # task groups of 4, 8 and 10 tiles: whole, split 4+4, split 5+5
    ([777], 8, 8, 32),
    ([1000], 16, 8, 128),              # G = 2
    ([500, 300, 129], 16, 8, 128),     # varlen: 24 units, the short sequence never split
    ([1024], 32, 32, 64),
]


@pytest.mark.parametrize("lens,H,Hk,hd", SHALLOW)
def test_parity_small(lens, H, Hk, hd):
    require_gpu()
    w = workloads.custom(57, lens, H, Hk, hd)
    buf, *_ = workloads.qkv_inputs(w)
    say(f"splitkv lens={lens} heads={H}/{Hk} hd={hd} T={w.total_tokens}")
    d_buf = dev(buf)
    ws = _workspace(w)
    got = _run(w, d_buf, ws)
    plain = _run(w, d_buf)
    q, k, v = A.head_split(bits(buf), H, Hk, hd)
    want = A.varlen_causal_attention(q, k, v, workloads.cu_seqlens(w))
    assert_close(got.float().cpu().numpy().astype(np.float64), want, f"splitkv {lens}")
    # the split rows sum their keys in another order than the one-pass kernel
    assert not torch.equal(got, plain), "no row was split (the split path did not run)"
    d = (got.float() - plain.float()).abs().max().item()
    say(f"  split against one-pass kernel: max_abs={d:.3e}")
    assert d <= 2e-2


@pytest.mark.parametrize("H,Hk", [(32, 32), (32, 8)])
def test_parity_s2048_sampled_rows(H, Hk):
    """The 2048-token shapes the split is for: one sequence, MHA and GQA."""
    require_gpu()
    w = workloads.custom(58, [2048], H, Hk, 128)
    buf, *_ = workloads.qkv_inputs(w)
    say(f"splitkv s=2048 heads={H}/{Hk}")
    got = _run(w, dev(buf), _workspace(w))
    rows = sample_rows(2048, 96, 7)
    q, k, v = A.head_split(bits(buf), H, Hk, 128)
    want = A.varlen_causal_attention(q, k, v, workloads.cu_seqlens(w), rows=rows)
    assert_close(got.float().cpu().numpy().astype(np.float64)[rows], want, f"splitkv s=2048 {H}/{Hk}")


def test_deterministic_and_workspace_reuse():
    """Repeated calls on one workspace give the same bits (a counter left
    non-zero would make both chunks merge, or neither), also after a call of
    another shape on the same workspace."""
    require_gpu()
    wa = workloads.custom(59, [2048], 32, 32, 128)
    wb = workloads.custom(60, [500, 300, 129], 16, 8, 128)
    ba, *_ = workloads.qkv_inputs(wa)
    bb, *_ = workloads.qkv_inputs(wb)
    da, db = dev(ba), dev(bb)
    n = max(_workspace(wa).numel(), _workspace(wb).numel())
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    say("splitkv determinism: s=2048 MHA, a varlen batch, s=2048 again")
    first = _run(wa, da, ws)
    other = _run(wb, db, ws)
    again = _run(wa, da, ws)
    assert torch.equal(first, again)
    assert torch.equal(other, _run(wb, db, ws))
    # every arrival counter (the workspace's first 4 KiB) is back at zero
    assert int(ws[:4096].view(torch.int32).abs().sum().item()) == 0, "arrival counters not reset"


def test_deep_grid_falls_back_bitwise():
    """More task groups than workgroup slots: the one-pass kernel runs."""
    require_gpu()
    w = workloads.custom(61, [8192], 32, 8, 128)
    buf, *_ = workloads.qkv_inputs(w)
    d_buf = dev(buf)
    say("splitkv fallback s=8192 GQA")
    assert torch.equal(_run(w, d_buf, _workspace(w)), _run(w, d_buf))


def test_short_sequence_falls_back_bitwise():
    """Fewer than 8 kv tiles: nothing is worth splitting."""
    require_gpu()
    w = workloads.custom(62, [300], 8, 8, 128)
    buf, *_ = workloads.qkv_inputs(w)
    d_buf = dev(buf)
    assert torch.equal(_run(w, d_buf, _workspace(w)), _run(w, d_buf))


@pytest.mark.parametrize("lens,H,Hk,hd", [([1024], 32, 8, 64), ([700, 700], 8, 4, 128)])
def test_parity_more_shapes(lens, H, Hk, hd):
    """GQA G = 4 at hd 64; and two sequences of 4 kv heads, 8 units on the
    8 XCDs."""
    require_gpu()
    w = workloads.custom(64, lens, H, Hk, hd)
    buf, *_ = workloads.qkv_inputs(w)
    say(f"splitkv lens={lens} heads={H}/{Hk} hd={hd}")
    d_buf = dev(buf)
    got = _run(w, d_buf, _workspace(w))
    assert not torch.equal(got, _run(w, d_buf)), "no row was split (the split path did not run)"
    q, k, v = A.head_split(bits(buf), H, Hk, hd)
    want = A.varlen_causal_attention(q, k, v, workloads.cu_seqlens(w))
    assert_close(got.float().cpu().numpy().astype(np.float64), want, f"splitkv {lens} {H}/{Hk} hd{hd}")


def test_units_off_the_xcd_count_fall_back_bitwise():
    """4 units (one sequence, 4 kv heads) do not spread evenly over the 8
    XCDs: the one-pass kernel runs."""
    require_gpu()
    w = workloads.custom(65, [1024], 16, 4, 128)
    buf, *_ = workloads.qkv_inputs(w)
    d_buf = dev(buf)
    assert torch.equal(_run(w, d_buf, _workspace(w)), _run(w, d_buf))


def test_workspace_errors():
    require_gpu()
    w = workloads.custom(63, [2048], 32, 32, 128)
    buf, *_ = workloads.qkv_inputs(w)
    d_buf = dev(buf)
    small = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(pca.PcaError, match="needed"):
        _run(w, d_buf, small)
    big = torch.zeros(_workspace(w).numel() + 512, dtype=torch.uint8, device="cuda")
    with pytest.raises(pca.PcaError, match="aligned"):
        _run(w, d_buf, big[64:])
