"""Host-side argument checks of the calls not covered in test_lib_cpu.py, and
the binding's refusal of host tensors and wrong element types.

Every case here must come back with a non-OK status and a message before any
HIP call: there is no GPU in the CPU test run, so a case that slipped past the
checks would reach the launch and return PCA_ERR_HIP (3) instead of the
expected code.  FAKE addresses are never dereferenced."""
import ctypes

import pytest
import torch

import prefill_causal_attention_amd as pca

FAKE = 0x10000
MISALIGNED = 0x10008
C = ctypes.c_float


def _status(fn, *a):
    lib = pca.load()
    st = getattr(lib, fn)(*a)
    return st, lib.pca_last_error().decode()


def _expect(fn, base, order, bad, wrap=None):
    """Call fn with base updated by each bad entry; assert the status code."""
    for (key, val), exp in bad.items():
        a = dict(base, **{key: val})
        args = [wrap[k](a[k]) if wrap and k in wrap else a[k] for k in order]
        st, msg = _status(fn, *args, None)
        assert st == exp and msg, (fn, key, val, st, msg)


PAGED_ORDER = ["q", "ldq", "cu", "ns", "mxq", "T", "ctx", "mxc", "bt", "mp", "ps", "dt", "kc", "vc", "ks", "vs",
               "np_", "nh", "nkv", "hd", "scale", "causal", "o", "ldo"]
PAGED_BASE = dict(q=FAKE, ldq=4096, cu=None, ns=1, mxq=512, T=512, ctx=FAKE, mxc=1024, bt=FAKE, mp=64, ps=16, dt=0,
                  kc=FAKE, vc=FAKE, ks=None, vs=None, np_=64, nh=32, nkv=8, hd=128, scale=0.088, causal=1, o=FAKE,
                  ldo=4096)


def test_paged_attention_validation():
    bad = {("q", 0): 1, ("o", 0): 1, ("kc", 0): 1, ("vc", 0): 1, ("bt", 0): 1, ("ctx", 0): 1,
           ("q", MISALIGNED): 1, ("kc", MISALIGNED): 1, ("bt", FAKE + 2): 1, ("ctx", FAKE + 1): 1,
           ("causal", 0): 1, ("nkv", 7): 1, ("nh", 0): 1, ("hd", 96): 2, ("ps", 32): 2, ("dt", 3): 2,
           ("ks", FAKE): 1,                                  # scales given for a bf16 cache
           ("ns", 2): 1,                                     # several sequences need cu_seqlens_q
           ("scale", 0.0): 1, ("scale", float("nan")): 1, ("ldq", 4000): 1, ("ldo", 100): 1, ("mp", 0): 1,
           ("np_", 0): 1, ("mxq", 100): 1,                   # max_seqlen_q below the single chunk
           ("mxc", 256): 1,                                  # max_ctx_len below max_seqlen_q
           ("mxc", 64 * 16 + 1): 1,                          # max_ctx_len past the block-table row
           ("np_", 1 << 20): 2}                              # pools of 2 GiB or more
    _expect("pca_prefill_attention_paged", PAGED_BASE, PAGED_ORDER, bad, {"scale": C})
    # fp8 pools need both scale pools, 4-byte aligned
    f8 = dict(PAGED_BASE, dt=1, ks=FAKE, vs=FAKE)
    _expect("pca_prefill_attention_paged", f8, PAGED_ORDER, {("ks", None): 1, ("vs", FAKE + 2): 1}, {"scale": C})
    # an empty chunk batch is a no-op that needs no buffers
    a = dict(PAGED_BASE, T=0, q=None, o=None, kc=None, vc=None, bt=None, ctx=None)
    st, _ = _status("pca_prefill_attention_paged", *[C(a[k]) if k == "scale" else a[k] for k in PAGED_ORDER], None)
    assert st == 0


def test_paged_window_attention_validation():
    """The windowed call checks its window, then everything the paged call checks."""
    order = PAGED_ORDER[:-2] + ["win"] + PAGED_ORDER[-2:]
    base = dict(PAGED_BASE, win=64)
    bad = {("win", -1): 1, ("win", -(1 << 30)): 1, ("q", 0): 1, ("causal", 0): 1, ("hd", 96): 2, ("ps", 32): 2,
           ("ks", FAKE): 1, ("mxc", 256): 1, ("scale", 0.0): 1}
    _expect("pca_prefill_attention_paged_window", base, order, bad, {"scale": C})
    # an empty chunk batch is a no-op that needs no buffers; a negative window is still refused
    a = dict(base, T=0, q=None, o=None, kc=None, vc=None, bt=None, ctx=None)
    st, _ = _status("pca_prefill_attention_paged_window", *[C(a[k]) if k == "scale" else a[k] for k in order], None)
    assert st == 0
    a["win"] = -5
    st, msg = _status("pca_prefill_attention_paged_window", *[C(a[k]) if k == "scale" else a[k] for k in order], None)
    assert st == 1 and "window" in msg


WIN_ORDER = ["q", "k", "v", "ldq", "ldk", "ldv", "cu", "ns", "mx", "T", "nh", "nkv", "hd", "scale", "causal", "win",
             "o", "ldo"]
WIN_BASE = dict(q=FAKE, k=FAKE, v=FAKE, ldq=4096, ldk=1024, ldv=1024, cu=None, ns=1, mx=64, T=64, nh=32, nkv=8, hd=128,
                scale=0.088, causal=1, win=16, o=FAKE, ldo=4096)


def test_window_attention_validation():
    bad = {("win", -1): 1, ("win", -(1 << 30)): 1, ("q", 0): 1, ("v", MISALIGNED): 1, ("causal", 0): 1,
           ("nkv", 5): 1, ("hd", 48): 2, ("ldk", 1000): 1, ("mx", 10): 1, ("T", -3): 1, ("ns", 0): 1,
           ("cu", FAKE + 2): 1, ("scale", float("inf")): 1}
    _expect("pca_prefill_attention_window", WIN_BASE, WIN_ORDER, bad, {"scale": C})


SPLIT_ORDER = WIN_ORDER[:15] + ["o", "ldo", "ws", "wsb"]


def _split_ws(ns, mx, nh, nkv, hd):
    return pca.load().pca_prefill_attention_splitkv_workspace(ns, mx, nh, nkv, hd)


def test_splitkv_workspace_size():
    """4 KiB of counters, then two chunks x 8 waves x 64 lanes x (hd/2 + 2)
    floats per task-group slot, slots = sequences x kv heads x
    ceil(G * ceil(L / 32) / 8), at most 1024."""
    def want(ns, mx, nh, nkv, hd):
        g = nh // nkv
        slots = min(1024, ns * nkv * -(-(g * -(-mx // 32)) // 8))
        return 4096 + slots * 2 * 8 * 64 * (hd // 2 + 2) * 4
    for args in [(1, 2048, 32, 32, 128), (1, 2048, 32, 8, 128), (3, 500, 16, 8, 128), (1, 600, 8, 8, 64),
                 (1, 777, 8, 8, 32), (1, 1, 2, 1, 32), (1, 8192, 32, 8, 128), (1, 32768, 40, 8, 128)]:
        assert _split_ws(*args) == want(*args), args
    assert _split_ws(1, 2048, 32, 32, 128) == 4096 + 256 * 270336         # 264 KiB per slot at hd 128
    assert _split_ws(1, 32768, 40, 8, 128) == 4096 + 1024 * 270336         # capped: never split
    for bad in [(0, 2048, 32, 8, 128), (1, 0, 32, 8, 128), (1, 2048, 30, 8, 128), (1, 2048, 32, 8, 96),
                (1, 2048, 0, 8, 128), (1, 2048, 32, 0, 128)]:
        assert _split_ws(*bad) == -1 and pca.load().pca_last_error(), bad


def test_splitkv_validation():
    need = _split_ws(1, 64, 32, 8, 128)
    base = dict(WIN_BASE, ws=FAKE, wsb=need)
    bad = {("ws", None): 1, ("ws", FAKE + 64): 1, ("wsb", need - 1): 1, ("wsb", -1): 1, ("wsb", 0): 1,
           ("q", 0): 1, ("causal", 0): 1, ("nkv", 5): 1, ("hd", 48): 2, ("mx", 10): 1, ("ns", 0): 1,
           ("scale", float("nan")): 1}
    _expect("pca_prefill_attention_splitkv", base, SPLIT_ORDER, bad, {"scale": C})


GEMM_ORDER = ["x", "ldx", "w", "ldw", "y", "ldy", "M", "N", "K"]
GEMM_BAD = {("x", 0): 1, ("w", 0): 1, ("y", 0): 1, ("x", MISALIGNED): 1, ("M", 0): 1, ("N", 0): 1, ("K", 4): 1,
            ("K", 68): 1, ("ldx", 32): 1, ("ldw", 60): 1, ("ldy", 100): 1, ("M", 1 << 31): 1,
            ("ldx", 1 << 22): 2}                            # a 256-row tile view past 2 GiB


def test_out_proj_residual_validation():
    order = ["x", "ldx", "w", "ldw", "res", "ldr", "y", "ldy", "M", "N", "K"]
    base = dict(x=FAKE, ldx=64, w=FAKE, ldw=64, res=0x200000, ldr=128, y=0x400000, ldy=128, M=16, N=128, K=64)
    bad = dict(GEMM_BAD)
    bad.update({("res", 0): 1, ("res", 0x200008): 1, ("ldr", 120): 1, ("ldr", 132): 1,
                ("res", 0x400000 + 256): 1,                 # partly overlaps out without being out
                ("res", 0x400000 - 256): 1})
    _expect("pca_out_proj_residual", base, order, bad)
    # in place: res == out needs ldr == ldout
    _expect("pca_out_proj_residual", dict(base, res=0x400000), order, {("ldr", 136): 1})


def test_rms_norm_qkv_proj_validation():
    order = ["x", "ldx", "w", "ldw", "eps", "inv", "y", "ldy", "M", "N", "K"]
    base = dict(x=FAKE, ldx=64, w=FAKE, ldw=64, eps=1e-6, inv=FAKE, y=FAKE, ldy=128, M=16, N=128, K=64)
    bad = dict(GEMM_BAD)
    bad.update({("inv", 0): 1, ("inv", FAKE + 2): 1, ("eps", -1e-6): 1, ("eps", float("nan")): 1,
                ("eps", float("inf")): 1})
    _expect("pca_rms_norm_qkv_proj", base, order, bad, {"eps": C})


def test_rms_norm_qkv_proj_noalloc_validation():
    """Same checks as the workspace call (before any HIP call), plus the row
    limit of the static workspace."""
    order = ["x", "ldx", "w", "ldw", "eps", "y", "ldy", "M", "N", "K"]
    base = dict(x=FAKE, ldx=64, w=FAKE, ldw=64, eps=1e-6, y=FAKE, ldy=128, M=16, N=128, K=64)
    bad = dict(GEMM_BAD)
    bad.update({("eps", -1.0): 1, ("eps", float("nan")): 1, ("M", pca.NOALLOC_MAX_ROWS + 1): 2})
    _expect("pca_rms_norm_qkv_proj_noalloc", base, order, bad, {"eps": C})


def test_noalloc_row_limit_matches_header():
    import os
    import re
    text = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pca.h")).read()
    assert int(re.search(r"#define PCA_NOALLOC_MAX_ROWS (\d+)", text).group(1)) == pca.NOALLOC_MAX_ROWS


def test_clock_stamp_validation():
    for ptr in (0, FAKE + 4):
        st, msg = _status("pca_clock_stamp", ptr, None)
        assert st == 1 and msg, ptr


def test_qkv_proj_fp8_validation():
    order = ["xq", "ldxq", "sx", "wq", "ldwq", "sw", "y", "ldy", "M", "N", "K"]
    base = dict(xq=FAKE, ldxq=64, sx=FAKE, wq=FAKE, ldwq=64, sw=FAKE, y=FAKE, ldy=128, M=16, N=128, K=64)
    bad = {("xq", 0): 1, ("sx", 0): 1, ("wq", 0): 1, ("sw", 0): 1, ("y", 0): 1, ("xq", MISALIGNED): 1,
           ("wq", FAKE + 4): 1, ("y", MISALIGNED): 1, ("sx", FAKE + 2): 1, ("sw", FAKE + 1): 1, ("M", 0): 1,
           ("N", -1): 1, ("K", 8): 1, ("K", 72): 1, ("ldxq", 56): 1, ("ldxq", 72): 1, ("ldwq", 80 + 8): 1,
           ("ldy", 120): 1, ("ldy", 132): 1, ("ldxq", 1 << 23): 2}
    _expect("pca_qkv_proj_fp8", base, order, bad)


def test_quantize_rows_fp8_validation():
    order = ["x", "ldx", "M", "K", "q", "ldq", "s"]
    base = dict(x=FAKE, ldx=64, M=16, K=64, q=FAKE, ldq=64, s=FAKE)
    bad = {("x", 0): 1, ("q", 0): 1, ("s", 0): 1, ("x", MISALIGNED): 1, ("q", FAKE + 4): 1, ("s", FAKE + 2): 1,
           ("M", 0): 1, ("K", 0): 1, ("K", 8): 1, ("K", 40): 1, ("ldx", 60): 1, ("ldx", 68): 1, ("ldq", 56): 1,
           ("ldq", 72): 1, ("M", 1 << 31): 1}
    _expect("pca_quantize_rows_fp8", base, order, bad)


# ---- the Python binding: host tensors and wrong element types never reach a kernel

def _cpu(shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def test_binding_rejects_host_tensors():
    x, w, y = _cpu((16, 64)), _cpu((128, 64)), _cpu((16, 128))
    with pytest.raises(ValueError, match="device tensor"):
        pca.qkv_proj(x, w, y)
    q, k, v, o = _cpu((64, 256)), _cpu((64, 128)), _cpu((64, 128)), _cpu((64, 256))
    with pytest.raises(ValueError, match="device tensor"):
        pca.prefill_attention(q, k, v, o, 2, 1, 128)
    bt = torch.zeros((1, 4), dtype=torch.int32)
    kc = _cpu((4, 16, 1, 128))
    with pytest.raises(ValueError, match="device tensor"):
        pca.kv_cache_write(k, v, bt, kc, kc.clone(), 1, 128)
    with pytest.raises(ValueError, match="device tensor"):
        pca.e4m3_encode(torch.zeros(64), torch.zeros(64, dtype=torch.uint8))
    with pytest.raises(ValueError, match="device tensor"):
        pca.quantize_rows_fp8(x, torch.zeros((16, 64), dtype=torch.uint8), torch.zeros(16))
    with pytest.raises(TypeError):
        pca.qkv_proj([1, 2], w, y)


def test_binding_rejects_wrong_dtypes(monkeypatch):
    # make every tensor look device-resident so the dtype check is what fires
    monkeypatch.setattr(torch.Tensor, "is_cuda", property(lambda self: True))
    x, w = _cpu((16, 64)), _cpu((128, 64))
    with pytest.raises(ValueError, match="dtype"):
        pca.qkv_proj(x, w, _cpu((16, 128), torch.float32))
    with pytest.raises(ValueError, match="dtype"):
        pca.qkv_proj(x.to(torch.float16), w, _cpu((16, 128)))
    q, kv, o = _cpu((64, 256)), _cpu((64, 128)), _cpu((64, 256))
    with pytest.raises(ValueError, match="dtype"):
        pca.prefill_attention(q, kv, kv, o, 2, 1, 128, cu_seqlens=torch.tensor([0, 64], dtype=torch.int64))
    bt = torch.zeros((1, 4), dtype=torch.int32)
    with pytest.raises(ValueError, match="dtype"):
        pca.kv_cache_write(kv, kv, bt.to(torch.int64), _cpu((4, 16, 1, 128)), _cpu((4, 16, 1, 128)), 1, 128)
    with pytest.raises(ValueError, match="dtype"):       # fp8 pools are uint8 codes
        pca.kv_cache_write(kv, kv, bt, _cpu((4, 16, 1, 128)), _cpu((4, 16, 1, 128)), 1, 128, cache_dtype="fp8_e4m3",
                           k_scale=torch.zeros((4, 16, 1)), v_scale=torch.zeros((4, 16, 1)))
    u8 = torch.zeros((4, 16, 1, 128), dtype=torch.uint8)
    with pytest.raises(ValueError, match="dtype"):       # scales are float32
        pca.kv_cache_write(kv, kv, bt, u8, u8.clone(), 1, 128, cache_dtype="fp8_e4m3",
                           k_scale=torch.zeros((4, 16, 1), dtype=torch.float64), v_scale=torch.zeros((4, 16, 1)))
    with pytest.raises(ValueError, match="dtype"):
        pca.e4m3_encode(torch.zeros(64, dtype=torch.float64), torch.zeros(64, dtype=torch.uint8))
    with pytest.raises(ValueError, match="dtype"):
        pca.prefill_attention_paged(q, o, _cpu((4, 16, 1, 128)), _cpu((4, 16, 1, 128)), bt,
                                    torch.tensor([64], dtype=torch.int64), 2, 1, 128, max_ctx=64)
    with pytest.raises(ValueError, match="unknown cache dtype"):
        pca.kv_cache_write(kv, kv, bt, u8, u8.clone(), 1, 128, cache_dtype="fp16")
