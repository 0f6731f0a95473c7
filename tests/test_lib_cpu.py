"""Host-only checks of libpca: it loads, exports every call include/pca.h
declares, kv_layout matches the oracle's accounting, and every compute call
rejects bad arguments before touching the device.  No GPU needed: the
argument checks run before any HIP call."""
import ctypes
import os
import re

import pytest

import prefill_causal_attention_amd as pca
from oracle import kvcache

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pca.h")

FAKE = 0x10000          # an aligned "device" address; never dereferenced by these calls
MISALIGNED = 0x10008


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:pca_status|const char\*|int64_t)\s+(pca_\w+)\s*\(", text, re.M)))


def test_library_loads_and_exports_header_symbols():
    lib = pca.load()
    names = _declared()
    assert set(names) >= {"pca_kv_layout", "pca_qkv_proj", "pca_prefill_attention", "pca_kv_cache_write",
                          "pca_last_error", "pca_version"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in pca.h but not exported"
    assert set(names) == set(pca.EXPORTED)
    assert pca.version().startswith("pca ")


@pytest.mark.parametrize("nh,nkv,hd,dtype", [(32, 32, 128, "bf16"), (32, 8, 128, "bf16"), (40, 8, 128, "fp8_e4m3"),
                                             (2, 2, 32, "bf16"), (8, 1, 64, "fp8_e4m3")])
def test_kv_layout_matches_oracle(nh, nkv, hd, dtype):
    got = pca.kv_layout(nh, nkv, hd, 16, dtype)
    want = kvcache.layout(nh, nkv, hd, 16, 1 if dtype == "fp8_e4m3" else 2)
    for k, v in want.items():
        assert got[k] == v, k
    assert got["page_size"] == 16 and got["elem_bytes"] == want["kv_bytes_per_token_layer"] // (2 * nkv * hd)


def test_kv_layout_page_figures(golden):
    for name, n_kv, hd, eb, layers, tokens, expected, _ in golden("kv_bytes_pages.txt"):
        if int(layers) == 1 and int(tokens) == 1:
            lay = pca.kv_layout(int(n_kv), int(n_kv), int(hd), 16, "bf16")
            assert lay["kv_bytes_per_token_layer"] == int(expected), name


@pytest.mark.parametrize("args", [(32, 7, 128), (0, 1, 128), (4, 0, 128), (4, 2, 0)])
def test_kv_layout_rejects(args):
    with pytest.raises(pca.PcaError) as e:
        pca.kv_layout(*args)
    assert e.value.status == 1


def _status(fn, *a):
    lib = pca.load()
    st = getattr(lib, fn)(*a)
    return st, lib.pca_last_error().decode()


def test_qkv_proj_validation():
    cases = [
        (0, 64, FAKE, 64, FAKE, 64, 4, 4, 64),            # null x
        (MISALIGNED, 64, FAKE, 64, FAKE, 64, 4, 4, 64),   # misaligned x
        (FAKE, 64, FAKE, 64, FAKE, 64, 0, 4, 64),         # M = 0
        (FAKE, 64, FAKE, 64, FAKE, 64, 4, 4, 60),         # K % 8
        (FAKE, 32, FAKE, 64, FAKE, 64, 4, 4, 64),         # ldx < K
        (FAKE, 64, FAKE, 64, FAKE, 2, 4, 4, 64),          # ldy < N
    ]
    for c in cases:
        st, msg = _status("pca_qkv_proj", *c, None)
        assert st == 1 and msg, c


def test_attention_validation():
    base = dict(q=FAKE, k=FAKE, v=FAKE, ldq=4096, ldk=1024, ldv=1024, cu=None, ns=1, mx=64, T=64,
                nh=32, nkv=8, hd=128, scale=0.088, causal=1, o=FAKE, ldo=4096)
    bad = [dict(nkv=7), dict(hd=96), dict(hd=256), dict(causal=0), dict(q=0), dict(o=MISALIGNED),
           dict(ldq=4000), dict(ldo=100), dict(ns=2), dict(scale=0.0), dict(scale=float("nan")),
           dict(mx=10), dict(T=-1)]
    want = {"hd": 2}
    for b in bad:
        a = dict(base, **b)
        st, msg = _status("pca_prefill_attention", a["q"], a["k"], a["v"], a["ldq"], a["ldk"], a["ldv"], a["cu"],
                          a["ns"], a["mx"], a["T"], a["nh"], a["nkv"], a["hd"], ctypes.c_float(a["scale"]),
                          a["causal"], a["o"], a["ldo"], None)
        exp = want.get(next(iter(b)), 1)
        assert st == exp and msg, (b, st, msg)


def test_attention_empty_batch_is_ok_without_buffers():
    st, _ = _status("pca_prefill_attention", None, None, None, 4096, 1024, 1024, None, 1, 0, 0, 32, 8, 128,
                    ctypes.c_float(0.088), 1, None, 4096, None)
    assert st == 0


def test_kv_write_validation():
    base = dict(k=FAKE, v=FAKE, ldk=1024, ldv=1024, cu=None, ns=1, T=64, bt=FAKE, mp=4, nkv=8, hd=128, ps=16,
                dt=0, kc=FAKE, vc=FAKE, ks=None, vs=None, np_=4)
    bad = {("ps", 32): 2, ("hd", 48): 2, ("dt", 5): 2, ("dt", 1): 1, ("ks", FAKE): 1, ("bt", 0): 1,
           ("kc", MISALIGNED): 1, ("ldk", 1000): 1, ("mp", 0): 1, ("np_", 0): 1, ("ns", 3): 1, ("nkv", 0): 1, ("np_", 1 << 27): 2}
    for (key, val), exp in bad.items():
        a = dict(base, **{key: val})
        st, msg = _status("pca_kv_cache_write", a["k"], a["v"], a["ldk"], a["ldv"], a["cu"], a["ns"], a["T"], a["bt"],
                          a["mp"], a["nkv"], a["hd"], a["ps"], a["dt"], a["kc"], a["vc"], a["ks"], a["vs"],
                          a["np_"], None)
        assert st == exp and msg, (key, val, st, msg)


def test_error_message_is_thread_local_and_cleared():
    st, msg = _status("pca_kv_cache_write", 0, 0, 0, 0, None, 1, 5, 0, 1, 1, 128, 16, 0, 0, 0, None, None, 1, None)
    assert st == 1 and "null" in msg
    pca.kv_layout(4, 2, 64)
    assert pca.load().pca_last_error().decode() == ""


def test_fused_kv_write_validation():
    # x, ldx, w_t, ldw, y, ldy, M, K, nh, nkv, hd, cu, ns, bt, mp, ps, dt, kc, vc, ks, vs, num_pages
    base = dict(x=FAKE, ldx=64, w=FAKE, ldw=64, y=FAKE, ldy=1536, M=64, K=64, nh=8, nkv=2, hd=128, cu=None, ns=1,
                bt=FAKE, mp=4, ps=16, dt=0, kc=FAKE, vc=FAKE, ks=None, vs=None, np_=4)
    bad = {("x", 0): 1, ("y", MISALIGNED): 1, ("K", 60): 1, ("ldy", 1000): 1, ("nkv", 3): 1, ("hd", 96): 2,
           ("ps", 8): 2, ("bt", 0): 1, ("kc", 0): 1, ("dt", 1): 1, ("ks", FAKE): 1, ("ns", 2): 1, ("np_", 0): 1,
           ("dt", 7): 2}
    for (key, val), exp in bad.items():
        a = dict(base, **{key: val})
        st, msg = _status("pca_qkv_proj_kv_write", a["x"], a["ldx"], a["w"], a["ldw"], a["y"], a["ldy"], a["M"],
                          a["K"], a["nh"], a["nkv"], a["hd"], a["cu"], a["ns"], a["bt"], a["mp"], a["ps"], a["dt"],
                          a["kc"], a["vc"], a["ks"], a["vs"], a["np_"], None)
        assert st == exp and msg, (key, val, st, msg)
    # fp8 needs K and V column blocks that start and span multiples of 128 columns
    a = dict(base, nh=3, nkv=1, hd=64, ldy=320, dt=1, ks=FAKE, vs=FAKE)
    st, msg = _status("pca_qkv_proj_kv_write", a["x"], a["ldx"], a["w"], a["ldw"], a["y"], a["ldy"], a["M"],
                      a["K"], a["nh"], a["nkv"], a["hd"], a["cu"], a["ns"], a["bt"], a["mp"], a["ps"], a["dt"],
                      a["kc"], a["vc"], a["ks"], a["vs"], a["np_"], None)
    assert st == 2 and "128" in msg, (st, msg)


def test_e4m3_encode_validation():
    assert _status("pca_e4m3_encode", None, None, 0, None)[0] == 0          # empty: no-op, no buffers needed
    for c in [(FAKE, FAKE, -1), (0, FAKE, 8), (FAKE, 0, 8), (MISALIGNED, FAKE, 8), (FAKE, FAKE + 2, 8)]:
        st, msg = _status("pca_e4m3_encode", *c, None)
        assert st == 1 and msg, c


def test_quantize_heads_fp8_validation():
    # x, ldx, T, H, hd, prescale, codes, ldc, exps, lde
    base = dict(x=FAKE, ldx=1024, T=4, H=8, hd=128, ps=1.0, c=FAKE, ldc=1024, e=FAKE, lde=8)
    assert _status("pca_quantize_heads_fp8", None, 1024, 0, 8, 128, ctypes.c_float(1.0), None, 1024, None, 8,
                   None)[0] == 0                                         # T == 0: no-op
    bad = {("x", 0): 1, ("x", MISALIGNED): 1, ("c", FAKE + 4): 1, ("hd", 96): 2, ("H", 0): 1, ("ldx", 1000): 1,
           ("ldc", 1016): 1, ("lde", 7): 1, ("ps", 0.0): 1, ("ps", float("inf")): 1, ("ps", float("nan")): 1,
           ("T", -1): 1}
    for (key, val), exp in bad.items():
        a = dict(base, **{key: val})
        st, msg = _status("pca_quantize_heads_fp8", a["x"], a["ldx"], a["T"], a["H"], a["hd"], ctypes.c_float(a["ps"]),
                          a["c"], a["ldc"], a["e"], a["lde"], None)
        assert st == exp and msg, (key, val, st, msg)


def test_fp8qk_attention_validation():
    base = dict(q=FAKE, ldq=4096, k=FAKE, ldk=1024, e=FAKE, lde=8, v=FAKE, ldv=1024, cu=None, ns=1, mx=64, T=64,
                nh=32, nkv=8, hd=128, scale=0.088, causal=1, o=FAKE, ldo=4096)
    bad = {("hd", 64): 2, ("nkv", 7): 1, ("causal", 0): 1, ("k", 0): 1, ("e", FAKE + 2): 1, ("ldk", 1032): 1,
           ("lde", 6): 1, ("lde", 10): 1, ("ldq", 4000): 1, ("scale", 0.0): 1, ("mx", 10): 1, ("v", MISALIGNED): 1}
    for (key, val), exp in bad.items():
        a = dict(base, **{key: val})
        st, msg = _status("pca_prefill_attention_fp8qk", a["q"], a["ldq"], a["k"], a["ldk"], a["e"], a["lde"], a["v"],
                          a["ldv"], a["cu"], a["ns"], a["mx"], a["T"], a["nh"], a["nkv"], a["hd"],
                          ctypes.c_float(a["scale"]), a["causal"], a["o"], a["ldo"], None)
        assert st == exp and msg, (key, val, st, msg)
    st, _ = _status("pca_prefill_attention_fp8qk", None, 4096, None, 1024, None, 8, None, 1024, None, 1, 0, 0, 32, 8,
                    128, ctypes.c_float(0.088), 1, None, 4096, None)
    assert st == 0                                                       # empty batch


def test_gemm_grids_too_large_for_one_launch_rejected():
    """M x N whose tile count exceeds int32 is refused before any launch (the
    product and the fp8 product), not wrapped into a wrong grid."""
    big = 1 << 30
    st, msg = _status("pca_qkv_proj", FAKE, 64, FAKE, 64, FAKE, big, big, big, 64, None)
    assert st == 2 and "too large" in msg, (st, msg)
    lib = pca.load()
    st = lib.pca_qkv_proj_fp8(FAKE, 64, FAKE, FAKE, 64, FAKE, FAKE, big, big, big, 64, None)
    msg = lib.pca_last_error().decode()
    assert st == 2 and "too large" in msg, (st, msg)
