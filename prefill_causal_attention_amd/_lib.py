"""ctypes binding of libpca (argument marshalling only).

Every step of the path runs in the HIP kernels of libpca.so; this module only
turns torch tensors into device pointers, strides and the current HIP stream.
There is no fallback: if the library is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpca.so")

PCA_OK, PCA_ERR_INVALID_ARG, PCA_ERR_UNSUPPORTED, PCA_ERR_HIP = 0, 1, 2, 3
DTYPES = {"bf16": 0, "fp8_e4m3": 1}

NOALLOC_MAX_ROWS = 262144      # PCA_NOALLOC_MAX_ROWS of include/pca.h

EXPORTED = ("pca_kv_layout", "pca_qkv_proj", "pca_qkv_proj_kv_write", "pca_rms_norm_qkv_proj",
            "pca_rms_norm_qkv_proj_noalloc", "pca_out_proj_residual",
            "pca_quantize_rows_fp8", "pca_qkv_proj_fp8", "pca_e4m3_encode",
            "pca_quantize_heads_fp8", "pca_prefill_attention_fp8qk",
            "pca_prefill_attention",
            "pca_prefill_attention_window", "pca_prefill_attention_splitkv",
            "pca_prefill_attention_splitkv_workspace", "pca_prefill_attention_paged",
            "pca_prefill_attention_paged_window", "pca_kv_cache_write",
            "pca_clock_stamp", "pca_last_error", "pca_version")


class PcaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed (status {status}): {msg}")
        self.status = status


class KvLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "qkv_ld", "q_off", "k_off", "v_off", "head_stride", "page_size", "pool_page_stride",
        "pool_slot_stride", "pool_head_stride", "scale_page_stride", "scale_slot_stride",
        "elem_bytes", "kv_bytes_per_token_layer", "scale_bytes_per_token_layer", "page_bytes")]

    def as_dict(self) -> dict:
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpca.so (built in-tree by __graft_entry__.build()); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is not built: run __graft_entry__.build() (hipcc for gfx950)")
    lib = ctypes.CDLL(path)
    i64, i32, vp, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float
    lib.pca_kv_layout.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(KvLayout)]
    lib.pca_qkv_proj.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, i64, vp]
    lib.pca_prefill_attention.argtypes = [vp, vp, vp, i64, i64, i64, vp, i32, i32, i64, i32, i32, i32,
                                          f32, i32, vp, i64, vp]
    lib.pca_kv_cache_write.argtypes = [vp, vp, i64, i64, vp, i32, i64, vp, i32, i32, i32, i32, i32,
                                       vp, vp, vp, vp, i64, vp]
    lib.pca_qkv_proj_kv_write.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, i32, i32, i32, vp, i32,
                                          vp, i32, i32, i32, vp, vp, vp, vp, i64, vp]
    lib.pca_quantize_rows_fp8.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp]
    lib.pca_e4m3_encode.argtypes = [vp, vp, i64, vp]
    lib.pca_quantize_heads_fp8.argtypes = [vp, i64, i64, i32, i32, f32, vp, i64, vp, i64, vp]
    lib.pca_prefill_attention_fp8qk.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, vp, i32, i32, i64, i32, i32, i32,
                                                f32, i32, vp, i64, vp]
    lib.pca_qkv_proj_fp8.argtypes = [vp, i64, vp, vp, i64, vp, vp, i64, i64, i64, i64, vp]
    lib.pca_rms_norm_qkv_proj.argtypes = [vp, i64, vp, i64, f32, vp, vp, i64, i64, i64, i64, vp]
    lib.pca_rms_norm_qkv_proj_noalloc.argtypes = [vp, i64, vp, i64, f32, vp, i64, i64, i64, i64, vp]
    lib.pca_out_proj_residual.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, i64, i64, i64, vp]
    lib.pca_prefill_attention_window.argtypes = [vp, vp, vp, i64, i64, i64, vp, i32, i32, i64, i32, i32, i32,
                                                 f32, i32, i32, vp, i64, vp]
    lib.pca_prefill_attention_splitkv.argtypes = [vp, vp, vp, i64, i64, i64, vp, i32, i32, i64, i32, i32, i32,
                                                  f32, i32, vp, i64, vp, i64, vp]
    lib.pca_prefill_attention_splitkv_workspace.argtypes = [i32, i32, i32, i32, i32]
    lib.pca_prefill_attention_splitkv_workspace.restype = ctypes.c_int64
    lib.pca_prefill_attention_paged.argtypes = [vp, i64, vp, i32, i32, i64, vp, i32, vp, i32, i32, i32, vp, vp,
                                                vp, vp, i64, i32, i32, i32, f32, i32, vp, i64, vp]
    lib.pca_prefill_attention_paged_window.argtypes = [vp, i64, vp, i32, i32, i64, vp, i32, vp, i32, i32, i32, vp,
                                                       vp, vp, vp, i64, i32, i32, i32, f32, i32, i32, vp, i64, vp]
    for fn in ("pca_kv_layout", "pca_qkv_proj", "pca_prefill_attention", "pca_kv_cache_write",
               "pca_qkv_proj_kv_write", "pca_prefill_attention_paged", "pca_prefill_attention_paged_window",
               "pca_prefill_attention_window",
               "pca_prefill_attention_splitkv",
               "pca_out_proj_residual", "pca_rms_norm_qkv_proj", "pca_rms_norm_qkv_proj_noalloc",
               "pca_quantize_rows_fp8", "pca_qkv_proj_fp8",
               "pca_e4m3_encode", "pca_quantize_heads_fp8", "pca_prefill_attention_fp8qk"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.pca_clock_stamp.argtypes = [vp, vp]
    lib.pca_clock_stamp.restype = ctypes.c_int
    lib.pca_last_error.restype = ctypes.c_char_p
    lib.pca_last_error.argtypes = []
    lib.pca_version.restype = ctypes.c_char_p
    lib.pca_version.argtypes = []
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != PCA_OK:
        raise PcaError(fn, status, load().pca_last_error().decode())


_DT = {}


def _dtype(kind: str):
    """torch dtype of an argument kind (torch is imported lazily: the host-only
    calls need no torch)."""
    if not _DT:
        import torch
        _DT.update(bf16=torch.bfloat16, u8=torch.uint8, f32=torch.float32, i32=torch.int32, i64=torch.int64)
    return _DT[kind]


def _dev(t, name: str, kind: str):
    """t must be a device tensor of the given element type; its pointer is
    handed to a kernel, so a host tensor or another dtype is rejected here."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor (got {type(t).__name__})")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (got device {t.device})")
    if t.dtype != _dtype(kind):
        raise ValueError(f"{name} must have dtype {_dtype(kind)} (got {t.dtype})")
    return t


def _ptr(t, name: str = "tensor", kind: str = "i32") -> Optional[int]:
    return None if t is None else _dev(t, name, kind).data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _rows(t, name: str, kind: str = "bf16"):
    """(pointer, row stride) of a 2-D row-major device view with unit column
    stride and the given element type."""
    _dev(t, name, kind)
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D view with unit column stride")
    return t.data_ptr(), t.stride(0)


def _flat(t, name: str, kind: str, n: int):
    """Pointer of a contiguous device tensor of at least n elements."""
    _dev(t, name, kind)
    if not t.is_contiguous() or t.numel() < n:
        raise ValueError(f"{name} must be contiguous with at least {n} elements (got {tuple(t.shape)})")
    return t.data_ptr()


def _table(t, name: str):
    """Pointer and row length of a 2-D contiguous int32 device table."""
    _dev(t, name, "i32")
    if t.dim() != 2 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-D int32 tensor [num_seqs, max_pages_per_seq]")
    return t.data_ptr(), t.shape[1]


def _cu(cu_seqlens, name: str = "cu_seqlens"):
    """(pointer or None, num_seqs) of an optional int32 [num_seqs + 1] table."""
    if cu_seqlens is None:
        return None, 1
    _flat(cu_seqlens, name, "i32", 1)
    return cu_seqlens.data_ptr(), cu_seqlens.numel() - 1


def _pool(t, name: str, cache_dtype: str):
    """Pointer of a contiguous page pool: bf16 pools hold 16-bit patterns
    (torch.bfloat16, or torch.int16 for the same bits), fp8 pools uint8 codes."""
    import torch
    if cache_dtype not in DTYPES:
        raise ValueError(f"unknown cache dtype {cache_dtype!r} (bf16 or fp8_e4m3)")
    if cache_dtype == "bf16" and isinstance(t, torch.Tensor) and t.dtype == torch.int16:
        _dev(t.view(torch.bfloat16), name, "bf16")
    else:
        _dev(t, name, "bf16" if cache_dtype == "bf16" else "u8")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


CLOCK_STAMP_WORDS = 4096       # 1024 blocks x (XCC id, HW_ID, shader-clock cycles, 100 MHz real time)


def clock_stamp(out, stream=None):
    """Enqueue pca_clock_stamp: the GPU's clock counters, read on the device, into
    the int64 device tensor out (CLOCK_STAMP_WORDS elements)."""
    _check("pca_clock_stamp", load().pca_clock_stamp(_flat(out, "out", "i64", CLOCK_STAMP_WORDS), _stream(stream)))
    return out


def shader_clock_mhz(before, after) -> dict:
    """Average shader clock per XCD between two stamps (host int64 arrays of
    CLOCK_STAMP_WORDS): for every CU that stamped both times (XCC id and the
    shader engine, array and CU bits of HW_ID), cycles elapsed over real time
    elapsed on that CU's own counters; per XCD the median over its CUs."""
    import numpy as np
    a, b = np.asarray(before).reshape(-1, 4), np.asarray(after).reshape(-1, 4)

    def by_cu(s):
        out = {}
        for x, hw, cyc, rt in s.tolist():
            out.setdefault((int(x), int(hw) & 0xFF00), []).append((cyc, rt))
        return {k: (np.median([c for c, _ in v]), np.median([r for _, r in v])) for k, v in out.items()}

    ca, cb = by_cu(a), by_cu(b)
    per_xcd = {}
    for k in set(ca) & set(cb):
        (c0, r0), (c1, r1) = ca[k], cb[k]
        if r1 > r0 and c1 > c0:
            per_xcd.setdefault(k[0], []).append((c1 - c0) / ((r1 - r0) / 100e6) / 1e6)
    return {x: float(np.median(v)) for x, v in sorted(per_xcd.items())}


def version() -> str:
    return load().pca_version().decode()


def kv_layout(n_head: int, n_kv_head: int, head_dim: int, page_size: int = 16,
              cache_dtype: str = "bf16") -> dict:
    out = KvLayout()
    _check("pca_kv_layout", load().pca_kv_layout(n_head, n_kv_head, head_dim, page_size,
                                                 DTYPES[cache_dtype], ctypes.byref(out)))
    return out.as_dict()


def qkv_proj(x, w_t, y, stream=None):
    """y[M, N] = x[M, K] @ w_t[N, K]^T on the GPU (bf16 tensors, 2-D views)."""
    px, ldx = _rows(x, "x")
    pw, ldw = _rows(w_t, "w_t")
    py, ldy = _rows(y, "y")
    M, K = x.shape
    N = w_t.shape[0]
    if w_t.shape[1] != K or tuple(y.shape) != (M, N):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, w_t {tuple(w_t.shape)}, y {tuple(y.shape)}")
    _check("pca_qkv_proj", load().pca_qkv_proj(px, ldx, pw, ldw, py, ldy, M, N, K, _stream(stream)))
    return y


def quantize_rows_fp8(x, q, scales, stream=None):
    """Row-wise E4M3 codes of the bf16 2-D view x into the uint8 view q, with
    the per-row scales (float32, (M,))."""
    px, ldx = _rows(x, "x")
    pq, ldq = _rows(q, "q", "u8")
    M, K = x.shape
    if tuple(q.shape) != (M, K):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, q {tuple(q.shape)}")
    ps = _flat(scales, "scales", "f32", M)
    _check("pca_quantize_rows_fp8", load().pca_quantize_rows_fp8(px, ldx, M, K, pq, ldq, ps, _stream(stream)))
    return q


def e4m3_encode(x, codes, stream=None):
    """E4M3 codes (RNE, saturating at +-448) of the contiguous float32 tensor x
    into the contiguous uint8 tensor codes of the same number of elements."""
    px = _flat(x, "x", "f32", 0)
    pc = _flat(codes, "codes", "u8", x.numel())
    if codes.numel() != x.numel():
        raise ValueError("x and codes must have the same number of elements")
    _check("pca_e4m3_encode", load().pca_e4m3_encode(px, pc, x.numel(), _stream(stream)))
    return codes


def qkv_proj_fp8(xq, sx, wq, sw, y, stream=None):
    """y = diag(sx) (dec(xq) @ dec(wq)^T) diag(sw) on fp8 matrix cores, bf16 out."""
    pxq, ldxq = _rows(xq, "xq", "u8")
    pwq, ldwq = _rows(wq, "wq", "u8")
    py, ldy = _rows(y, "y")
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K or tuple(y.shape) != (M, N):
        raise ValueError(f"shape mismatch: xq {tuple(xq.shape)}, wq {tuple(wq.shape)}, y {tuple(y.shape)}")
    psx, psw = _flat(sx, "sx", "f32", M), _flat(sw, "sw", "f32", N)
    _check("pca_qkv_proj_fp8", load().pca_qkv_proj_fp8(pxq, ldxq, psx, pwq, ldwq, psw, py, ldy,
                                                       M, N, K, _stream(stream)))
    return y


def rms_norm_qkv_proj(x, w_t_g, y, inv_rms, eps: float = 1e-6, stream=None):
    """y = diag(inv_rms) (x @ w_t_g^T) with inv_rms[m] = 1/sqrt(mean x[m]^2 + eps)
    written into the float32 device tensor inv_rms (M,); w_t_g is W^T with the
    norm gain folded along K."""
    px, ldx = _rows(x, "x")
    pw, ldw = _rows(w_t_g, "w_t_g")
    py, ldy = _rows(y, "y")
    M, K = x.shape
    N = w_t_g.shape[0]
    if w_t_g.shape[1] != K or tuple(y.shape) != (M, N):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, w_t_g {tuple(w_t_g.shape)}, y {tuple(y.shape)}")
    pr = _flat(inv_rms, "inv_rms", "f32", M)
    _check("pca_rms_norm_qkv_proj", load().pca_rms_norm_qkv_proj(px, ldx, pw, ldw, float(eps), pr,
                                                                 py, ldy, M, N, K, _stream(stream)))
    return y


def rms_norm_qkv_proj_noalloc(x, w_t_g, y, eps: float = 1e-6, stream=None):
    """rms_norm_qkv_proj with the 1/rms workspace in the library's static
    device array (no allocation by the call; M <= NOALLOC_MAX_ROWS; calls that
    overlap in time on one GPU race on that array)."""
    px, ldx = _rows(x, "x")
    pw, ldw = _rows(w_t_g, "w_t_g")
    py, ldy = _rows(y, "y")
    M, K = x.shape
    N = w_t_g.shape[0]
    if w_t_g.shape[1] != K or tuple(y.shape) != (M, N):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, w_t_g {tuple(w_t_g.shape)}, y {tuple(y.shape)}")
    _check("pca_rms_norm_qkv_proj_noalloc", load().pca_rms_norm_qkv_proj_noalloc(
        px, ldx, pw, ldw, float(eps), py, ldy, M, N, K, _stream(stream)))
    return y


def out_proj_residual(o, w_t, res, out, stream=None):
    """out[M, N] = res + o[M, K] @ w_t[N, K]^T (bf16, fp32 accumulate, one
    rounding); res may be out itself."""
    po, ldo = _rows(o, "o")
    pw, ldw = _rows(w_t, "w_t")
    pr, ldr = _rows(res, "res")
    pout, ldout = _rows(out, "out")
    M, K = o.shape
    N = w_t.shape[0]
    if w_t.shape[1] != K or tuple(res.shape) != (M, N) or tuple(out.shape) != (M, N):
        raise ValueError(f"shape mismatch: o {tuple(o.shape)}, w_t {tuple(w_t.shape)}, res {tuple(res.shape)}, "
                         f"out {tuple(out.shape)}")
    _check("pca_out_proj_residual", load().pca_out_proj_residual(po, ldo, pw, ldw, pr, ldr, pout, ldout, M, N, K,
                                                                 _stream(stream)))
    return out


def qkv_proj_kv_write(x, w_t, y, block_table, k_cache, v_cache, n_head: int, n_kv_head: int, head_dim: int,
                      cu_seqlens=None, cache_dtype: str = "bf16", k_scale=None, v_scale=None,
                      page_size: int = 16, stream=None):
    """qkv_proj with the KV-cache write in the GEMM epilogue: y as from
    qkv_proj, pools as from kv_cache_write of y's K and V columns."""
    px, ldx = _rows(x, "x")
    pw, ldw = _rows(w_t, "w_t")
    py, ldy = _rows(y, "y")
    M, K = x.shape
    N = (n_head + 2 * n_kv_head) * head_dim
    if tuple(w_t.shape) != (N, K) or tuple(y.shape) != (M, N):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, w_t {tuple(w_t.shape)}, y {tuple(y.shape)}, N={N}")
    pcu, num_seqs = _cu(cu_seqlens)
    pbt, mp = _table(block_table, "block_table")
    pk, pv = _pool(k_cache, "k_cache", cache_dtype), _pool(v_cache, "v_cache", cache_dtype)
    num_pages = k_cache.numel() // (page_size * n_kv_head * head_dim)
    _check("pca_qkv_proj_kv_write", load().pca_qkv_proj_kv_write(
        px, ldx, pw, ldw, py, ldy, M, K, n_head, n_kv_head, head_dim, pcu, num_seqs,
        pbt, mp, page_size, DTYPES[cache_dtype], pk, pv, _ptr(k_scale, "k_scale", "f32"),
        _ptr(v_scale, "v_scale", "f32"), num_pages, _stream(stream)))
    return y


def prefill_attention(q, k, v, o, n_head: int, n_kv_head: int, head_dim: int,
                      cu_seqlens=None, max_seqlen: Optional[int] = None, scale: Optional[float] = None,
                      total_tokens: Optional[int] = None, window: int = 0, stream=None):
    """Causal GQA attention.  q, k, v, o: 2-D token-major views (T, >= heads*hd)
    with unit column stride (e.g. column slices of the fused projection output).
    cu_seqlens: int32 device tensor [num_seqs + 1] or None (one sequence).
    window > 0: sliding window (row r sees keys r - window < c <= r)."""
    pq, ldq = _rows(q, "q")
    pk, ldk = _rows(k, "k")
    pv, ldv = _rows(v, "v")
    po, ldo = _rows(o, "o")
    T = q.shape[0] if total_tokens is None else int(total_tokens)
    if min(k.shape[0], v.shape[0], o.shape[0]) < T:
        raise ValueError(f"q, k, v and o need at least total_tokens = {T} rows")
    pcu, num_seqs = _cu(cu_seqlens)
    if max_seqlen is None:
        max_seqlen = T
    if scale is None:
        scale = head_dim ** -0.5
    if window:
        _check("pca_prefill_attention_window", load().pca_prefill_attention_window(
            pq, pk, pv, ldq, ldk, ldv, pcu, num_seqs, int(max_seqlen), T,
            n_head, n_kv_head, head_dim, float(scale), 1, int(window), po, ldo, _stream(stream)))
        return o
    _check("pca_prefill_attention", load().pca_prefill_attention(
        pq, pk, pv, ldq, ldk, ldv, pcu, num_seqs, int(max_seqlen), T,
        n_head, n_kv_head, head_dim, float(scale), 1, po, ldo, _stream(stream)))
    return o


def prefill_attention_splitkv_workspace(num_seqs: int, max_seqlen: int, n_head: int, n_kv_head: int,
                                        head_dim: int) -> int:
    """Bytes of the workspace prefill_attention_splitkv needs for these sizes."""
    n = load().pca_prefill_attention_splitkv_workspace(int(num_seqs), int(max_seqlen), int(n_head), int(n_kv_head),
                                                       int(head_dim))
    if n < 0:
        raise PcaError("pca_prefill_attention_splitkv_workspace", -1, load().pca_last_error().decode())
    return int(n)


def prefill_attention_splitkv(q, k, v, o, workspace, n_head: int, n_kv_head: int, head_dim: int,
                              cu_seqlens=None, max_seqlen: Optional[int] = None, scale: Optional[float] = None,
                              total_tokens: Optional[int] = None, stream=None):
    """prefill_attention with split key ranges on shallow grids.  workspace: a
    contiguous uint8 device tensor of at least prefill_attention_splitkv_workspace
    bytes, 256-byte aligned, zeroed once before its first use (each call leaves
    its counters zero); calls sharing it must not overlap."""
    pq, ldq = _rows(q, "q")
    pk, ldk = _rows(k, "k")
    pv, ldv = _rows(v, "v")
    po, ldo = _rows(o, "o")
    _dev(workspace, "workspace", "u8")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    T = q.shape[0] if total_tokens is None else int(total_tokens)
    if min(k.shape[0], v.shape[0], o.shape[0]) < T:
        raise ValueError(f"q, k, v and o need at least total_tokens = {T} rows")
    pcu, num_seqs = _cu(cu_seqlens)
    if max_seqlen is None:
        max_seqlen = T
    if scale is None:
        scale = head_dim ** -0.5
    _check("pca_prefill_attention_splitkv", load().pca_prefill_attention_splitkv(
        pq, pk, pv, ldq, ldk, ldv, pcu, num_seqs, int(max_seqlen), T,
        n_head, n_kv_head, head_dim, float(scale), 1, po, ldo, workspace.data_ptr(), workspace.numel(),
        _stream(stream)))
    return o


def quantize_heads_fp8(x, codes, exps, n_heads: int, head_dim: int, prescale: float = 1.0, stream=None):
    """Per-(token, head) E4M3 rows of x * prescale with power-of-two scales.
    x: bf16 (T, >= n_heads*head_dim) view; codes: uint8 (T, >= n_heads*head_dim)
    view; exps: uint8 (T, >= n_heads) view (scale bytes e + 127)."""
    px, ldx = _rows(x, "x")
    pc, ldc = _rows(codes, "codes", "u8")
    pe, lde = _rows(exps, "exps", "u8")
    T = x.shape[0]
    if codes.shape[0] != T or exps.shape[0] != T:
        raise ValueError("x, codes and exps must have the same number of rows")
    _check("pca_quantize_heads_fp8", load().pca_quantize_heads_fp8(px, ldx, T, n_heads, head_dim, float(prescale),
                                                                   pc, ldc, pe, lde, _stream(stream)))
    return codes, exps


def prefill_attention_fp8qk(q, k_codes, k_exps, v, o, n_head: int, n_kv_head: int, head_dim: int,
                            cu_seqlens=None, max_seqlen: Optional[int] = None, scale: Optional[float] = None,
                            total_tokens: Optional[int] = None, stream=None):
    """Causal GQA attention with fp8 score operands: q bf16 (quantised inside
    after the scale * log2(e) factor), K as codes + scale bytes from
    quantize_heads_fp8, v bf16; o bf16 (T, n_head*head_dim)."""
    pq, ldq = _rows(q, "q")
    pk, ldk = _rows(k_codes, "k_codes", "u8")
    pe, lde = _rows(k_exps, "k_exps", "u8")
    pv, ldv = _rows(v, "v")
    po, ldo = _rows(o, "o")
    T = q.shape[0] if total_tokens is None else int(total_tokens)
    if min(k_codes.shape[0], k_exps.shape[0], v.shape[0], o.shape[0]) < T:
        raise ValueError(f"q, k_codes, k_exps, v and o need at least total_tokens = {T} rows")
    pcu, num_seqs = _cu(cu_seqlens)
    if max_seqlen is None:
        max_seqlen = T
    if scale is None:
        scale = head_dim ** -0.5
    _check("pca_prefill_attention_fp8qk", load().pca_prefill_attention_fp8qk(
        pq, ldq, pk, ldk, pe, lde, pv, ldv, pcu, num_seqs, int(max_seqlen), T,
        n_head, n_kv_head, head_dim, float(scale), 1, po, ldo, _stream(stream)))
    return o


def prefill_attention_paged(q, o, k_cache, v_cache, block_table, ctx_lens, n_head: int, n_kv_head: int,
                            head_dim: int, cu_seqlens=None, max_seqlen: Optional[int] = None,
                            max_ctx: Optional[int] = None, scale: Optional[float] = None,
                            cache_dtype: str = "bf16", k_scale=None, v_scale=None, page_size: int = 16,
                            total_tokens: Optional[int] = None, window: int = 0, stream=None):
    """Causal GQA attention of chunk rows q over the cached keys of their
    sequences (prefix then the chunk itself) read through the block table.
    ctx_lens: int32 device tensor [num_seqs], keys per sequence.
    window > 0: sliding window over the key positions (row at position p
    sees keys p - window < c <= p)."""
    pq, ldq = _rows(q, "q")
    po, ldo = _rows(o, "o")
    T = q.shape[0] if total_tokens is None else int(total_tokens)
    if o.shape[0] < T:
        raise ValueError(f"q and o need at least total_tokens = {T} rows")
    pcu, num_seqs = _cu(cu_seqlens, "cu_seqlens")
    pctx = _flat(ctx_lens, "ctx_lens", "i32", num_seqs)
    if max_seqlen is None:
        max_seqlen = T
    if max_ctx is None:
        max_ctx = int(ctx_lens.max().item()) if ctx_lens.numel() else 0
    if scale is None:
        scale = head_dim ** -0.5
    pbt, mp = _table(block_table, "block_table")
    pk, pv = _pool(k_cache, "k_cache", cache_dtype), _pool(v_cache, "v_cache", cache_dtype)
    num_pages = k_cache.numel() // (page_size * n_kv_head * head_dim)
    args = (pq, ldq, pcu, num_seqs, int(max_seqlen), T, pctx, int(max_ctx),
            pbt, mp, page_size, DTYPES[cache_dtype], pk, pv, _ptr(k_scale, "k_scale", "f32"),
            _ptr(v_scale, "v_scale", "f32"), num_pages, n_head, n_kv_head, head_dim, float(scale), 1)
    if window:
        _check("pca_prefill_attention_paged_window", load().pca_prefill_attention_paged_window(
            *args, int(window), po, ldo, _stream(stream)))
    else:
        _check("pca_prefill_attention_paged", load().pca_prefill_attention_paged(*args, po, ldo, _stream(stream)))
    return o


def kv_cache_write(k, v, block_table, k_cache, v_cache, n_kv_head: int, head_dim: int,
                   cu_seqlens=None, cache_dtype: str = "bf16", k_scale=None, v_scale=None,
                   page_size: int = 16, total_tokens: Optional[int] = None, stream=None):
    """Scatter K/V rows into the page pools through the block table (int32 device
    tensor [num_seqs, max_pages_per_seq]).  Pools are device tensors of
    num_pages * page_size * n_kv_head * head_dim elements (bf16 or uint8)."""
    pk, ldk = _rows(k, "k")
    pv, ldv = _rows(v, "v")
    T = k.shape[0] if total_tokens is None else int(total_tokens)
    if v.shape[0] < T:
        raise ValueError(f"k and v need at least total_tokens = {T} rows")
    pcu, num_seqs = _cu(cu_seqlens)
    pbt, mp = _table(block_table, "block_table")
    pkc, pvc = _pool(k_cache, "k_cache", cache_dtype), _pool(v_cache, "v_cache", cache_dtype)
    num_pages = k_cache.numel() // (page_size * n_kv_head * head_dim)
    _check("pca_kv_cache_write", load().pca_kv_cache_write(
        pk, pv, ldk, ldv, pcu, num_seqs, T, pbt, mp,
        n_kv_head, head_dim, page_size, DTYPES[cache_dtype], pkc, pvc,
        _ptr(k_scale, "k_scale", "f32"), _ptr(v_scale, "v_scale", "f32"), num_pages, _stream(stream)))
