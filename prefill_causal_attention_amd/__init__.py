"""Prefill attention-unit path for MI355X (gfx950): the Python face of libpca.

Calls (same names as the C ABI in include/pca.h, minus the ``pca_`` prefix):
  kv_layout          head-split offsets, page-pool strides and KV byte counts
  qkv_proj           fused QKV projection GEMM (bf16 MFMA, fp32 accumulate)
  qkv_proj_kv_write  the same GEMM, its epilogue also writing K/V into the pages
  out_proj_residual  output projection W_o with the residual add (one rounding)
  rms_norm_qkv_proj  the input RMSNorm folded into the QKV GEMM (row scale in the epilogue)
  rms_norm_qkv_proj_noalloc  the same with the library's static workspace (no allocation)
  quantize_rows_fp8  row-wise E4M3 quantisation of GEMM operands
  qkv_proj_fp8       the QKV GEMM on fp8 operands (fp8 matrix cores, fp32 accumulate)
  e4m3_encode        elementwise float32 -> E4M3 codes (the encoder of every fp8 result)
  prefill_attention  causal GQA flash attention with online softmax
  quantize_heads_fp8 per-(token, head) E4M3 rows with power-of-two scales
  prefill_attention_fp8qk  the same attention with fp8 Q.K^T operands
  prefill_attention_paged  the same for a chunk over its cached (paged) prefix
  prefill_attention_splitkv  the same with split key ranges for shallow grids (caller's workspace)
  prefill_attention_splitkv_workspace  bytes of that workspace
  kv_cache_write     scatter of K/V into 16-token pages (bf16 or fp8 E4M3)
All compute runs in hand-written HIP kernels; PyTorch only provides device
memory and the current stream.
"""
from ._lib import (CLOCK_STAMP_WORDS, EXPORTED, NOALLOC_MAX_ROWS, PcaError, clock_stamp, shader_clock_mhz, e4m3_encode, kv_cache_write, kv_layout, load,  # noqa: F401
                   out_proj_residual, prefill_attention, prefill_attention_fp8qk, prefill_attention_paged,
                   prefill_attention_splitkv, prefill_attention_splitkv_workspace,
                   qkv_proj, qkv_proj_fp8, qkv_proj_kv_write, quantize_heads_fp8, quantize_rows_fp8,
                   rms_norm_qkv_proj, rms_norm_qkv_proj_noalloc, version)

__all__ = ["kv_layout", "qkv_proj", "qkv_proj_kv_write", "rms_norm_qkv_proj", "rms_norm_qkv_proj_noalloc",
           "out_proj_residual", "quantize_rows_fp8",
           "qkv_proj_fp8", "e4m3_encode", "quantize_heads_fp8", "prefill_attention", "prefill_attention_fp8qk",
           "prefill_attention_paged", "prefill_attention_splitkv", "prefill_attention_splitkv_workspace",
           "kv_cache_write", "load", "version",
           "PcaError", "EXPORTED", "NOALLOC_MAX_ROWS", "clock_stamp", "shader_clock_mhz", "CLOCK_STAMP_WORDS"]
