"""Seeded synthetic inputs for the prefill attention-unit path.

This module is shared by the tests, the bench and the smoke check.  It only
draws random numbers and rounds them to the storage format (bf16 RNE, the
same rounding every consumer sees); it holds none of the method's arithmetic.

Recipe (one per workload, the five workloads the path is exercised on):
  * every tensor is drawn with ``numpy.random.default_rng(seed)`` in float32,
    ``seed = 1000 * workload_index + tensor_id`` with workload_index 1..5 and
    tensor ids X=1, W=2, Q=3, K=4, V=5, lengths=6, block table=7;
  * X ~ N(0, 1); W_qkv ~ N(0, 1/h) drawn in (h, N) form; Q/K/V (tiny MHA
    workload) ~ N(0, 1); then rounded to bf16 round-to-nearest-even once;
  * varlen lengths: ``rng.integers(256, 4097, 16)``;
  * block tables: identity, or a seeded permutation of the page pool.
The pages the path follows measure on synthetic-like "8k-token long document"
prompts and 7B/70B-class shapes; these draws stand in for them.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

PAGE_SIZE = 16

TENSOR_X, TENSOR_W, TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_LENGTHS, TENSOR_BT = 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int            # 1-based, in the order listed below
    name: str
    seqlens: tuple        # one entry per packed sequence
    h: int                # hidden size (0: no projection, Q/K/V drawn directly)
    n_head: int
    n_kv_head: int
    head_dim: int
    cache: str            # "contiguous", "bf16" (paged) or "fp8" (paged)
    block_table: str      # "none", "identity", "permutation"
    spare_pages: int = 0

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def num_seqs(self) -> int:
        return len(self.seqlens)

    @property
    def max_seqlen(self) -> int:
        return int(max(self.seqlens))

    @property
    def n_qkv(self) -> int:
        return (self.n_head + 2 * self.n_kv_head) * self.head_dim

    @property
    def group(self) -> int:
        return self.n_head // self.n_kv_head

    @property
    def pages_per_seq(self) -> List[int]:
        return [-(-L // PAGE_SIZE) for L in self.seqlens]

    @property
    def num_pages(self) -> int:
        return sum(self.pages_per_seq) + self.spare_pages

    def attention_flops(self) -> float:
        # causal count 2*2*L^2*hd*n_head/2, summed over the packed sequences
        return float(sum(2 * L * L * self.head_dim * self.n_head for L in self.seqlens))

    def gemm_flops(self) -> float:
        return 2.0 * self.total_tokens * self.h * self.n_qkv

    def seed(self, tensor_id: int) -> int:
        return 1000 * self.index + tensor_id


def _varlen_lengths(index: int) -> tuple:
    rng = np.random.default_rng(1000 * index + TENSOR_LENGTHS)
    return tuple(int(x) for x in rng.integers(256, 4097, 16))


WORKLOADS = [
    Workload(1, "tiny_mha_s64", (64,), 0, 2, 2, 32, "contiguous", "none"),
    Workload(2, "mha_s2048", (2048,), 4096, 32, 32, 128, "bf16", "identity"),
    Workload(3, "gqa_s8192", (8192,), 4096, 32, 8, 128, "bf16", "permutation"),
    Workload(4, "varlen16_gqa", _varlen_lengths(4), 4096, 32, 8, 128, "bf16", "permutation", spare_pages=64),
    Workload(5, "long_gqa_s32768_fp8kv", (32768,), 5120, 40, 8, 128, "fp8", "permutation"),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def normal_bf16(seed: int, shape, std: float = 1.0) -> torch.Tensor:
    """float32 N(0, std^2) draw rounded once to bf16 (torch's cast is RNE); CPU tensor."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return torch.from_numpy(x).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The uint16 storage bits of a bf16 tensor (no arithmetic)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def cu_seqlens(w: Workload) -> np.ndarray:
    cu = np.zeros(w.num_seqs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(w.seqlens, dtype=np.int64))
    return cu


def block_table(w: Workload) -> Optional[np.ndarray]:
    """int32 [num_seqs][max_pages_per_seq]; each sequence starts on a fresh page,
    all pages come from one pool of ``num_pages``; unused entries are -1."""
    if w.block_table == "none":
        return None
    pps = w.pages_per_seq
    need = sum(pps)
    if w.block_table == "identity":
        order = np.arange(w.num_pages, dtype=np.int64)
    else:
        rng = np.random.default_rng(w.seed(TENSOR_BT))
        order = rng.permutation(w.num_pages)
    bt = np.full((w.num_seqs, max(pps)), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(pps):
        bt[b, :n] = order[pos:pos + n]
        pos += n
    assert pos == need
    return bt


def projection_inputs(w: Workload):
    """X (T, h) bf16 and W_qkv drawn in (h, N) form, bf16 (CPU tensors)."""
    x = normal_bf16(w.seed(TENSOR_X), (w.total_tokens, w.h))
    wq = normal_bf16(w.seed(TENSOR_W), (w.h, w.n_qkv), std=float(1.0 / np.sqrt(w.h)))
    return x, wq


def qkv_inputs(w: Workload, ld: Optional[int] = None):
    """Q, K, V drawn directly (no projection), packed in one (T, ld) bf16 buffer
    with column blocks [Q | K | V], the layout the projection writes.
    Returns (buf, q_off, k_off, v_off)."""
    T = w.total_tokens
    nq, nk = w.n_head * w.head_dim, w.n_kv_head * w.head_dim
    ld = ld or (nq + 2 * nk)
    buf = torch.zeros((T, ld), dtype=torch.bfloat16)
    buf[:, :nq] = normal_bf16(w.seed(TENSOR_Q), (T, nq))
    buf[:, nq:nq + nk] = normal_bf16(w.seed(TENSOR_K), (T, nk))
    buf[:, nq + nk:nq + 2 * nk] = normal_bf16(w.seed(TENSOR_V), (T, nk))
    return buf, 0, nq, nq + nk


def custom(index: int, seqlens, n_head: int, n_kv_head: int, head_dim: int, h: int = 0,
           cache: str = "bf16", block_table: str = "permutation", spare_pages: int = 0,
           name: str = "custom") -> Workload:
    """A workload of arbitrary shape for parity cases (index only picks seeds)."""
    return Workload(index, name, tuple(int(x) for x in seqlens), h, n_head, n_kv_head,
                    head_dim, cache, block_table, spare_pages)
