"""Seeded synthetic workloads for exact attention: shapes and input generators.

This module holds the workload table and the random-input recipe shared by the
CPU oracle's tests, the GPU parity tests, smoke() and bench.py.  It contains
none of the attention arithmetic: it only draws numbers.

Recipe (the same everywhere):
  * numpy ``Generator(PCG64(seed))``;
  * Q, then K, then V are drawn with ``standard_normal(dtype=float32)`` in C
    order over their full ``[B, H, S, D]`` shape, one leading-batch slice at a
    time (the draw stream is the same as one whole-array draw);
  * each value is rounded to IEEE fp16 (round-to-nearest-even).
The causal and non-causal runs of one workload reuse the same tensors.

Paged KV caches (for paged decoding) are laid out from the same contiguous
K / V draws: every sequence's context is cut into logical blocks of
block_size tokens, and the logical blocks of all sequences are dealt to
physical pages [num_blocks, H, block_size, D] in a seeded random order
(``paged_layout`` / ``to_pages``), so that consecutive blocks of one sequence
are scattered through the cache as they would be after many allocations and
frees.  Pages that no table entry names are filled with NaN, so a read of one
would show up in the result.

Packed variable-length batches (``make_varlen``) use the same recipe over the
packed [total_tokens, H, D] shape (Q, then K, then V), with sequence lengths
drawn uniformly from a range by a seeded generator of their own; the
cumulative lengths start at 0 and cover every token.

The shapes follow the pages' workloads: the LLaMA-7B prefill shape
(1, 32, 4096, 4096, 128) and the 8K-context single-query decode shape of the
"FlashAttention-2 MMA" benchmark tables, the B8/H16/S256/D64 shape of
"Flash Attention 101"'s A100 benchmark, a D=256 large-head prefill, and the
"Large Head" (D = 512) and "Massive Head" (D = 1024) shapes of the
"FlashAttention-2 MMA" benchmark matrix.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Sq: int
    Sk: int
    D: int
    causal: tuple  # the mask settings this workload is run with
    seed: int
    kind: str  # "prefill" or "decode"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def shape_q(self):
        return (self.B, self.H, self.Sq, self.D)

    def shape_kv(self):
        return (self.B, self.H, self.Sk, self.D)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 128, 128, 64, (False, True), 1, "prefill"),
    "small": Workload("small", 8, 16, 256, 256, 64, (False, True), 2, "prefill"),
    "llama7b_prefill": Workload("llama7b_prefill", 1, 32, 4096, 4096, 128, (True,), 3, "prefill"),
    "decode_8k": Workload("decode_8k", 16, 32, 1, 8192, 128, (False,), 4, "decode"),
    "d256_prefill": Workload("d256_prefill", 1, 16, 2048, 2048, 256, (True,), 5, "prefill"),
    # large heads (Split-D)
    "d512_prefill": Workload("d512_prefill", 1, 8, 1024, 1024, 512, (False, True), 9, "prefill"),
    "d1024_prefill": Workload("d1024_prefill", 1, 4, 512, 512, 1024, (False, True), 10, "prefill"),
}


def _draw_fp16(gen: np.random.Generator, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.float16)
    for b in range(shape[0]):
        out[b] = gen.standard_normal(shape[1:], dtype=np.float32).astype(np.float16)
    return out


def make_qkv(B: int, H: int, Sq: int, Sk: int, D: int, seed: int):
    """Q [B,H,Sq,D], K and V [B,H,Sk,D] as fp16 numpy arrays, N(0,1) draws."""
    gen = np.random.Generator(np.random.PCG64(seed))
    q = _draw_fp16(gen, (B, H, Sq, D))
    k = _draw_fp16(gen, (B, H, Sk, D))
    v = _draw_fp16(gen, (B, H, Sk, D))
    return q, k, v


def workload_inputs(w: Workload):
    return make_qkv(w.B, w.H, w.Sq, w.Sk, w.D, w.seed)


# Paged decoding: the 8K decode shape with its K / V held in 16-token pages.
PAGED_BLOCK_SIZE = 16
PAGED_PERM_SEED = 6


def paged_layout(B: int, max_blocks: int, seed: int, spare: int = 0):
    """Block tables [B, max_blocks] int32 naming distinct physical pages in a
    seeded random order, plus the page count (B * max_blocks + spare)."""
    num_blocks = B * max_blocks + spare
    gen = np.random.Generator(np.random.PCG64(seed))
    perm = gen.permutation(num_blocks)[: B * max_blocks]
    return perm.reshape(B, max_blocks).astype(np.int32), num_blocks


def to_pages(x: np.ndarray, tables: np.ndarray, num_blocks: int, block_size: int) -> np.ndarray:
    """Scatter contiguous [B, H, S, D] rows into pages [num_blocks, H, block_size, D]:
    rows j*block_size .. of sequence b go to page tables[b, j].  S may be shorter
    than the tables' reach (the rest of those pages stays NaN), unnamed pages are NaN."""
    B, H, S, D = x.shape
    pages = np.full((num_blocks, H, block_size, D), np.nan, dtype=x.dtype)
    for b in range(B):
        for j in range(-(-S // block_size)):
            lo, hi = j * block_size, min(S, (j + 1) * block_size)
            pages[tables[b, j], :, : hi - lo, :] = x[b, :, lo:hi, :]
    return pages


# Packed variable-length prefill: 16 sequences of 256..4096 tokens (LLaMA-7B
# heads), the ragged counterpart of the 4096-token prefill.
VARLEN_B, VARLEN_H, VARLEN_D = 16, 32, 128
VARLEN_MIN, VARLEN_MAX = 256, 4096
VARLEN_LEN_SEED, VARLEN_SEED = 8, 7


def varlen_lengths(B: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """B sequence lengths drawn uniformly from [lo, hi]."""
    gen = np.random.Generator(np.random.PCG64(seed))
    return gen.integers(lo, hi + 1, size=B).astype(np.int64)


def make_varlen(lengths, H: int, D: int, seed: int, lengths_k=None):
    """Packed q [total_q, H, D] and k, v [total_k, H, D] fp16 (N(0,1) draws,
    Q then K then V) with their cumulative lengths [B + 1] int32."""
    lengths = np.asarray(lengths, dtype=np.int64)
    lengths_k = lengths if lengths_k is None else np.asarray(lengths_k, dtype=np.int64)
    cu_q = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lengths_k)]).astype(np.int32)
    gen = np.random.Generator(np.random.PCG64(seed))
    q = _draw_fp16(gen, (int(cu_q[-1]), H, D)) if cu_q[-1] > 0 else np.zeros((0, H, D), np.float16)
    k = _draw_fp16(gen, (int(cu_k[-1]), H, D)) if cu_k[-1] > 0 else np.zeros((0, H, D), np.float16)
    v = _draw_fp16(gen, (int(cu_k[-1]), H, D)) if cu_k[-1] > 0 else np.zeros((0, H, D), np.float16)
    return q, k, v, cu_q, cu_k


def sample_rows(w: Workload, count: int, seed: int = 12345):
    """A seeded sample of (b, h, i) output rows, always including the first
    and last row of the first and last (b, h) slice."""
    gen = np.random.Generator(np.random.PCG64(seed))
    picks = {(0, 0, 0), (w.B - 1, w.H - 1, w.Sq - 1), (0, 0, w.Sq - 1), (w.B - 1, w.H - 1, 0)}
    while len(picks) < count + 4:
        picks.add((int(gen.integers(w.B)), int(gen.integers(w.H)), int(gen.integers(w.Sq))))
    return sorted(picks)
