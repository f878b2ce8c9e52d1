"""Decoding over a paged KV cache, fp64 -- test infrastructure only (see package doc).

Definition followed
  * Paged KV memory: K and V are stored as physical pages
    [num_blocks, H, block_size, d], and a per-sequence block table names the
    physical page holding each logical block of block_size consecutive token
    positions: "Adaptive High-Performance Attention Kernels in CUDA",
    Advanced Production Features, 4. PagedAttention.
  * Single-query decoding attends the query of sequence b to its whole
    context, non-causally, with the same scaled-softmax definition as
    ``dense.attention`` (see that module's header for its passages).

Readings where the page is silent (shared with the C-ABI contract)
  * The context of sequence b is token positions 0 .. seq_lens[b]-1, with
    seq_lens[b] clamped to [0, max_blocks * block_size].
  * Token t lives in page table[b][t // block_size] at row t % block_size.
    A table entry outside [0, num_blocks) marks its tokens absent: they are
    not read and do not take part in the softmax.
  * A sequence with no present token gets O = 0 and LSE = -inf (the log of
    an empty sum).
"""
from __future__ import annotations

import numpy as np

from .dense import attention


def context_tokens(table_row, seq_len, block_size, num_blocks):
    """Present token positions of one sequence and their (page, row) addresses."""
    L = int(min(max(int(seq_len), 0), len(table_row) * block_size))
    toks, pages, rows = [], [], []
    for t in range(L):
        p = int(table_row[t // block_size])
        if 0 <= p < num_blocks:
            toks.append(t)
            pages.append(p)
            rows.append(t % block_size)
    return toks, pages, rows


def gather_context(cache, table_row, seq_len):
    """The present context rows of one sequence, [H, n, D] in token order."""
    num_blocks, H, block_size, D = cache.shape
    _, pages, rows = context_tokens(table_row, seq_len, block_size, num_blocks)
    if not pages:
        return np.zeros((H, 0, D), dtype=np.float64)
    g = np.asarray(cache)[np.asarray(pages), :, np.asarray(rows), :]  # [n, H, D]
    return np.ascontiguousarray(np.transpose(g, (1, 0, 2))).astype(np.float64)


def decode_paged(q, k_cache, v_cache, block_tables, seq_lens, scale):
    """O [B, H, 1, D] and LSE [B, H, 1] of paged single-query decoding (fp64).

    q: [B, H, 1, D]; k_cache, v_cache: [num_blocks, H, block_size, D];
    block_tables: [B, max_blocks] ints; seq_lens: [B] ints.
    """
    q = np.asarray(q)
    B, H, Sq, D = q.shape
    if Sq != 1:
        raise ValueError("decoding takes one query row per sequence")
    if k_cache.shape != v_cache.shape or k_cache.shape[1] != H or k_cache.shape[3] != D:
        raise ValueError("cache shape mismatch")
    O = np.zeros((B, H, 1, D), dtype=np.float64)
    L = np.full((B, H, 1), -np.inf, dtype=np.float64)
    for b in range(B):
        kb = gather_context(k_cache, block_tables[b], seq_lens[b])
        if kb.shape[1] == 0:
            continue
        vb = gather_context(v_cache, block_tables[b], seq_lens[b])
        o, lse = attention(q[b : b + 1], kb[None], vb[None], False, scale)
        O[b] = o[0]
        L[b] = lse[0]
    return O, L
