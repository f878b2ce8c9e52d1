"""Attention over a packed batch of variable-length sequences, fp64 -- test
infrastructure only (see package doc).

Definition followed
  * Ragged / variable-length batches: the tokens of all sequences form one
    stream [total_tokens, H, d], and cumulative sequence lengths cu_seqlens
    mark where each sequence starts, with no padding: "Adaptive
    High-Performance Attention Kernels in CUDA", Advanced Production
    Features, 3. Ragged / Variable-Length Sequences.
  * Within a sequence the computation is ``dense.attention`` (see that
    module's header for its passages); sequences never see each other.

Readings where the page is silent (shared with the C-ABI contract)
  * Sequence b owns query tokens cu_q[b] .. cu_q[b+1]-1 and key tokens
    cu_k[b] .. cu_k[b+1]-1; the causal rule is the dense one inside each
    sequence (its query i sees its keys 0..i).
  * The cumulative arrays are not trusted: each start is clamped to
    [0, total] and each length to [0, min(total - start, max_seqlen)].
  * A query row whose sequence has no key gets O = 0 and LSE = -inf; query
    rows no sequence covers are not produced (NaN here).
  * LSE is laid out [H, total_q].
"""
from __future__ import annotations

import numpy as np

from .dense import attention


def sequence_bounds(cu, b, total, max_len):
    """(start, length) of sequence b after the clamps listed above."""
    start = min(max(int(cu[b]), 0), total)
    length = min(max(int(cu[b + 1]) - start, 0), total - start, max_len)
    return start, length


def attention_varlen(q, k, v, cu_q, cu_k, causal, scale, max_q=None, max_k=None):
    """O [total_q, H, Dv] and LSE [H, total_q] (fp64) of a packed batch.

    q: [total_q, H, D]; k: [total_k, H, D]; v: [total_k, H, Dv];
    cu_q, cu_k: [B + 1] ints.  Rows that no sequence covers are NaN.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    total_q, H, D = q.shape
    total_k = k.shape[0]
    if k.shape[1:] != (H, D) or v.shape[:2] != (total_k, H):
        raise ValueError("shape mismatch")
    B = len(cu_q) - 1
    max_q = total_q if max_q is None else max_q
    max_k = total_k if max_k is None else max_k
    O = np.full((total_q, H, v.shape[2]), np.nan, dtype=np.float64)
    L = np.full((H, total_q), np.nan, dtype=np.float64)
    for b in range(B):
        sq, lq = sequence_bounds(cu_q, b, total_q, max_q)
        sk, lk = sequence_bounds(cu_k, b, total_k, max_k)
        if lq == 0:
            continue
        if lk == 0:
            O[sq : sq + lq] = 0.0
            L[:, sq : sq + lq] = -np.inf
            continue
        qb = np.transpose(q[sq : sq + lq], (1, 0, 2))[None]  # [1, H, lq, D]
        kb = np.transpose(k[sk : sk + lk], (1, 0, 2))[None]
        vb = np.transpose(v[sk : sk + lk], (1, 0, 2))[None]
        o, lse = attention(qb, kb, vb, causal, scale)
        O[sq : sq + lq] = np.transpose(o[0], (1, 0, 2))
        L[:, sq : sq + lq] = lse[0]
    return O, L
