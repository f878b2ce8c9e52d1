"""Plain fp64 attention on the CPU -- test infrastructure only (see package doc).

Definitions followed
  * Scores S = scale * Q K^T, probabilities P = exp(S - m) / l with m the row
    max and l the row sum of exp(S - m): "Adaptive High-Performance Attention
    Kernels in CUDA", Advanced Production Features, 2. Custom CUDA Backward
    Pass (its S_ij and P_ij; the pages fix scale = 1/sqrt(d), here scale is an
    argument as in the library's C-ABI).
  * Causal masking keeps key index <= query index: "FlashAttention-2 MMA",
    Technical Details, Causal Masking.  Taken literally (top-left aligned), so
    query row i sees keys 0..i whatever Sq and Sk are.
  * The per-row log-sum-exp LSE_i = m_i + ln(l_i), natural log of the scaled
    scores (m and l as above).
  * Split-KV decoding: keys split into contiguous partitions, partial
    attention per partition, then a log-sum-exp weighted merge:
    "Adaptive High-Performance Attention Kernels in CUDA", Advanced Production
    Features, 1. Split-K FlashDecoding.  Each partial is kept normalised
    (O_s = sum_j exp(S_j - m_s) v_j / l_s) together with lse_s = m_s + ln l_s;
    the merge weights exp(lse_s - lse) equal the page's exp(m_s - m_global)
    scaled by l_s / l_global, so the result is the page's formula.

Everything is computed in float64 from the exact input values (fp16 inputs
are widened exactly).  One (b, h) slice is materialised at a time so large
inputs never need a full-size fp64 copy.
"""
from __future__ import annotations

import numpy as np


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    B, H, Sq, D = q.shape
    if k.shape[:2] != (B, H) or v.shape[:2] != (B, H):
        raise ValueError("batch/head mismatch")
    if k.shape[3] != D:
        raise ValueError("q and k head dims differ")
    if v.shape[2] != k.shape[2]:
        raise ValueError("k and v sequence lengths differ")
    if k.shape[2] < 1:
        raise ValueError("at least one key is required")
    return B, H, Sq, k.shape[2], D, v.shape[3]


def _scores(q2, k2, causal, scale):
    """S = scale * q2 @ k2^T for one slice; masked entries are -inf."""
    S = scale * (q2 @ k2.T)
    if causal:
        Sq, Sk = S.shape
        masked = np.arange(Sk)[None, :] > np.arange(Sq)[:, None]
        S[masked] = -np.inf
    return S


def _softmax_stats(S):
    """Row max m, E = exp(S - m), row sum l (masked entries give exp(-inf) = 0)."""
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    return m, E, l


def _lse(m, l):
    """Per-row log-sum-exp of the scaled scores, natural log."""
    return m + np.log(l)


def softmax_probs(q, k, causal, scale):
    """P = softmax(scale * q k^T + mask) for a single [Sq, D] x [Sk, D] slice."""
    S = _scores(_as64(q), _as64(k), causal, scale)
    m, E, l = _softmax_stats(S)
    return E / l


def attention(q, k, v, causal, scale):
    """O = softmax(scale * Q K^T + mask) V and LSE, both float64.

    q: [B, H, Sq, D]; k: [B, H, Sk, D]; v: [B, H, Sk, Dv].
    Returns O [B, H, Sq, Dv] and LSE [B, H, Sq].
    """
    B, H, Sq, Sk, D, Dv = _check_shapes(q, k, v)
    O = np.empty((B, H, Sq, Dv), dtype=np.float64)
    L = np.empty((B, H, Sq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            S = _scores(_as64(q[b, h]), _as64(k[b, h]), causal, scale)
            m, E, l = _softmax_stats(S)
            P = E / l
            O[b, h] = P @ _as64(v[b, h])
            L[b, h] = _lse(m, l)[:, 0]
    return O, L


def attention_rows(q, k, v, causal, scale, rows):
    """The definition evaluated for selected output rows only.

    rows: iterable of (b, h, i).  A causal row i is attention of query i over
    keys 0..min(i, Sk-1) without a mask.  Returns O [n, Dv] and LSE [n].
    """
    rows = list(rows)
    _check_shapes(q, k, v)
    Sk = k.shape[2]
    O = np.empty((len(rows), v.shape[3]), dtype=np.float64)
    L = np.empty(len(rows), dtype=np.float64)
    for n, (b, h, i) in enumerate(rows):
        keys = min(i + 1, Sk) if causal else Sk
        qi = _as64(q[b, h, i : i + 1])
        S = _scores(qi, _as64(k[b, h, :keys]), False, scale)
        m, E, l = _softmax_stats(S)
        O[n] = ((E / l) @ _as64(v[b, h, :keys]))[0]
        L[n] = _lse(m, l)[0, 0]
    return O, L


def split_bounds(Sk, num_splits):
    """Contiguous key partitions [c_s, c_{s+1}) with c_s = s * ceil(Sk / ns).

    The last partitions may be short or empty when ns does not divide Sk.
    """
    if num_splits < 1:
        raise ValueError("num_splits must be >= 1")
    chunk = -(-Sk // num_splits)
    return [(min(s * chunk, Sk), min((s + 1) * chunk, Sk)) for s in range(num_splits)]


def split_partials(q, k, v, scale, num_splits):
    """Phase one of split-KV decoding: per-partition normalised partial output
    O_s and lse_s (non-causal).  Empty partitions give O_s = 0, lse_s = -inf.

    Returns O_s [B, H, ns, Sq, Dv] and lse_s [B, H, ns, Sq].
    """
    B, H, Sq, Sk, D, Dv = _check_shapes(q, k, v)
    bounds = split_bounds(Sk, num_splits)
    Os = np.zeros((B, H, num_splits, Sq, Dv), dtype=np.float64)
    Ls = np.full((B, H, num_splits, Sq), -np.inf, dtype=np.float64)
    for s, (lo, hi) in enumerate(bounds):
        if hi > lo:
            o, l = attention(q, k[:, :, lo:hi], v[:, :, lo:hi], False, scale)
            Os[:, :, s] = o
            Ls[:, :, s] = l
    return Os, Ls


def merge_partials(Os, Ls):
    """Phase two: lse = ln sum_s exp(lse_s); O = sum_s exp(lse_s - lse) O_s.

    Os: [..., ns, Sq, Dv]; Ls: [..., ns, Sq].  Partitions with lse_s = -inf
    weigh zero.  Returns O [..., Sq, Dv], LSE [..., Sq].
    """
    Os = _as64(Os)
    Ls = _as64(Ls)
    mx = Ls.max(axis=-2, keepdims=True)
    w = np.exp(Ls - mx)
    tot = w.sum(axis=-2, keepdims=True)
    lse = _lse(mx, tot)
    O = (np.exp(Ls - lse)[..., None] * Os).sum(axis=-3)
    return O, lse[..., 0, :]


def decode_splitkv(q, k, v, scale, num_splits):
    """Split-KV decoding as the pages describe it: split, then merge."""
    Os, Ls = split_partials(q, k, v, scale, num_splits)
    return merge_partials(Os, Ls)
