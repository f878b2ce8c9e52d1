"""Gradients of exact attention, fp64 -- test infrastructure only (see package doc).

Definition followed
  * The backward pass of "Adaptive High-Performance Attention Kernels in
    CUDA", Advanced Production Features, 2. Custom CUDA Backward Pass:
    scores S and probabilities P of the forward are recomputed, the row
    constant D_i = sum_k dO_ik O_ik is formed, and dS_ij = P_ij (dP_ij - D_i)
    with dP = dO V^T; nothing but m, l (here LSE) is kept from the forward.
  * With O = P V and S = scale * Q K^T (masked entries -inf, P = 0 there):
        dV = P^T dO,   dQ = scale * dS K,   dK = scale * dS^T Q.
    These are the chain rule through O = softmax(S) V, written out.

Everything is fp64 from the exact input values, one (b, h) slice at a time;
P comes from ``dense``'s score and softmax steps (the definition), not from
any stored forward statistics.
"""
from __future__ import annotations

import numpy as np

from . import dense


def attention_backward(q, k, v, do, causal, scale):
    """(dQ, dK, dV) of O = softmax(scale Q K^T + mask) V for upstream dO.

    q: [B, H, Sq, D]; k, v: [B, H, Sk, D]; do: [B, H, Sq, D].  All float64 out.
    """
    B, H, Sq, Sk, D, Dv = dense._check_shapes(q, k, v)
    dQ = np.empty((B, H, Sq, D), dtype=np.float64)
    dK = np.empty((B, H, Sk, D), dtype=np.float64)
    dV = np.empty((B, H, Sk, Dv), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            q2 = np.asarray(q[b, h], dtype=np.float64)
            k2 = np.asarray(k[b, h], dtype=np.float64)
            v2 = np.asarray(v[b, h], dtype=np.float64)
            do2 = np.asarray(do[b, h], dtype=np.float64)
            S = dense._scores(q2, k2, causal, scale)
            m, E, l = dense._softmax_stats(S)
            P = E / l
            O = P @ v2
            Dr = np.sum(do2 * O, axis=1, keepdims=True)   # D_i = dO_i . O_i
            dP = do2 @ v2.T
            dS = P * (dP - Dr)
            dV[b, h] = P.T @ do2
            dQ[b, h] = scale * (dS @ k2)
            dK[b, h] = scale * (dS.T @ q2)
    return dQ, dK, dV
