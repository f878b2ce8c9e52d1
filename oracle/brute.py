"""Pure-Python scalar attention for tiny inputs -- test infrastructure only.

A second, independent evaluation of the same definition as ``dense.py``
(scaled scores, causal rule key <= query, softmax by exp(s - max) / sum,
LSE = max + ln(sum); see that module's header for the passages), written
with explicit loops over queries, keys and the head dimension and Python
floats (IEEE double), no numpy arithmetic.  Used to pin the numpy oracle.
"""
from __future__ import annotations

import math


def attention_brute(q, k, v, causal, scale):
    """q, k, v: nested lists or arrays [B][H][S][D].  Returns (O, LSE) as
    nested Python lists [B][H][Sq][Dv] and [B][H][Sq]."""
    B = len(q)
    O_all, L_all = [], []
    for b in range(B):
        O_b, L_b = [], []
        for h in range(len(q[b])):
            qs, ks, vs = q[b][h], k[b][h], v[b][h]
            Sk = len(ks)
            O_h, L_h = [], []
            for i in range(len(qs)):
                scores = []
                for j in range(Sk):
                    if causal and j > i:
                        continue
                    dot = 0.0
                    for d in range(len(qs[i])):
                        dot += float(qs[i][d]) * float(ks[j][d])
                    scores.append((j, scale * dot))
                mx = -math.inf
                for _, s in scores:
                    if s > mx:
                        mx = s
                den = 0.0
                weights = []
                for j, s in scores:
                    e = math.exp(s - mx)
                    weights.append((j, e))
                    den += e
                Dv = len(vs[0])
                row = [0.0] * Dv
                for j, e in weights:
                    for d in range(Dv):
                        row[d] += e * float(vs[j][d])
                O_h.append([x / den for x in row])
                L_h.append(mx + math.log(den))
            O_b.append(O_h)
            L_b.append(L_h)
        O_all.append(O_b)
        L_all.append(L_b)
    return O_all, L_all
