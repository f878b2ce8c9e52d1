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


def decode_paged_brute(q, k_cache, v_cache, block_tables, seq_lens, scale):
    """Paged single-query decoding with scalar loops: token t of sequence b is
    read from page block_tables[b][t // block_size], row t % block_size; pages
    outside [0, num_blocks) are skipped, the context is clamped to the table's
    reach, and an empty context gives O = 0, LSE = -inf (the readings listed
    in ``paged.py``).  Returns nested lists [B][H][1][D] and [B][H][1]."""
    num_blocks = len(k_cache)
    block_size = len(k_cache[0][0])
    O_all, L_all = [], []
    for b in range(len(q)):
        reach = len(block_tables[b]) * block_size
        ctx = min(max(int(seq_lens[b]), 0), reach)
        O_b, L_b = [], []
        for h in range(len(q[b])):
            qv = q[b][h][0]
            scores = []
            for t in range(ctx):
                page = int(block_tables[b][t // block_size])
                if page < 0 or page >= num_blocks:
                    continue
                krow = k_cache[page][h][t % block_size]
                dot = 0.0
                for d in range(len(qv)):
                    dot += float(qv[d]) * float(krow[d])
                scores.append((page, t % block_size, scale * dot))
            Dv = len(v_cache[0][0][0])
            if not scores:
                O_b.append([[0.0] * Dv])
                L_b.append([-math.inf])
                continue
            mx = max(s for _, _, s in scores)
            den = 0.0
            row = [0.0] * Dv
            for page, r, s in scores:
                e = math.exp(s - mx)
                den += e
                vrow = v_cache[page][h][r]
                for d in range(Dv):
                    row[d] += e * float(vrow[d])
            O_b.append([[x / den for x in row]])
            L_b.append([mx + math.log(den)])
        O_all.append(O_b)
        L_all.append(L_b)
    return O_all, L_all


def attention_varlen_brute(q, k, v, cu_q, cu_k, causal, scale):
    """Packed variable-length attention with scalar loops over the flat
    token stream: query token cu_q[b] + i of head h attends to key tokens
    cu_k[b] + j (j <= i when causal) of the same head.  Inputs are nested
    lists [total][H][D] and well-formed cumulative lengths.  Returns O as
    nested lists [total_q][H][Dv] (None for rows no sequence covers) and LSE
    [H][total_q]; a sequence without keys gives O = 0, LSE = -inf."""
    total_q = len(q)
    H = len(q[0])
    Dv = len(v[0][0]) if len(v) else 0
    O = [[None] * H for _ in range(total_q)]
    L = [[None] * total_q for _ in range(H)]
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        for i in range(q1 - q0):
            for h in range(H):
                scores = []
                for j in range(k1 - k0):
                    if causal and j > i:
                        continue
                    dot = 0.0
                    for d in range(len(q[q0 + i][h])):
                        dot += float(q[q0 + i][h][d]) * float(k[k0 + j][h][d])
                    scores.append((j, scale * dot))
                if not scores:
                    O[q0 + i][h] = [0.0] * Dv
                    L[h][q0 + i] = -math.inf
                    continue
                mx = max(s for _, s in scores)
                den = 0.0
                row = [0.0] * Dv
                for j, s in scores:
                    e = math.exp(s - mx)
                    den += e
                    for d in range(Dv):
                        row[d] += e * float(v[k0 + j][h][d])
                O[q0 + i][h] = [x / den for x in row]
                L[h][q0 + i] = mx + math.log(den)
    return O, L
