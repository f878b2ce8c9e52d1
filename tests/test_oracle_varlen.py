"""Pins for the packed variable-length oracle (no GPU).

``oracle.varlen.attention_varlen`` cuts each sequence out of the packed
[total, H, D] stream and applies the dense definition.  It is pinned
against:
  * an independent scalar-loop evaluation over the flat token stream
    (``oracle.brute.attention_varlen_brute``), with unequal query and key
    lengths, empty sequences and both mask settings;
  * the already-pinned dense oracle when every sequence has one length
    (packing is then a transpose of [B, H, S, D]);
  * independence of sequences, and the clamps of untrusted cumulative
    lengths.
The last test plants plausible mistakes and checks that a pin catches each.
"""
import numpy as np
import pytest

import oracle
from oracle import dense as od
from oracle import varlen as ov
from workloads import make_qkv, make_varlen


def _nested(x):
    return np.asarray(x, dtype=np.float64).tolist()


# ---------------------------------------------------------------- pin suite

def pin_brute():
    cases = [
        # lengths_q, lengths_k, H, D
        ([5, 1, 7], None, 2, 4),
        ([3, 6, 2], [4, 6, 9], 3, 3),    # cross attention, Lq != Lk
        ([4, 0, 5], [4, 3, 0], 2, 5),    # an empty query sequence and a sequence without keys
    ]
    for n, (lq, lk, H, D) in enumerate(cases):
        q, k, v, cu_q, cu_k = make_varlen(lq, H, D, 200 + n, lengths_k=lk)
        for causal in (False, True):
            O, L = ov.attention_varlen(q, k, v, cu_q, cu_k, causal, 0.45)
            Ob, Lb = oracle.attention_varlen_brute(_nested(q), _nested(k), _nested(v), cu_q.tolist(),
                                                   cu_k.tolist(), causal, 0.45)
            Ob = np.array([[np.nan] * D if r is None else r for row in Ob for r in row]).reshape(O.shape)
            Lb = np.array([[np.nan if x is None else x for x in row] for row in Lb])
            np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-12)
            assert np.array_equal(np.isneginf(L), np.isneginf(Lb))
            fin = np.isfinite(L)
            np.testing.assert_allclose(L[fin], Lb[fin], rtol=1e-12, atol=1e-12)


def pin_equal_lengths_are_dense():
    B, H, S, D = 3, 4, 9, 8
    q, k, v = make_qkv(B, H, S, S, D, 300)
    pack = lambda x: np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)).reshape(B * S, H, D))
    cu = np.arange(0, (B + 1) * S, S, dtype=np.int32)
    for causal in (False, True):
        O, L = ov.attention_varlen(pack(q), pack(k), pack(v), cu, cu, causal, 0.3)
        Od, Ld = od.attention(q, k, v, causal, 0.3)
        np.testing.assert_allclose(O, pack(Od), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(L, np.transpose(Ld, (1, 0, 2)).reshape(H, B * S), rtol=1e-12, atol=1e-12)


def pin_sequences_independent():
    q, k, v, cu_q, cu_k = make_varlen([6, 9, 4], 2, 4, 301)
    O1, L1 = ov.attention_varlen(q, k, v, cu_q, cu_k, True, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[cu_k[1] : cu_k[2]] = 7.0   # change sequence 1 only
    v2[cu_k[1] : cu_k[2]] = -3.0
    O2, L2 = ov.attention_varlen(q, k2, v2, cu_q, cu_k, True, 0.5)
    for b in (0, 2):
        np.testing.assert_array_equal(O1[cu_q[b] : cu_q[b + 1]], O2[cu_q[b] : cu_q[b + 1]])
        np.testing.assert_array_equal(L1[:, cu_q[b] : cu_q[b + 1]], L2[:, cu_q[b] : cu_q[b + 1]])
    assert not np.array_equal(O1[cu_q[1] : cu_q[2]], O2[cu_q[1] : cu_q[2]])


def pin_clamps():
    q, k, v, cu_q, cu_k = make_varlen([5, 4], 2, 4, 302)
    O, L = ov.attention_varlen(q, k, v, cu_q, cu_k, False, 0.5)
    # a start below 0 is 0, an end past the tensor is the tensor's end
    Oc, Lc = ov.attention_varlen(q, k, v, np.array([-3, 5, 99]), np.array([-1, 5, 1000]), False, 0.5)
    np.testing.assert_array_equal(O, Oc)
    np.testing.assert_array_equal(L, Lc)
    # max_q cuts each sequence's query rows (the rest is not produced)
    Om, Lm = ov.attention_varlen(q, k, v, cu_q, cu_k, False, 0.5, max_q=3)
    np.testing.assert_array_equal(Om[0:3], O[0:3])
    assert np.isnan(Om[3:5]).all() and np.isnan(Lm[:, 3:5]).all()
    np.testing.assert_array_equal(Om[5:8], O[5:8])
    # a sequence without keys: O = 0, LSE = -inf
    Oe, Le = ov.attention_varlen(q, k, v, cu_q, np.array([0, 0, 4]), False, 0.5)
    assert (Oe[0:5] == 0).all() and np.isneginf(Le[:, 0:5]).all()


PINS = [pin_brute, pin_equal_lengths_are_dense, pin_sequences_independent, pin_clamps]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def test_varlen_recipe():
    q, k, v, cu_q, cu_k = make_varlen([3, 5], 2, 4, 9)
    assert q.shape == (8, 2, 4) and q.dtype == np.float16 and cu_q.tolist() == [0, 3, 8]
    assert np.array_equal(cu_q, cu_k)
    gen = np.random.Generator(np.random.PCG64(9))
    assert np.array_equal(gen.standard_normal((8, 2, 4), dtype=np.float32).astype(np.float16), q)


# -------------------------------------------------- planted mistakes (mutants)

def _mut_causal_bottom_right(orig):
    # key j visible to query i when j <= i + (lk - lq)
    def f(q, k, v, cu_q, cu_k, causal, scale, max_q=None, max_k=None):
        if not causal:
            return orig(q, k, v, cu_q, cu_k, causal, scale, max_q, max_k)
        total_q, H, D = q.shape
        O = np.full((total_q, H, v.shape[2]), np.nan)
        L = np.full((H, total_q), np.nan)
        for b in range(len(cu_q) - 1):
            sq, lq = ov.sequence_bounds(cu_q, b, total_q, total_q)
            sk, lk = ov.sequence_bounds(cu_k, b, k.shape[0], k.shape[0])
            for i in range(lq):
                n = min(lk, i + 1 + (lk - lq))
                if n <= 0:
                    O[sq + i] = 0
                    L[:, sq + i] = -np.inf
                    continue
                qb = np.transpose(q[sq + i : sq + i + 1], (1, 0, 2))[None]
                kb = np.transpose(k[sk : sk + n], (1, 0, 2))[None]
                vb = np.transpose(v[sk : sk + n], (1, 0, 2))[None]
                o, lse = od.attention(qb, kb, vb, False, scale)
                O[sq + i] = o[0, :, 0]
                L[:, sq + i] = lse[0, :, 0]
        return O, L
    return f


def _mut_end_off_by_one(orig):
    def f(cu, b, total, max_len):
        start, length = orig(cu, b, total, max_len)
        return start, max(length - 1, 0)
    return f


def _mut_head_major_packing(orig):
    # reads the stream as [H, total, D] instead of [total, H, D]
    def f(q, k, v, cu_q, cu_k, causal, scale, max_q=None, max_k=None):
        re = lambda x: np.ascontiguousarray(x.reshape(x.shape[1], x.shape[0], x.shape[2]).transpose(1, 0, 2))
        return orig(re(q), re(k), re(v), cu_q, cu_k, causal, scale, max_q, max_k)
    return f


MUTANTS = [
    ("attention_varlen", _mut_causal_bottom_right),
    ("sequence_bounds", _mut_end_off_by_one),
    ("attention_varlen", _mut_head_major_packing),
]


@pytest.mark.parametrize("target,mutant", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(ov, target, mutant(getattr(ov, target)))
    failed = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {mutant.__name__}"
