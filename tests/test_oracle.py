"""Pins for the CPU fp64 oracle (no GPU).

The oracle is checked against things other than itself: hand-derived worked
examples (tests/golden/), closed forms, invariants of the definition, an
independent pure-Python brute force, and torch's scaled_dot_product_attention
in fp64 on the CPU (the routine the pages validate against).  The last test
plants plausible mistakes in the oracle and checks that some pin fails for
each of them.
"""
import glob
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import dense as oa
from workloads import WORKLOADS, make_qkv, sample_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape) * scale


# ---------------------------------------------------------------- pin suite
# Each pin raises AssertionError on failure.  They are run as tests below and
# again against deliberately broken copies of the oracle.

def pin_golden():
    files = sorted(glob.glob(os.path.join(GOLDEN, "*.json")))
    assert len(files) >= 5
    for f in files:
        g = json.load(open(f))
        q, k, v = (np.array(g[x], dtype=np.float64) for x in ("q", "k", "v"))
        if "num_splits" in g:
            Os, Ls = oracle.split_partials(q, k, v, g["scale"], g["num_splits"])
            np.testing.assert_allclose(Os, np.array(g["O_partials"]), atol=1e-12, err_msg=f)
            np.testing.assert_allclose(Ls, np.array(g["LSE_partials"]), atol=1e-12, err_msg=f)
            O, L = oracle.decode_splitkv(q, k, v, g["scale"], g["num_splits"])
        else:
            O, L = oracle.attention(q, k, v, g["causal"], g["scale"])
        np.testing.assert_allclose(O, np.array(g["O"]), rtol=1e-12, atol=1e-12, err_msg=f)
        np.testing.assert_allclose(L, np.array(g["LSE"]), rtol=1e-12, atol=1e-12, err_msg=f)


BRUTE_SHAPES = [
    # B, H, Sq, Sk, D, scale
    (1, 1, 1, 1, 1, 1.0),
    (2, 2, 5, 7, 4, 0.5),
    (1, 2, 9, 4, 3, 0.7),   # more queries than keys (causal rows past Sk see every key)
    (1, 1, 6, 11, 64, 0.125),
    (1, 1, 33, 33, 8, 0.35),
    (1, 1, 3, 5, 512, 0.05),     # the large head dims of the Split-D path
    (1, 1, 2, 3, 1024, 0.03125),
]


def pin_brute():
    for n, (B, H, Sq, Sk, D, sc) in enumerate(BRUTE_SHAPES):
        q = _rand((B, H, Sq, D), 10 + n)
        k = _rand((B, H, Sk, D), 20 + n)
        v = _rand((B, H, Sk, D + 1), 30 + n)  # Dv != D on purpose
        for causal in (False, True):
            O, L = oracle.attention(q, k, v, causal, sc)
            Ob, Lb = oracle.attention_brute(q.tolist(), k.tolist(), v.tolist(), causal, sc)
            np.testing.assert_allclose(O, np.array(Ob), atol=1e-10, rtol=0)
            np.testing.assert_allclose(L, np.array(Lb), atol=1e-10, rtol=0)


def pin_q_zero():
    Sq, Sk, D = 7, 10, 5
    q = np.zeros((1, 1, Sq, D))
    k = _rand((1, 1, Sk, D), 1)
    v = _rand((1, 1, Sk, D), 2)
    O, L = oracle.attention(q, k, v, False, 0.3)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(v[0, 0].mean(0), (Sq, D)), atol=1e-13)
    np.testing.assert_allclose(L, math.log(Sk), atol=1e-13)
    O, L = oracle.attention(q, k, v, True, 0.3)
    for i in range(Sq):
        np.testing.assert_allclose(O[0, 0, i], v[0, 0, : i + 1].mean(0), atol=1e-13)
        assert abs(L[0, 0, i] - math.log(i + 1)) < 1e-13


def pin_v_const():
    q = _rand((2, 1, 6, 4), 3)
    k = _rand((2, 1, 9, 4), 4)
    v = np.full((2, 1, 9, 3), -2.75)
    for causal in (False, True):
        O, _ = oracle.attention(q, k, v, causal, 0.9)
        np.testing.assert_allclose(O, -2.75, atol=1e-13)


def pin_single_key():
    q = _rand((1, 2, 5, 6), 5)
    k = _rand((1, 2, 1, 6), 6)
    v = _rand((1, 2, 1, 6), 7)
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, causal, 0.4)
        np.testing.assert_allclose(O, np.broadcast_to(v, O.shape), atol=1e-14)
        np.testing.assert_allclose(L, 0.4 * np.einsum("bhqd,bhkd->bhq", q, k), atol=1e-13)


def pin_causal_row0():
    q = _rand((1, 1, 8, 4), 8)
    k = _rand((1, 1, 8, 4), 9)
    v = _rand((1, 1, 8, 4), 10)
    O, L = oracle.attention(q, k, v, True, 0.6)
    np.testing.assert_allclose(O[0, 0, 0], v[0, 0, 0], atol=1e-14)
    assert abs(L[0, 0, 0] - 0.6 * float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-13


def pin_softmax_rows():
    q = _rand((12, 5), 11)
    k = _rand((12, 5), 12)
    for causal in (False, True):
        P = oracle.softmax_probs(q, k, causal, 0.8)
        np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-12)
        assert (P >= 0).all()
        if causal:
            assert (P[np.triu_indices(12, 1)] == 0).all()
            assert (P[np.tril_indices(12)] > 0).all()


def pin_split_merge():
    Sk = 100
    q = _rand((2, 3, 3, 8), 13)
    k = _rand((2, 3, Sk, 8), 14)
    v = _rand((2, 3, Sk, 8), 15)
    O, L = oracle.attention(q, k, v, False, 0.5)
    for ns in (1, 2, 3, 7, 64, 100):
        Om, Lm = oracle.decode_splitkv(q, k, v, 0.5, ns)
        np.testing.assert_allclose(Om, O, atol=1e-12, rtol=0)
        np.testing.assert_allclose(Lm, L, atol=1e-12, rtol=0)
    b = oracle.split_bounds(100, 64)
    assert b[0] == (0, 2) and b[49] == (98, 100) and b[50] == (100, 100) and b[63] == (100, 100)
    assert sum(hi - lo for lo, hi in b) == 100


def pin_key_shift():
    q = _rand((1, 2, 6, 5), 16)
    k = _rand((1, 2, 6, 5), 17)
    v = _rand((1, 2, 6, 5), 18)
    c = _rand((5,), 19)
    for causal in (False, True):
        O1, L1 = oracle.attention(q, k, v, causal, 0.7)
        O2, L2 = oracle.attention(q, k + c, v, causal, 0.7)
        np.testing.assert_allclose(O2, O1, atol=1e-12)
        np.testing.assert_allclose(L2, L1 + 0.7 * (q @ c), atol=1e-12)


def pin_permutation():
    q = _rand((1, 1, 5, 4), 20)
    k = _rand((1, 1, 9, 4), 21)
    v = _rand((1, 1, 9, 4), 22)
    perm = np.random.Generator(np.random.PCG64(23)).permutation(9)
    O1, L1 = oracle.attention(q, k, v, False, 1.1)
    O2, L2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], False, 1.1)
    np.testing.assert_allclose(O2, O1, atol=1e-13)
    np.testing.assert_allclose(L2, L1, atol=1e-13)


def pin_causal_truncation():
    q = _rand((1, 1, 7, 3), 24)
    k = _rand((1, 1, 7, 3), 25)
    v = _rand((1, 1, 7, 3), 26)
    O, L = oracle.attention(q, k, v, True, 0.9)
    for i in range(7):
        Oi, Li = oracle.attention_brute(q[:, :, i : i + 1].tolist(), k[:, :, : i + 1].tolist(), v[:, :, : i + 1].tolist(), False, 0.9)
        np.testing.assert_allclose(O[0, 0, i], Oi[0][0][0], atol=1e-13)
        assert abs(L[0, 0, i] - Li[0][0][0]) < 1e-13


def pin_sdpa():
    torch = pytest.importorskip("torch")
    for (B, H, S, D, sc) in [(2, 3, 17, 16, 0.25), (1, 2, 64, 64, 0.125), (1, 2, 19, 512, 0.05),
                             (1, 1, 11, 1024, 0.03125)]:
        q = _rand((B, H, S, D), 27)
        k = _rand((B, H, S, D), 28)
        v = _rand((B, H, S, D), 29)
        for causal in (False, True):
            O, _ = oracle.attention(q, k, v, causal, sc)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal, scale=sc
            ).numpy()
            np.testing.assert_allclose(O, ref, atol=1e-12, rtol=0)


PINS = [
    pin_golden,
    pin_brute,
    pin_q_zero,
    pin_v_const,
    pin_single_key,
    pin_causal_row0,
    pin_softmax_rows,
    pin_split_merge,
    pin_key_shift,
    pin_permutation,
    pin_causal_truncation,
    pin_sdpa,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# --------------------------------------------------------------- other checks

def test_attention_rows_match_full():
    q, k, v = make_qkv(1, 2, 40, 40, 16, 99)
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, causal, 0.25)
        rows = [(0, 0, 0), (0, 1, 17), (0, 1, 39), (0, 0, 23)]
        Or, Lr = oracle.attention_rows(q, k, v, causal, 0.25, rows)
        for n, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(Or[n], O[b, h, i], atol=1e-13)
            assert abs(Lr[n] - L[b, h, i]) < 1e-13


def test_inputs_recipe():
    w = WORKLOADS["tiny"]
    q, k, v = make_qkv(w.B, w.H, w.Sq, w.Sk, w.D, w.seed)
    q2, k2, v2 = make_qkv(w.B, w.H, w.Sq, w.Sk, w.D, w.seed)
    assert q.dtype == np.float16 and q.shape == (1, 2, 128, 64) and k.shape == (1, 2, 128, 64)
    assert np.array_equal(q, q2) and np.array_equal(k, k2) and np.array_equal(v, v2)
    allv = np.concatenate([q.ravel(), k.ravel(), v.ravel()]).astype(np.float64)
    assert abs(allv.mean()) < 0.02 and abs(allv.std() - 1.0) < 0.02
    # the chunked draw equals one whole-array draw of the same stream
    gen = np.random.Generator(np.random.PCG64(w.seed))
    whole = gen.standard_normal((1, 2, 128, 64), dtype=np.float32).astype(np.float16)
    assert np.array_equal(whole, q)
    assert len(sample_rows(WORKLOADS["llama7b_prefill"], 16)) == 20


# -------------------------------------------------- planted mistakes (mutants)

def _mut_no_scale(orig):
    return lambda q2, k2, causal, scale: orig(q2, k2, causal, 1.0)


def _mut_mask_reversed(orig):
    def f(q2, k2, causal, scale):
        S = scale * (q2 @ k2.T)
        if causal:
            Sq, Sk = S.shape
            S[np.arange(Sk)[None, :] < np.arange(Sq)[:, None]] = -np.inf
        return S
    return f


def _mut_mask_strict(orig):
    def f(q2, k2, causal, scale):
        S = scale * (q2 @ k2.T)
        if causal:
            Sq, Sk = S.shape
            S[np.arange(Sk)[None, :] >= np.arange(Sq)[:, None]] = -np.inf
        return S
    return f


def _mut_transposed(orig):
    def f(q2, k2, causal, scale):
        # S^T in place of S (only expressible when the shapes agree)
        S = scale * (k2 @ q2.T) if q2.shape == k2.shape else scale * (q2 @ k2.T)
        if causal:
            Sq, Sk = S.shape
            S[np.arange(Sk)[None, :] > np.arange(Sq)[:, None]] = -np.inf
        return S
    return f


def _mut_no_max(orig):
    def f(S):
        E = np.exp(S)
        return np.zeros((S.shape[0], 1)), E, E.sum(axis=1, keepdims=True)
    return f


def _mut_log2(orig):
    return lambda m, l: m + np.log2(l)


def _mut_lse_no_max(orig):
    return lambda m, l: np.log(l)


def _mut_merge_unnormalised(orig):
    def f(Os, Ls):
        mx = Ls.max(axis=-2, keepdims=True)
        w = np.exp(Ls - mx)
        O = (w[..., None] * Os).sum(axis=-3)
        return O, (mx + np.log(w.sum(axis=-2, keepdims=True)))[..., 0, :]
    return f


def _mut_merge_max_only(orig):
    def f(Os, Ls):
        mx = Ls.max(axis=-2, keepdims=True)
        w = np.exp(Ls - mx)
        lse = mx + np.log(w.sum(axis=-2, keepdims=True))
        O = (np.exp(Ls - lse)[..., None] * Os).sum(axis=-3)
        return O, mx[..., 0, :]
    return f


MUTANTS = [
    ("_scores", _mut_no_scale),
    ("_scores", _mut_mask_reversed),
    ("_scores", _mut_mask_strict),
    ("_scores", _mut_transposed),
    ("_softmax_stats", _mut_no_max),
    ("_lse", _mut_log2),
    ("_lse", _mut_lse_no_max),
    ("merge_partials", _mut_merge_unnormalised),
    ("merge_partials", _mut_merge_max_only),
]


@pytest.mark.parametrize("target,mutant", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(oa, target, mutant(getattr(oa, target)))
    failed = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {mutant.__name__}"
