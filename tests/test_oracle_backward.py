"""Pins for the backward oracle (no GPU).

``oracle.backward.attention_backward`` writes out the pages' backward
formulas.  It is pinned against:
  * torch autograd through ``scaled_dot_product_attention`` in fp64 on the
    CPU (a library routine computing the same gradients independently);
  * central finite differences of sum(O * dO) on tiny inputs (the
    definition of a gradient, no formula involved);
  * closed forms: one key -> dQ = dK = 0 and dV = sum of dO rows; constant
    V -> dQ = dK = 0; and rows of dS summing to zero, seen as
    sum_j dK_j = scale * sum_i (sum_j dS_ij) q_i = 0 for every column.
The last test plants plausible mistakes and checks that a pin catches each.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as ob
from oracle import dense as od
from workloads import make_qkv


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


# ---------------------------------------------------------------- pin suite

def pin_autograd():
    import torch

    for (B, H, Sq, Sk, D, causal, seed) in [(1, 2, 7, 9, 8, False, 1), (2, 1, 11, 11, 16, True, 2),
                                            (1, 1, 13, 5, 4, True, 3)]:
        q, k, v = make_qkv(B, H, Sq, Sk, D, seed)
        do = _rand((B, H, Sq, D), seed + 50)
        scale = 0.37
        tq, tk, tv = (torch.tensor(x.astype(np.float64), requires_grad=True) for x in (q, k, v))
        mask = None
        if causal:
            mask = torch.ones(Sq, Sk, dtype=torch.bool).tril()
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
        out.backward(torch.tensor(do))
        dQ, dK, dV = ob.attention_backward(q, k, v, do, causal, scale)
        np.testing.assert_allclose(dQ, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dK, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def pin_finite_differences():
    B, H, Sq, Sk, D = 1, 1, 4, 5, 3
    q, k, v = (x.astype(np.float64) for x in make_qkv(B, H, Sq, Sk, D, 9))
    do = _rand((B, H, Sq, D), 10)
    for causal in (False, True):
        dQ, dK, dV = ob.attention_backward(q, k, v, do, causal, 0.6)
        f = lambda qq, kk, vv: float(np.sum(od.attention(qq, kk, vv, causal, 0.6)[0] * do))
        eps = 1e-6
        for grad, which in ((dQ, 0), (dK, 1), (dV, 2)):
            base = [q, k, v]
            num = np.zeros_like(base[which])
            for idx in np.ndindex(base[which].shape):
                plus = [x.copy() for x in base]
                minus = [x.copy() for x in base]
                plus[which][idx] += eps
                minus[which][idx] -= eps
                num[idx] = (f(*plus) - f(*minus)) / (2 * eps)
            np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


def pin_closed_forms():
    q, k, v = make_qkv(1, 2, 6, 1, 4, 11)
    do = _rand((1, 2, 6, 4), 12)
    dQ, dK, dV = ob.attention_backward(q, k, v, do, False, 0.5)
    assert np.abs(dQ).max() < 1e-12 and np.abs(dK).max() < 1e-12
    np.testing.assert_allclose(dV[:, :, 0], do.sum(axis=2), rtol=1e-12, atol=1e-12)
    q, k, _ = make_qkv(1, 1, 5, 7, 4, 13)
    v = np.full((1, 1, 7, 4), 0.75)
    for causal in (False, True):
        dQ, dK, _ = ob.attention_backward(q, k, v, _rand((1, 1, 5, 4), 14), causal, 0.5)
        assert np.abs(dQ).max() < 1e-12 and np.abs(dK).max() < 1e-12
    # rows of dS sum to zero -> the key gradients sum to zero
    q, k, v = make_qkv(2, 2, 8, 9, 5, 15)
    for causal in (False, True):
        _, dK, _ = ob.attention_backward(q, k, v, _rand((2, 2, 8, 5), 16), causal, 0.3)
        assert np.abs(dK.sum(axis=2)).max() < 1e-10


PINS = [pin_autograd, pin_finite_differences, pin_closed_forms]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# -------------------------------------------------- planted mistakes (mutants)

def _mut_no_row_constant(orig):
    # dS = P dP (forgets D)
    def f(q, k, v, do, causal, scale):
        B, H, Sq, Sk, D, Dv = od._check_shapes(q, k, v)
        dQ, dK, dV = orig(q, k, v, do, causal, scale)
        for b in range(B):
            for h in range(H):
                S = od._scores(np.asarray(q[b, h], float), np.asarray(k[b, h], float), causal, scale)
                m, E, l = od._softmax_stats(S)
                P = E / l
                dS = P * (np.asarray(do[b, h], float) @ np.asarray(v[b, h], float).T)
                dQ[b, h] = scale * dS @ np.asarray(k[b, h], float)
                dK[b, h] = scale * dS.T @ np.asarray(q[b, h], float)
        return dQ, dK, dV
    return f


def _mut_no_scale(orig):
    return lambda q, k, v, do, causal, scale: tuple(
        x / s for x, s in zip(orig(q, k, v, do, causal, scale), (scale, scale, 1.0)))


def _mut_dv_untransposed(orig):
    def f(q, k, v, do, causal, scale):
        dQ, dK, dV = orig(q, k, v, do, causal, scale)
        if dV.shape[2] == do.shape[2]:
            B, H = q.shape[:2]
            for b in range(B):
                for h in range(H):
                    S = od._scores(np.asarray(q[b, h], float), np.asarray(k[b, h], float), causal, scale)
                    m, E, l = od._softmax_stats(S)
                    dV[b, h] = (E / l) @ np.asarray(do[b, h], float)
        return dQ, dK, dV
    return f


MUTANTS = [
    ("attention_backward", _mut_no_row_constant),
    ("attention_backward", _mut_no_scale),
    ("attention_backward", _mut_dv_untransposed),
]


@pytest.mark.parametrize("target,mutant", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(ob, target, mutant(getattr(ob, target)))
    failed = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {mutant.__name__}"
