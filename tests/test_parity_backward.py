"""GPU parity of the backward pass (fa_bwd) against the CPU fp64 oracle.

The GPU pass takes o and lse from the GPU forward and the fp16 dO; the
oracle differentiates the definition in fp64 from the same fp16 q, k, v, dO.
Bar, per gradient tensor G with oracle value R:
    max |G - R| <= 2e-3 + 4e-3 * max |R|
Every output is rounded to fp16 (relative 2^-12 of the entry), and fp16 P
and dS enter the products with relative rounding 2^-11 each, so an entry's
error is a few 2^-11 of the largest terms it sums.  4e-3 = 8 * 2^-11 of the
tensor's largest entry, about 4x the worst seen (9.3e-4); 2e-3 covers
entries near zero, as the forward's O tolerance does.
"""
import numpy as np
import pytest

import oracle
from workloads import make_qkv

pytestmark = pytest.mark.gpu

ATOL = 2e-3
RTOL = 4e-3


@pytest.fixture(scope="module")
def torch_dev():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU (the HIP library has no CPU path)"
    return torch, torch.device("cuda:0")


@pytest.fixture(scope="module")
def fa():
    import exact_attention_54_amd as m

    return m


def run_bwd(torch_dev, fa, q, k, v, do, causal, scale):
    torch, dev = torch_dev
    qd, kd, vd, dod = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return [x.float().cpu().numpy() for x in (dq, dk, dv)]


def check(got, ref, what):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.isfinite(g).all(), f"{what} {name}: non-finite"
        err = float(np.abs(g - r).max())
        scale = float(np.abs(r).max())
        print(f"{what} {name}: max|err|={err:.3e} max|ref|={scale:.3e} rel={err / max(scale, 1e-30):.2e}", flush=True)
        assert err <= ATOL + RTOL * scale, f"{what} {name}: max|err| {err:.3e} vs max|ref| {scale:.3e}"


SHAPES = [
    # B, H, Sq, Sk
    (1, 2, 128, 128),
    (1, 3, 200, 333),
    (2, 1, 77, 77),
    (1, 2, 129, 65),
    (1, 1, 1, 1),
    (1, 1, 257, 257),
    (1, 2, 300, 100),
    (1, 1, 100, 300),
    (2, 2, 512, 512),
]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("shape", SHAPES, ids=["x".join(map(str, s)) for s in SHAPES])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_parity(torch_dev, fa, D, shape, causal):
    B, H, Sq, Sk = shape
    q, k, v = make_qkv(B, H, Sq, Sk, D, 700 + Sq + D)
    do = make_qkv(B, H, Sq, 1, D, 800 + Sq)[0]
    scale = 1.0 / np.sqrt(D)
    got = run_bwd(torch_dev, fa, q, k, v, do, causal, scale)
    ref = oracle.attention_backward(q, k, v, do, causal, scale)
    check(got, ref, f"bwd D={D} {shape} causal={causal}")


def test_backward_llama_shape_two_heads(torch_dev, fa):
    # the full (1, 32, 4096, 4096, 128) causal backward, checked on heads 0 and 31
    B, H, S, D = 1, 32, 4096, 128
    q, k, v = make_qkv(B, H, S, S, D, 3)
    do = make_qkv(B, H, S, 1, D, 13)[0]
    scale = 1.0 / np.sqrt(D)
    dq, dk, dv = run_bwd(torch_dev, fa, q, k, v, do, True, scale)
    for h in (0, 31):
        sl = slice(h, h + 1)
        ref = oracle.attention_backward(q[:, sl], k[:, sl], v[:, sl], do[:, sl], True, scale)
        check([dq[:, sl], dk[:, sl], dv[:, sl]], ref, f"llama head {h}")


def test_backward_bitwise_repeatable(torch_dev, fa):
    torch, dev = torch_dev
    q, k, v = make_qkv(1, 4, 300, 300, 128, 71)
    do = make_qkv(1, 4, 300, 1, 128, 72)[0]
    a = run_bwd(torch_dev, fa, q, k, v, do, True, 0.1)
    b = run_bwd(torch_dev, fa, q, k, v, do, True, 0.1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_errors_raise(torch_dev, fa):
    torch, dev = torch_dev
    q = torch.zeros((1, 1, 8, 256), dtype=torch.float16, device=dev)
    o, lse = fa.fa_fwd(q, q, q)
    with pytest.raises(fa.FAError) as e:
        fa.fa_bwd(q, q, q, o, lse, q)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
