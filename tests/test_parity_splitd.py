"""GPU parity of the Split-D forward (fa_fwd with D = 512 and 1024) against
the CPU fp64 oracle.

Same bar as the other forward tests: max |O - O_oracle| <= 2e-3 and
max |LSE - LSE_oracle| <= 1e-3.  The "Large Head" (1, 8, 1024, 1024, 512)
and "Massive Head" (1, 4, 512, 512, 1024) workloads are checked on every
element under both masks; ragged shapes hit a single key, partial query and
key tiles, more queries than keys and the reverse; closed forms (a zero query
averages V, causal row 0 is V[0]) and a wide score spread that forces the
running-max rescale on most tiles complete the set.
"""
import math

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, make_qkv, workload_inputs

pytestmark = pytest.mark.gpu

O_TOL = 2e-3
LSE_TOL = 1e-3


@pytest.fixture(scope="module")
def torch_dev():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU (the HIP library has no CPU path)"
    return torch, torch.device("cuda:0")


@pytest.fixture(scope="module")
def fa():
    import exact_attention_54_amd as m

    return m


def gpu_fwd(torch_dev, fa, q, k, v, causal, scale):
    torch, dev = torch_dev
    qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def assert_close(o, lse, O, L, what):
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{what}: non-finite output"
    eo = float(np.abs(o - O).max())
    el = float(np.abs(lse - L).max())
    print(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= O_TOL, f"{what}: max|dO| = {eo:.3e}"
    assert el <= LSE_TOL, f"{what}: max|dLSE| = {el:.3e}"


@pytest.mark.parametrize("name", ["d512_prefill", "d1024_prefill"])
@pytest.mark.parametrize("causal", [False, True])
def test_large_head_workload_full(torch_dev, fa, name, causal):
    w = WORKLOADS[name]
    q, k, v = workload_inputs(w)
    o, lse = gpu_fwd(torch_dev, fa, q, k, v, causal, w.scale)
    O, L = oracle.attention(q, k, v, causal, w.scale)
    assert_close(o, lse, O, L, f"{name} causal={causal}")


RAGGED = [
    # B, H, Sq, Sk
    (1, 1, 1, 1),
    (1, 2, 33, 65),
    (2, 1, 100, 77),
    (1, 1, 257, 129),
    (1, 1, 300, 100),   # more queries than keys
    (1, 1, 100, 300),
    (1, 1, 31, 1000),
]


@pytest.mark.parametrize("D", [512, 1024])
@pytest.mark.parametrize("shape", RAGGED, ids=["x".join(map(str, s)) for s in RAGGED])
@pytest.mark.parametrize("causal", [False, True])
def test_large_head_ragged(torch_dev, fa, D, shape, causal):
    B, H, Sq, Sk = shape
    q, k, v = make_qkv(B, H, Sq, Sk, D, seed=3000 + Sq + 7 * Sk + D)
    scale = 1.0 / math.sqrt(D)
    o, lse = gpu_fwd(torch_dev, fa, q, k, v, causal, scale)
    O, L = oracle.attention(q, k, v, causal, scale)
    assert_close(o, lse, O, L, f"D={D} {shape} causal={causal}")


@pytest.mark.parametrize("D", [512, 1024])
def test_large_head_closed_forms(torch_dev, fa, D):
    B, H, S = 1, 2, 150
    _, k, v = make_qkv(B, H, S, S, D, seed=31)
    q0 = np.zeros((B, H, S, D), np.float16)
    o, lse = gpu_fwd(torch_dev, fa, q0, k, v, False, 0.125)
    vm = v.astype(np.float64).mean(axis=2, keepdims=True)
    assert np.abs(o - vm).max() <= O_TOL and np.abs(lse - math.log(S)).max() <= LSE_TOL
    o, lse = gpu_fwd(torch_dev, fa, q0, k, v, True, 0.125)
    cm = np.cumsum(v.astype(np.float64), axis=2) / np.arange(1, S + 1)[None, None, :, None]
    assert np.abs(o - cm).max() <= O_TOL
    assert np.abs(lse - np.log(np.arange(1, S + 1))[None, None, :]).max() <= LSE_TOL
    q, _, _ = make_qkv(B, H, S, S, D, seed=32)
    o, _ = gpu_fwd(torch_dev, fa, q, k, v, True, 1.0 / math.sqrt(D))
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0].astype(np.float32))


@pytest.mark.parametrize("D", [512, 1024])
def test_large_head_wide_scores(torch_dev, fa, D):
    # scale 0.2 on D >= 512 unit-normal rows: scores spread over tens of
    # units, so the running max moves on most key tiles
    q, k, v = make_qkv(1, 2, 200, 260, D, seed=33)
    for causal in (False, True):
        o, lse = gpu_fwd(torch_dev, fa, q, k, v, causal, 0.2)
        O, L = oracle.attention(q, k, v, causal, 0.2)
        assert_close(o, lse, O, L, f"D={D} scale=0.2 causal={causal}")


def test_large_head_bitwise_repeatable(torch_dev, fa):
    q, k, v = make_qkv(1, 3, 200, 300, 512, seed=34)
    a = gpu_fwd(torch_dev, fa, q, k, v, True, 0.05)
    b = gpu_fwd(torch_dev, fa, q, k, v, True, 0.05)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
