"""GPU parity of fa_fwd on seeded random shapes against the CPU fp64 oracle.

Forty shapes drawn from one seed: D in {32, 64, 128, 256}, one to four
(batch, head) slices, query and key lengths up to 1500 (ragged), both mask
settings.  Grids this small are the ones fa_fwd gives a key-range split,
so the draw covers many (split start, parts) plans next to unsplit ones;
each case prints its plan.  Bar as for every prefill: max |dO| <= 2e-3,
max |dLSE| <= 1e-3.
"""
import math

import numpy as np
import pytest

import oracle
from workloads import make_qkv

pytestmark = pytest.mark.gpu

O_TOL = 2e-3
LSE_TOL = 1e-3


def draw_shapes(n, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    shapes = []
    for _ in range(n):
        D = int(g.choice([32, 64, 128, 256]))
        B = int(g.integers(1, 3))
        H = int(g.integers(1, 3))
        Sq = int(g.integers(1, 1501))
        Sk = Sq if g.random() < 0.5 else int(g.integers(1, 1501))
        causal = bool(g.random() < 0.6)
        shapes.append((B, H, Sq, Sk, D, causal))
    return shapes


SHAPES = draw_shapes(40, 2024)


@pytest.fixture(scope="module")
def env():
    import torch

    import exact_attention_54_amd as fa

    assert torch.cuda.is_available(), "GPU tests need a GPU (the HIP library has no CPU path)"
    dev = torch.device("cuda:0")
    return torch, dev, fa, torch.cuda.get_device_properties(dev).multi_processor_count


@pytest.mark.parametrize("shape", SHAPES, ids=["x".join(map(str, s)) for s in SHAPES])
def test_random_shape(env, shape):
    torch, dev, fa, cus = env
    B, H, Sq, Sk, D, causal = shape
    q, k, v = make_qkv(B, H, Sq, Sk, D, seed=3000 + Sq + 7 * Sk + D)
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    O, L = oracle.attention(q, k, v, causal, scale)
    parts = fa.fa_fwd_key_splits(B, H, Sq, Sk, D, causal, cus)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    eo = float(np.abs(o - O).max())
    el = float(np.abs(lse - L).max())
    print(f"{shape} key parts {parts}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= O_TOL and el <= LSE_TOL
