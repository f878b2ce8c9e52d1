"""GPU check of fa_decode_splitkv_noalloc, the allocation-free split decode
(its partials in the library's static scratch array), through the C ABI:
its output must equal fa_decode_splitkv's (same split count, so the same
kernels and bit-identical results) and the CPU fp64 oracle's within the
decode bar (max |dO| <= 2e-3, max |dLSE| <= 1e-3), on two calls in a row,
the second with a smaller input, so the second reads no stale partial of
the first."""
import math

import numpy as np
import pytest

import oracle
from workloads import make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    import exact_attention_54_amd as fa
    from exact_attention_54_amd import _capi

    assert torch.cuda.is_available(), "GPU tests need a GPU (the HIP library has no CPU path)"
    return torch, torch.device("cuda:0"), fa, _capi.load()


def noalloc(env, qd, kd, vd, ns, scale):
    torch, dev, fa, lib = env
    B, H, _, D = qd.shape
    Sk = kd.shape[2]
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, 1), float("nan"), dtype=torch.float32, device=dev)
    st = lib.fa_decode_splitkv_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                       B, H, 1, Sk, D, 0, scale, torch.cuda.current_stream().cuda_stream, ns)
    assert st == 0, fa.fa_last_error()
    return o, lse


# (B, H, Sk, D, num_splits): a large split call, then a smaller one
CASES = [(2, 8, 5000, 128, 16), (1, 3, 700, 64, 5)]


def test_noalloc_matches_split_decode_on_two_calls(env):
    torch, dev, fa, lib = env
    for i, (B, H, Sk, D, ns) in enumerate(CASES):
        print(f"noalloc call {i}: B={B} H={H} Sk={Sk} D={D} ns={ns}", flush=True)
        q, k, v = make_qkv(B, H, 1, Sk, D, seed=500 + i)
        qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
        scale = 1.0 / math.sqrt(D)
        o, lse = noalloc(env, qd, kd, vd, ns, scale)
        o_ref, lse_ref = fa.fa_decode_splitkv(qd, kd, vd, scale=scale, num_splits=ns)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), f"call {i}: differs from fa_decode_splitkv"
        O, L = oracle.attention(q, k, v, False, scale)
        eo = float(np.abs(o.float().cpu().numpy() - O).max())
        el = float(np.abs(lse.cpu().numpy() - L).max())
        print(f"noalloc call {i}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
        assert eo <= 2e-3 and el <= 1e-3


def test_noalloc_automatic_split_count(env):
    # ns = 0: the library's choice (many partitions at batch 1, 32K keys)
    torch, dev, fa, lib = env
    B, H, Sk, D = 1, 8, 32768, 128
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    assert fa.fa_decode_auto_splits(B, H, Sk, cus) > 1
    q, k, v = make_qkv(B, H, 1, Sk, D, seed=520)
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    o, lse = noalloc(env, qd, kd, vd, 0, 0.1)
    o_ref, lse_ref = fa.fa_decode_splitkv(qd, kd, vd, scale=0.1, num_splits=0)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
