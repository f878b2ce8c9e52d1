"""GPU parity at long key ranges: a million-key decode and a 256K-key prefill.

Same bar as the other forward tests (max |O - O_oracle| <= 2e-3, max
|LSE - LSE_oracle| <= 1e-3).  These sizes stress what short tests cannot:
fp32 row sums over 2^20 keys, thousands of key tiles with the lazy
reference max, 32-bit byte offsets within a 512 MiB slice, and the decode's
partitioning when one (batch, head) holds a million keys.
"""
import numpy as np
import pytest

import oracle
from workloads import make_qkv

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


def check(o, lse, O, L, what):
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{what}: non-finite output"
    eo = float(np.abs(o - O).max())
    el = float(np.abs(lse - L).max())
    print(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= O_TOL and el <= LSE_TOL, f"{what}: {eo:.3e} {el:.3e}"


@pytest.fixture(scope="module")
def million_keys(torch_dev):
    torch, dev = torch_dev
    q, k, v = make_qkv(1, 2, 1, 1 << 20, 128, seed=61)   # K, V: 512 MiB each
    O, L = oracle.attention(q, k, v, False, 0.5)   # peaky: a handful of keys dominate each row
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    return (qd, kd, vd), (O, L)


@pytest.mark.parametrize("ns", [0, 1, 7])
def test_decode_million_keys(torch_dev, fa, million_keys, ns):
    torch, _ = torch_dev
    (qd, kd, vd), (O, L) = million_keys
    o, lse = fa.fa_decode_splitkv(qd, kd, vd, scale=0.5, num_splits=ns)
    torch.cuda.synchronize()
    check(o.float().cpu().numpy(), lse.cpu().numpy(), O, L, f"decode 2^20 keys ns={ns}")


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_256k_keys(torch_dev, fa, causal):
    torch, dev = torch_dev
    q, k, v = make_qkv(1, 2, 130, 1 << 18, 128, seed=62)
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, scale=0.3)
    torch.cuda.synchronize()
    O, L = oracle.attention(q, k, v, causal, 0.3)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), O, L, f"prefill 130 x 2^18 keys causal={causal}")


def test_prefill_128k_keys_key_split(torch_dev, fa):
    # D = 256, 130 queries over 2^17 keys: two query tiles on a whole GPU,
    # so fa_fwd splits each key range (up to 8 parts of ~500 key tiles) and
    # merges them; part offsets reach tens of MiB inside the slice
    torch, dev = torch_dev
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    assert fa.fa_fwd_key_splits(1, 1, 130, 1 << 17, 256, False, cus) > 1
    q, k, v = make_qkv(1, 1, 130, 1 << 17, 256, seed=63)
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=False, scale=0.25)  # peaky: O of order one
    torch.cuda.synchronize()
    O, L = oracle.attention(q, k, v, False, 0.25)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), O, L, "prefill D=256 130 x 2^17 keys, key split")
