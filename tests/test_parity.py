"""GPU parity: the HIP path through the C ABI against the CPU fp64 oracle.

Bar (fp16 unit-normal inputs): max |O - O_oracle| <= 2e-3 and
max |LSE - LSE_oracle| <= 1e-3, element by element on the same seeded inputs.
Every full-size workload is compared on every element (tiny, small, the
LLaMA-7B-shaped prefill, D=256 prefill, and the 8K decode in both its
one-kernel and two-kernel forms); sampled rows of the LLaMA-7B-shaped
prefill are a fast subset.
"""
import math

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, make_qkv, sample_rows, workload_inputs

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


def to_dev(torch_dev, *arrays):
    torch, dev = torch_dev
    return [torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in arrays]


def gpu_fwd(torch_dev, fa, q, k, v, causal, scale):
    torch, _ = torch_dev
    qd, kd, vd = to_dev(torch_dev, q, k, v)
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def gpu_decode(torch_dev, fa, q, k, v, scale, ns):
    torch, _ = torch_dev
    qd, kd, vd = to_dev(torch_dev, q, k, v)
    o, lse = fa.fa_decode_splitkv(qd, kd, vd, scale=scale, num_splits=ns)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def assert_close(o, lse, O, L, what):
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{what}: non-finite output"
    eo = float(np.abs(o - O).max())
    el = float(np.abs(lse - L).max())
    print(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= O_TOL, f"{what}: max|dO| = {eo:.3e}"
    assert el <= LSE_TOL, f"{what}: max|dLSE| = {el:.3e}"


# ------------------------------------------------------------ the workloads

@pytest.mark.parametrize("name,causal", [
    ("tiny", False), ("tiny", True), ("small", False), ("small", True), ("d256_prefill", True),
])
def test_workload_prefill_full(torch_dev, fa, name, causal):
    w = WORKLOADS[name]
    q, k, v = workload_inputs(w)
    o, lse = gpu_fwd(torch_dev, fa, q, k, v, causal, w.scale)
    O, L = oracle.attention(q, k, v, causal, w.scale)
    assert_close(o, lse, O, L, f"{name} causal={causal}")


@pytest.fixture(scope="module")
def llama(torch_dev, fa):
    w = WORKLOADS["llama7b_prefill"]
    q, k, v = workload_inputs(w)
    o, lse = gpu_fwd(torch_dev, fa, q, k, v, True, w.scale)
    return w, q, k, v, o, lse


def test_llama_prefill_sampled_rows(llama):
    w, q, k, v, o, lse = llama
    rows = sample_rows(w, 192)
    O, L = oracle.attention_rows(q, k, v, True, w.scale, rows)
    idx = tuple(np.array(rows).T)
    assert_close(o[idx], lse[idx], O, L, "llama7b sampled rows")


def test_llama_prefill_every_element(llama):
    # the whole output: all 32 heads of O and LSE against the oracle
    w, q, k, v, o, lse = llama
    O, L = oracle.attention(q, k, v, True, w.scale)
    assert_close(o, lse, O, L, "llama7b every element")


@pytest.fixture(scope="module")
def decode_8k():
    w = WORKLOADS["decode_8k"]
    q, k, v = workload_inputs(w)
    O, L = oracle.attention(q, k, v, False, w.scale)
    return w, q, k, v, O, L


# 0: the library's automatic choice (one partition, merged in LDS, at this
# size); 4: the two-kernel form with the partitions that fill the CUs
# (B*H*ns = 2048 phase-one workgroups = 8 per CU) and the merge kernel
@pytest.mark.parametrize("ns", [0, 4])
def test_decode_workload_full(torch_dev, fa, decode_8k, ns):
    w, q, k, v, O, L = decode_8k
    o, lse = gpu_decode(torch_dev, fa, q, k, v, w.scale, ns)
    assert_close(o, lse, O, L, f"decode_8k ns={ns}")


# -------------------------------------------------- ragged and edge shapes

RAGGED = [
    # B, H, Sq, Sk
    (1, 3, 200, 333),
    (2, 1, 1, 77),
    (1, 2, 100, 100),
    (1, 1, 300, 100),   # more queries than keys
    (1, 1, 100, 300),
    (1, 1, 1, 1),
    (1, 2, 129, 65),
    (1, 1, 257, 257),
    (1, 2, 1000, 1000),  # long unrolled main loop with a ragged tail
    (1, 1, 777, 1500),
]


@pytest.mark.parametrize("D", [32, 64, 128, 256])
@pytest.mark.parametrize("shape", RAGGED, ids=["x".join(map(str, s)) for s in RAGGED])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_prefill(torch_dev, fa, D, shape, causal):
    B, H, Sq, Sk = shape
    q, k, v = make_qkv(B, H, Sq, Sk, D, seed=1000 + Sq + 7 * Sk + D)
    scale = 1.0 / math.sqrt(D)
    o, lse = gpu_fwd(torch_dev, fa, q, k, v, causal, scale)
    O, L = oracle.attention(q, k, v, causal, scale)
    assert_close(o, lse, O, L, f"D={D} {shape} causal={causal}")


WIDE = [
    # B*H = 256 slices: enough workgroups that D <= 128 runs 8-wavefront workgroups
    (4, 64, 300, 333),
    (2, 128, 257, 1000),
    (1, 256, 1, 700),
]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("shape", WIDE, ids=["x".join(map(str, s)) for s in WIDE])
@pytest.mark.parametrize("causal", [False, True])
def test_wide_grid_prefill(torch_dev, fa, D, shape, causal):
    B, H, Sq, Sk = shape
    q, k, v = make_qkv(B, H, Sq, Sk, D, seed=2000 + Sq + Sk + D)
    scale = 1.0 / math.sqrt(D)
    o, lse = gpu_fwd(torch_dev, fa, q, k, v, causal, scale)
    O, L = oracle.attention(q, k, v, causal, scale)
    assert_close(o, lse, O, L, f"wide D={D} {shape} causal={causal}")


@pytest.mark.parametrize("scale", [0.05, 0.3, 1.0])
def test_other_scales_and_large_scores(torch_dev, fa, scale):
    q, k, v = make_qkv(1, 2, 160, 160, 128, seed=77)
    q = (q.astype(np.float32) * 3).astype(np.float16)  # wider score spread
    for causal in (False, True):
        o, lse = gpu_fwd(torch_dev, fa, q, k, v, causal, scale)
        O, L = oracle.attention(q, k, v, causal, scale)
        assert_close(o, lse, O, L, f"scale={scale} causal={causal}")


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_closed_forms_on_gpu(torch_dev, fa, D):
    B, H, S = 1, 2, 150
    _, k, v = make_qkv(B, H, S, S, D, seed=5)
    q0 = np.zeros((B, H, S, D), np.float16)
    o, lse = gpu_fwd(torch_dev, fa, q0, k, v, False, 0.125)
    vm = v.astype(np.float64).mean(axis=2, keepdims=True)
    assert np.abs(o - vm).max() <= O_TOL and np.abs(lse - math.log(S)).max() <= LSE_TOL
    o, lse = gpu_fwd(torch_dev, fa, q0, k, v, True, 0.125)
    cm = np.cumsum(v.astype(np.float64), axis=2) / np.arange(1, S + 1)[None, None, :, None]
    assert np.abs(o - cm).max() <= O_TOL
    assert np.abs(lse - np.log(np.arange(1, S + 1))[None, None, :]).max() <= LSE_TOL
    # causal row 0 is exactly V[0]
    q, _, _ = make_qkv(B, H, S, S, D, seed=6)
    o, _ = gpu_fwd(torch_dev, fa, q, k, v, True, 1.0 / math.sqrt(D))
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0].astype(np.float32))
    # constant V gives that constant
    vc = np.full_like(v, 0.75)
    o, _ = gpu_fwd(torch_dev, fa, q, k, vc, True, 1.0 / math.sqrt(D))
    assert np.abs(o - 0.75).max() <= O_TOL


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("D", [32, 64, 128, 256])
@pytest.mark.parametrize("ns", [1, 2, 3, 7, 64, 0])
def test_decode_split_sweep(torch_dev, fa, D, ns):
    B, H, Sk = 2, 4, 8191
    q, k, v = make_qkv(B, H, 1, Sk, D, seed=300 + D)
    scale = 1.0 / math.sqrt(D)
    o, lse = gpu_decode(torch_dev, fa, q, k, v, scale, ns)
    O, L = oracle.attention(q, k, v, False, scale)
    assert_close(o, lse, O, L, f"decode D={D} ns={ns}")


def test_fwd_single_query_runs_the_decode(torch_dev, fa):
    # fa_fwd with Sq = 1, non-causal: the split-KV decode (bitwise the same
    # result as fa_decode_splitkv), here over a long context with few heads
    torch, _ = torch_dev
    q, k, v = make_qkv(1, 2, 1, 50000, 128, seed=71)
    qd, kd, vd = to_dev(torch_dev, q, k, v)
    o1, l1 = fa.fa_fwd(qd, kd, vd, causal=False)
    o2, l2 = fa.fa_decode_splitkv(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    O, L = oracle.attention(q, k, v, False, 1.0 / math.sqrt(128))
    assert_close(o1.float().cpu().numpy(), l1.cpu().numpy(), O, L, "fa_fwd Sq=1")
    # causal Sq = 1 sees key 0 only (top-left mask): O = V[0]
    o3, l3 = fa.fa_fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o3.float().cpu().numpy()[:, :, 0], v[:, :, 0].astype(np.float32))


@pytest.mark.parametrize("Sk,ns", [(1, 1), (5, 5), (100, 64), (300, 0), (1000, 999)])
def test_decode_small_and_empty_partitions(torch_dev, fa, Sk, ns):
    q, k, v = make_qkv(3, 2, 1, Sk, 128, seed=Sk)
    o, lse = gpu_decode(torch_dev, fa, q, k, v, 0.2, ns)
    O, L = oracle.attention(q, k, v, False, 0.2)
    assert_close(o, lse, O, L, f"decode Sk={Sk} ns={ns}")


def test_decode_partials_match_oracle(torch_dev, fa):
    torch, dev = torch_dev
    B, H, Sk, D, ns = 2, 3, 100, 128, 64   # chunk 2: partitions 50..63 are empty
    q, k, v = make_qkv(B, H, 1, Sk, D, seed=41)
    nbytes = fa.fa_decode_workspace_bytes(B, H, D, ns)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=dev)
    qd, kd, vd = to_dev(torch_dev, q, k, v)
    o, lse = fa.fa_decode_splitkv_ws(qd, kd, vd, ws, scale=0.125, num_splits=ns)
    torch.cuda.synchronize()
    w = ws.cpu().numpy()
    Os = w[: B * H * ns * D].reshape(B, H, ns, D)
    Ls = w[B * H * ns * D : B * H * ns * (D + 1)].reshape(B, H, ns)
    Oo, Lo = oracle.split_partials(q, k, v, 0.125, ns)
    assert (Ls[:, :, 50:] == -np.inf).all() and (Os[:, :, 50:] == 0).all()
    assert_close(Os[:, :, :50], Ls[:, :, :50], Oo[:, :, :50, 0], Lo[:, :, :50, 0], "decode partials")
    O, L = oracle.attention(q, k, v, False, 0.125)
    assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), O, L, "decode merged via _ws")


def test_decode_single_partition_leaves_workspace_alone(torch_dev, fa):
    # one partition: one kernel merges in LDS and writes o and lse directly
    torch, dev = torch_dev
    B, H, Sk, D = 2, 3, 777, 128
    q, k, v = make_qkv(B, H, 1, Sk, D, seed=43)
    nbytes = fa.fa_decode_workspace_bytes(B, H, D, 1)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=dev)
    qd, kd, vd = to_dev(torch_dev, q, k, v)
    o, lse = fa.fa_decode_splitkv_ws(qd, kd, vd, ws, scale=0.125, num_splits=1)
    torch.cuda.synchronize()
    assert torch.isnan(ws).all()
    O, L = oracle.attention(q, k, v, False, 0.125)
    assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), O, L, "decode ns=1 via _ws")


# ------------------------------------------------- determinism and errors

def test_run_to_run_bitwise(torch_dev, fa):
    torch, _ = torch_dev
    q, k, v = make_qkv(2, 4, 300, 300, 128, seed=9)
    qd, kd, vd = to_dev(torch_dev, q, k, v)
    for causal in (False, True):
        a = fa.fa_fwd(qd, kd, vd, causal=causal)
        b = fa.fa_fwd(qd, kd, vd, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    qd1 = qd[:, :, :1].contiguous()
    a = fa.fa_decode_splitkv(qd1, kd, vd, num_splits=5)
    b = fa.fa_decode_splitkv(qd1, kd, vd, num_splits=5)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_side_stream(torch_dev, fa):
    torch, dev = torch_dev
    q, k, v = make_qkv(1, 4, 130, 130, 64, seed=11)
    qd, kd, vd = to_dev(torch_dev, q, k, v)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device=dev)  # default priority
    with torch.cuda.stream(s):
        o, lse = fa.fa_fwd(qd, kd, vd, causal=True)
    s.synchronize()
    O, L = oracle.attention(q, k, v, True, 0.125)
    assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), O, L, "side stream")


def test_split_decodes_on_two_streams_and_growth(torch_dev, fa):
    # split decodes queued back to back on two streams with no host sync:
    # each call takes its own workspace from the stream-ordered pool on its
    # stream and frees it there, and the split counts (so the workspace
    # sizes) grow from one round to the next
    torch, dev = torch_dev
    cases = [make_qkv(1, 4, 1, 3000, 128, seed=81), make_qkv(2, 6, 1, 9000, 64, seed=82)]
    dev_in = [to_dev(torch_dev, *c) for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]  # default priority
    outs = []
    for rep in range(3):
        for i, (qd, kd, vd) in enumerate(dev_in):
            with torch.cuda.stream(streams[i]):
                outs.append((i, fa.fa_decode_splitkv(qd, kd, vd, num_splits=16 + 8 * rep)))
    for st in streams:
        st.synchronize()
    for n, (i, (o, lse)) in enumerate(outs):
        q, k, v = cases[i]
        O, L = oracle.attention(q, k, v, False, 1.0 / math.sqrt(q.shape[-1]))
        assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), O, L, f"decode stream {i} call {n}")


def test_errors_raise(torch_dev, fa):
    torch, dev = torch_dev
    q = torch.zeros(1, 1, 2, 128, dtype=torch.float16, device=dev)
    with pytest.raises(fa.FAError) as e:
        fa.fa_decode_splitkv(q, q, q)
    assert e.value.status == fa.FA_ERR_INVALID_ARG
    q96 = torch.zeros(1, 1, 2, 96, dtype=torch.float16, device=dev)
    with pytest.raises(fa.FAError) as e:
        fa.fa_fwd(q96, q96, q96)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
