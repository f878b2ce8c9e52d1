"""GPU parity of the key-split prefill against the CPU fp64 oracle.

fa_fwd splits the key ranges of a small grid's query tiles (the split-KV
scheme of "Adaptive High-Performance Attention Kernels in CUDA", Split-K /
Flash-Decoding, on prefill tiles) and merges the parts with log-sum-exp
weights: at D <= 128 (causal grids of the 4-wavefront kernel) the heaviest
query tiles in equal parts, at D = 256 the key tiles of all query tiles cut
into one run per CU (a tile cut between runs is merged by a second kernel).
Every shape here is checked to be one that fa_fwd_key_splits() splits on
this device, so these tests run the split kernels and their merges; the bar
is the one of every prefill: max |dO| <= 2e-3, max |dLSE| <= 1e-3.  Also
covered: bitwise repeatability, split calls of different workspace sizes
queued without a sync, split calls on two streams at once (each with its own
pool workspace), fa_fwd_ws with a caller workspace (bit-identical to fa_fwd;
a short workspace is refused), a caller workspace reused across calls and
holding arbitrary bytes, and a captured graph of one split call replayed.
"""
import math

import numpy as np
import pytest

import oracle
from workloads import make_qkv

pytestmark = pytest.mark.gpu

O_TOL = 2e-3
LSE_TOL = 1e-3
D = 256


@pytest.fixture(scope="module")
def env():
    import torch

    import exact_attention_54_amd as fa

    assert torch.cuda.is_available(), "GPU tests need a GPU (the HIP library has no CPU path)"
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    return torch, dev, fa, cus


def inputs(env, B, H, Sq, Sk, causal, seed, D=D):
    torch, dev, fa, cus = env
    ns = fa.fa_fwd_key_splits(B, H, Sq, Sk, D, causal, cus)
    assert ns > 1, f"{(B, H, Sq, Sk, D, causal)} is not split on {cus} CUs"
    q, k, v = make_qkv(B, H, Sq, Sk, D, seed=seed)
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    return (q, k, v), (qd, kd, vd), ns


def check(o, lse, O, L, what):
    o = o.float().cpu().numpy() if hasattr(o, "cpu") else o
    lse = lse.cpu().numpy() if hasattr(lse, "cpu") else lse
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{what}: non-finite output"
    eo = float(np.abs(o - O).max())
    el = float(np.abs(lse - L).max())
    print(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= O_TOL, f"{what}: max|dO| = {eo:.3e}"
    assert el <= LSE_TOL, f"{what}: max|dLSE| = {el:.3e}"


def test_split_calls_of_different_sizes_queued(env):
    # small split call, the largest split call of this file, small again,
    # queued back to back without a sync: each takes a workspace of its own
    # size from the stream-ordered pool and returns it on the stream
    torch = env[0]
    small = inputs(env, 1, 2, 1000, 1000, True, seed=31)
    large = inputs(env, 1, 4, 2048, 2048, False, seed=32)
    seq = [(small, True), (large, False), (small, True)]
    outs = [env[2].fa_fwd(*case[1], causal=causal, scale=1 / 16) for case, causal in seq]
    torch.cuda.synchronize()
    for ((host, _, ns), causal), (o, lse) in zip(seq, outs):
        O, L = oracle.attention(*host, causal, 1 / 16)
        check(o, lse, O, L, f"queued {host[0].shape} causal={causal} ns={ns}")


SPLIT = [
    # B, H, Sq, Sk, causal
    (1, 8, 1024, 1024, True),
    (1, 4, 2048, 2048, False),
    (1, 2, 1000, 1000, True),
    (1, 2, 500, 1500, False),   # more keys than queries
    (1, 1, 777, 1500, True),
    (1, 1, 3000, 1000, True),   # more queries than keys
    (2, 1, 129, 1000, False),   # a ragged query tile of one row
]


@pytest.mark.parametrize("shape", SPLIT, ids=["x".join(map(str, s)) for s in SPLIT])
def test_split_prefill_matches_oracle(env, shape):
    B, H, Sq, Sk, causal = shape
    host, dev_in, ns = inputs(env, B, H, Sq, Sk, causal, seed=100 + Sq + Sk)
    scale = 1.0 / math.sqrt(D)
    o, lse = env[2].fa_fwd(*dev_in, causal=causal, scale=scale)
    env[0].cuda.synchronize()
    O, L = oracle.attention(*host, causal, scale)
    check(o, lse, O, L, f"split {shape} ns={ns}")


def test_split_long_causal_sampled_rows(env):
    # (1, 8, 4096, 4096): every heavy tile cut once between two runs; rows
    # sampled across every tile, both ends of the 128-row tiles among them
    torch = env[0]
    host, dev_in, ns = inputs(env, 1, 8, 4096, 4096, True, seed=41)
    o, lse = env[2].fa_fwd(*dev_in, causal=True, scale=1 / 16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = [(0, h, i) for h in (0, 7) for i in (0, 127, 128, 3071, 3072, 3199, 3200, 4095)]
    rows += [(0, int(h), int(i)) for h, i in zip(rng.integers(0, 8, 48), rng.integers(0, 4096, 48))]
    O, L = oracle.attention_rows(*host, True, 1 / 16, rows)
    idx = tuple(np.array(rows).T)
    check(o.float().cpu().numpy()[idx], lse.cpu().numpy()[idx], O, L, f"long causal sampled rows ns={ns}")


def test_split_d256_benchmark_shape_sampled_rows(env):
    # (1, 16, 2048, 2048) causal, the D = 256 prefill workload: runs of ~34
    # key tiles, each heavy tile cut once; rows sampled from every head at the
    # ends of query tiles and at random
    torch = env[0]
    host, dev_in, ns = inputs(env, 1, 16, 2048, 2048, True, seed=42)
    o, lse = env[2].fa_fwd(*dev_in, causal=True, scale=1 / 16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    rows = [(0, h, i) for h in range(16) for i in (0, 127, 128, 1023, 1024, 1919, 1920, 2047)]
    rows += [(0, int(h), int(i)) for h, i in zip(rng.integers(0, 16, 64), rng.integers(0, 2048, 64))]
    O, L = oracle.attention_rows(*host, True, 1 / 16, rows)
    idx = tuple(np.array(rows).T)
    check(o.float().cpu().numpy()[idx], lse.cpu().numpy()[idx], O, L, f"d256 benchmark shape sampled rows ns={ns}")


def test_split_run_to_run_bitwise(env):
    torch = env[0]
    _, dev_in, _ = inputs(env, 1, 8, 1024, 1024, True, seed=51)
    a = env[2].fa_fwd(*dev_in, causal=True, scale=1 / 16)
    b = env[2].fa_fwd(*dev_in, causal=True, scale=1 / 16)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_split_calls_on_two_streams(env):
    # split calls alternate between two streams with no host sync; each
    # call's workspace comes from the pool on its own stream, so the two
    # streams run concurrently without sharing a buffer
    torch, dev, fa, _ = env
    shapes = [(1, 2, 1000, 1000, True), (2, 1, 129, 1000, False)]
    cases = [inputs(env, B, H, Sq, Sk, c, seed=60 + i) + (c,) for i, (B, H, Sq, Sk, c) in enumerate(shapes)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]  # default priority
    outs = []
    for rep in range(3):
        for i, (host, dev_in, ns, causal) in enumerate(cases):
            with torch.cuda.stream(streams[i]):
                outs.append((i, fa.fa_fwd(*dev_in, causal=causal, scale=1 / 16)))
    for s in streams:
        s.synchronize()
    refs = [oracle.attention(*host, causal, 1 / 16) for host, _, _, causal in cases]
    for n, (i, (o, lse)) in enumerate(outs):
        check(o, lse, *refs[i], f"stream {i} call {n}")


SPLIT_SMALL_D = [
    # B, H, Sq, Sk, D (causal)
    (1, 2, 1000, 1000, 128),
    (1, 1, 1000, 3000, 128),    # more keys than queries
    (1, 1, 3000, 1000, 128),    # more queries than keys
    (1, 2, 1000, 1000, 64),
    (1, 2, 2000, 2000, 64),
    (1, 2, 2000, 2000, 32),
]


@pytest.mark.parametrize("shape", SPLIT_SMALL_D, ids=["x".join(map(str, s)) for s in SPLIT_SMALL_D])
def test_split_small_head_dims_match_oracle(env, shape):
    B, H, Sq, Sk, d = shape
    host, dev_in, ns = inputs(env, B, H, Sq, Sk, True, seed=200 + Sq + Sk + d, D=d)
    scale = 1.0 / math.sqrt(d)
    o, lse = env[2].fa_fwd(*dev_in, causal=True, scale=scale)
    env[0].cuda.synchronize()
    O, L = oracle.attention(*host, True, scale)
    check(o, lse, O, L, f"split D={d} {shape} ns={ns}")


@pytest.mark.parametrize("d", [64, 128])
def test_split_head_shard_of_llama_prefill_sampled_rows(env, d):
    # (1, 4, 4096, 4096): one GPU's 4 of the 32 heads when the LLaMA-7B-shaped
    # prefill is sharded by heads over 8 GPUs
    torch = env[0]
    host, dev_in, ns = inputs(env, 1, 4, 4096, 4096, True, seed=300 + d, D=d)
    scale = 1.0 / math.sqrt(d)
    o, lse = env[2].fa_fwd(*dev_in, causal=True, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = [(0, h, i) for h in (0, 3) for i in (0, 127, 128, 1023, 1024, 2047, 2048, 3071, 3072, 4095)]
    rows += [(0, int(h), int(i)) for h, i in zip(rng.integers(0, 4, 40), rng.integers(0, 4096, 40))]
    O, L = oracle.attention_rows(*host, True, scale, rows)
    idx = tuple(np.array(rows).T)
    check(o.float().cpu().numpy()[idx], lse.cpu().numpy()[idx], O, L, f"head shard D={d} sampled rows ns={ns}")


def test_fwd_ws_caller_workspace_matches_fwd(env):
    # fa_fwd_ws with a caller workspace of exactly fa_fwd_workspace_bytes is
    # bit-identical to fa_fwd (same plan, same kernels); one byte short is
    # refused before any launch
    torch, dev, fa, cus = env
    host, dev_in, ns = inputs(env, 1, 8, 1024, 1024, True, seed=71)
    nbytes = fa.fa_fwd_workspace_bytes(1, 8, 1024, 1024, D, True, cus)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    a = fa.fa_fwd(*dev_in, causal=True, scale=1 / 16)
    b = fa.fa_fwd_ws(*dev_in, ws, causal=True, scale=1 / 16)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    O, L = oracle.attention(*host, True, 1 / 16)
    check(b[0], b[1], O, L, f"fa_fwd_ws ns={ns}")
    with pytest.raises(fa.FAError) as e:
        fa.fa_fwd_ws(*dev_in, ws[:-1], causal=True, scale=1 / 16)
    assert e.value.status == fa.FA_ERR_INVALID_ARG
    # an unsplit call needs no workspace
    q, k, v = make_qkv(1, 2, 300, 300, 64, seed=72)
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    assert fa.fa_fwd_workspace_bytes(1, 2, 300, 300, 64, False, cus) == 0
    o, lse = fa.fa_fwd_ws(qd, kd, vd, None, causal=False, scale=0.125)
    torch.cuda.synchronize()
    O, L = oracle.attention(q, k, v, False, 0.125)
    check(o, lse, O, L, "fa_fwd_ws without workspace")


def test_fwd_ws_workspace_reuse_and_contents(env):
    # one caller workspace for a sequence of D = 256 split calls: first
    # filled with 0xff bytes, then reused without clearing for other inputs,
    # then filled with random bytes; nothing a call reads from it is left
    # from an earlier call, so every call matches the oracle and equal inputs
    # give bit-identical outputs
    torch, dev, fa, cus = env
    shape = (1, 8, 1024, 1024)
    nbytes = fa.fa_fwd_workspace_bytes(*shape, D, True, cus)
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device=dev)
    cases = [inputs(env, *shape, True, seed=s) for s in (81, 82)]
    refs = [oracle.attention(*host, True, 1 / 16) for host, _, _ in cases]
    first = fa.fa_fwd_ws(*cases[0][1], ws, causal=True, scale=1 / 16)
    torch.cuda.synchronize()
    check(*first, *refs[0], "workspace of 0xff bytes")
    for rep in range(3):  # queued without a sync, one workspace
        outs = [fa.fa_fwd_ws(*dev_in, ws, causal=True, scale=1 / 16) for _, dev_in, _ in cases]
        torch.cuda.synchronize()
        for i, out in enumerate(outs):
            check(*out, *refs[i], f"reused workspace, call {rep}.{i}")
        assert torch.equal(outs[0][0], first[0]) and torch.equal(outs[0][1], first[1])
    ws.copy_(torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev))
    again = fa.fa_fwd_ws(*cases[0][1], ws, causal=True, scale=1 / 16)
    torch.cuda.synchronize()
    assert torch.equal(again[0], first[0]) and torch.equal(again[1], first[1])


def test_fwd_ws_split_call_graph_replays(env):
    # one D = 256 split call (split kernel and merge kernel) captured in a
    # graph and replayed; each replay (with eager work and a sync in
    # between) is bit-identical to the eager call
    torch, dev, fa, cus = env
    shape = (1, 8, 1024, 1024)
    host, dev_in, ns = inputs(env, *shape, True, seed=91)
    nbytes = fa.fa_fwd_workspace_bytes(*shape, D, True, cus)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    o = torch.empty_like(dev_in[0])
    lse = torch.empty(dev_in[0].shape[:3], dtype=torch.float32, device=dev)
    eager = fa.fa_fwd_ws(*dev_in, ws, causal=True, scale=1 / 16)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fa.fa_fwd_ws(*dev_in, ws, o, lse, causal=True, scale=1 / 16)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fa_fwd_ws(*dev_in, ws, o, lse, causal=True, scale=1 / 16)
    for rep in range(4):
        o.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eager[0]) and torch.equal(lse, eager[1]), f"replay {rep}"
        fa.fa_fwd_ws(*dev_in, ws, causal=True, scale=1 / 16)  # eager work between replays
        torch.cuda.synchronize()
    O, L = oracle.attention(*host, True, 1 / 16)
    check(o, lse, O, L, f"graph replay ns={ns}")
