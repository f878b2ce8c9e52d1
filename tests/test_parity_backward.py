"""GPU parity of the backward pass (fa_bwd, fa_bwd_ws) against the CPU fp64 oracle;
fa_bwd_ws is also checked bit for bit against fa_bwd and under graph replay.

The GPU pass takes o and lse from the GPU forward and the fp16 dO; the
oracle differentiates the definition in fp64 from the same fp16 q, k, v, dO.

Bar, element by element: every gradient entry G with oracle value R sums
terms whose magnitudes the oracle also gives, and its error is bounded by
fp16 rounding of those terms,
    |G - R| <= 8 u T + u |R| + 1e-6,    u = 2^-11 (fp16 unit roundoff),
where T is the sum of the absolute values of the terms the entry adds up:
    T_dV[j, d] = sum_i P_ij |dO_id|
    T_dS[i, j] = P_ij (|dP_ij| + T_D[i]),  T_D[i] = sum_d |dO_id| (|O_id| + sum_j P_ij |V_jd|)
    T_dQ[i, d] = scale sum_j T_dS[i, j] |K_jd|
    T_dK[j, d] = scale sum_i T_dS[i, j] |Q_id|
The kernels round P and dS to fp16 for the products (u of each term), take
P from the GPU forward's LSE (whose error, at most the forward's 1e-3 bar and
~2.4e-4 seen, is at most 2u of each term) and D_i from the fp16 O (whose
rounding and fp16-P error are at most 2u of T_D); that is 5u of T, and 8u
leaves margin.  u |R| is the rounding of the fp16 output itself, 1e-6 its
subnormal floor.  Unlike a bar scaled by the tensor's largest entry, this
one holds each small entry to the rounding of its own terms.
"""
import numpy as np
import pytest

import oracle
from workloads import make_qkv

pytestmark = pytest.mark.gpu

U = 2.0 ** -11
KAPPA = 8.0


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


def term_magnitudes(q, k, v, do, causal, scale):
    """(T_dQ, T_dK, T_dV): per entry, the sum of |terms| the entry adds up (fp64)."""
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    tq = np.empty((B, H, Sq, D))
    tk = np.empty((B, H, Sk, D))
    tv = np.empty((B, H, Sk, D))
    for b in range(B):
        for h in range(H):
            q2, k2, v2, do2 = (np.asarray(x[b, h], dtype=np.float64) for x in (q, k, v, do))
            P = oracle.softmax_probs(q2, k2, causal, scale)
            O = P @ v2
            dP = do2 @ v2.T
            TD = (np.abs(do2) * (np.abs(O) + P @ np.abs(v2))).sum(axis=1)
            TdS = P * (np.abs(dP) + TD[:, None])
            tv[b, h] = P.T @ np.abs(do2)
            tq[b, h] = scale * (TdS @ np.abs(k2))
            tk[b, h] = scale * (TdS.T @ np.abs(q2))
    return tq, tk, tv


def check(got, ref, terms, what):
    for name, g, r, t in zip(("dQ", "dK", "dV"), got, ref, terms):
        assert np.isfinite(g).all(), f"{what} {name}: non-finite"
        err = np.abs(g - r)
        bound = KAPPA * U * t + U * np.abs(r) + 1e-6
        worst = float((err / bound).max())
        i = np.unravel_index(int(np.argmax(err / bound)), err.shape)
        print(f"{what} {name}: max|err|={float(err.max()):.3e} max err/bound={worst:.3f} at {i} "
              f"(err {float(err[i]):.3e}, T {float(t[i]):.3e}, ref {float(r[i]):.3e})", flush=True)
        assert worst <= 1.0, f"{what} {name}: entry {i} err {float(err[i]):.3e} > bound {float(bound[i]):.3e}"


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


@pytest.mark.parametrize("D", [32, 64, 128, 256])
@pytest.mark.parametrize("shape", SHAPES, ids=["x".join(map(str, s)) for s in SHAPES])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_parity(torch_dev, fa, D, shape, causal):
    B, H, Sq, Sk = shape
    q, k, v = make_qkv(B, H, Sq, Sk, D, 700 + Sq + D)
    do = make_qkv(B, H, Sq, 1, D, 800 + Sq)[0]
    scale = 1.0 / np.sqrt(D)
    got = run_bwd(torch_dev, fa, q, k, v, do, causal, scale)
    ref = oracle.attention_backward(q, k, v, do, causal, scale)
    check(got, ref, term_magnitudes(q, k, v, do, causal, scale), f"bwd D={D} {shape} causal={causal}")


def test_backward_llama_shape_two_heads(torch_dev, fa):
    # the full (1, 32, 4096, 4096, 128) causal backward, checked on heads 0 and 31
    B, H, S, D = 1, 32, 4096, 128
    q, k, v = make_qkv(B, H, S, S, D, 3)
    do = make_qkv(B, H, S, 1, D, 13)[0]
    scale = 1.0 / np.sqrt(D)
    dq, dk, dv = run_bwd(torch_dev, fa, q, k, v, do, True, scale)
    for h in (0, 31):
        sl = slice(h, h + 1)
        args = (q[:, sl], k[:, sl], v[:, sl], do[:, sl], True, scale)
        check([dq[:, sl], dk[:, sl], dv[:, sl]], oracle.attention_backward(*args), term_magnitudes(*args),
              f"llama head {h}")


def test_backward_d256_workload(torch_dev, fa):
    # the (1, 16, 2048, 2048, 256) causal shape of the D = 256 prefill, every
    # element of every head
    B, H, S, D = 1, 16, 2048, 256
    q, k, v = make_qkv(B, H, S, S, D, 5)
    do = make_qkv(B, H, S, 1, D, 15)[0]
    scale = 1.0 / 16
    got = run_bwd(torch_dev, fa, q, k, v, do, True, scale)
    check(got, oracle.attention_backward(q, k, v, do, True, scale), term_magnitudes(q, k, v, do, True, scale),
          "d256 workload")


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
    q = torch.zeros((1, 1, 8, 512), dtype=torch.float16, device=dev)
    o, lse = fa.fa_fwd(q, q, q)
    with pytest.raises(fa.FAError) as e:
        fa.fa_bwd(q, q, q, o, lse, q)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED


def test_backward_ws_matches_fa_bwd(torch_dev, fa):
    # fa_bwd_ws with a caller workspace (first filled with 0xff bytes, then
    # reused for a second shape) gives fa_bwd's results bit for bit; a
    # workspace one byte short is refused before any launch
    torch, dev = torch_dev
    D = 64
    shapes = [(1, 2, 300, 300), (2, 1, 129, 65)]
    nbytes = max(fa.fa_bwd_workspace_bytes(B, H, Sq, D) for B, H, Sq, _ in shapes)
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device=dev)
    for i, (B, H, Sq, Sk) in enumerate(shapes):
        q, k, v = make_qkv(B, H, Sq, Sk, D, 90 + i)
        do = make_qkv(B, H, Sq, 1, D, 95 + i)[0]
        qd, kd, vd, dod = (torch.from_numpy(x).to(dev) for x in (q, k, v, do))
        o, lse = fa.fa_fwd(qd, kd, vd, causal=True, scale=0.125)
        a = fa.fa_bwd(qd, kd, vd, o, lse, dod, causal=True, scale=0.125)
        b = fa.fa_bwd_ws(qd, kd, vd, o, lse, dod, ws, causal=True, scale=0.125)
        torch.cuda.synchronize()
        assert all(torch.equal(x, y) for x, y in zip(a, b)), (B, H, Sq, Sk)
        check([x.float().cpu().numpy() for x in b], oracle.attention_backward(q, k, v, do, True, 0.125),
              term_magnitudes(q, k, v, do, True, 0.125), f"bwd_ws {(B, H, Sq, Sk)}")
    short = fa.fa_bwd_workspace_bytes(shapes[-1][0], shapes[-1][1], shapes[-1][2], D) - 1
    with pytest.raises(fa.FAError) as e:
        fa.fa_bwd_ws(qd, kd, vd, o, lse, dod, ws[:short], causal=True, scale=0.125)
    assert e.value.status == fa.FA_ERR_INVALID_ARG


def test_backward_ws_graph_replays(torch_dev, fa):
    # fa_bwd_ws (three kernels, no allocation) captured in a graph and
    # replayed; each replay, with eager work and a sync in between, is
    # bit-identical to the eager call
    torch, dev = torch_dev
    B, H, S, D = 1, 4, 384, 128
    q, k, v = make_qkv(B, H, S, S, D, 97)
    do = make_qkv(B, H, S, 1, D, 98)[0]
    qd, kd, vd, dod = (torch.from_numpy(x).to(dev) for x in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=True, scale=0.1)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, S, D), dtype=torch.uint8, device=dev)
    grads = [torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)]
    eager = fa.fa_bwd_ws(qd, kd, vd, o, lse, dod, ws, causal=True, scale=0.1)
    torch.cuda.synchronize()
    eager = [x.clone() for x in eager]
    side = torch.cuda.Stream(device=dev)  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fa.fa_bwd_ws(qd, kd, vd, o, lse, dod, ws, *grads, causal=True, scale=0.1)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fa_bwd_ws(qd, kd, vd, o, lse, dod, ws, *grads, causal=True, scale=0.1)
    for rep in range(3):
        for x in grads:
            x.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(grads, eager)), f"replay {rep}"
        fa.fa_bwd_ws(qd, kd, vd, o, lse, dod, ws, causal=True, scale=0.1)  # eager work between replays
        torch.cuda.synchronize()
