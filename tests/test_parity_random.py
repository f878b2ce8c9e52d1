"""GPU parity on seeded random cases against the CPU fp64 oracle.

- fa_fwd: forty shapes drawn from one seed, D in {32, 64, 128, 256}, one to
  four (batch, head) slices, query and key lengths up to 1500 (ragged),
  both mask settings, plus ten Split-D shapes (D 512, 1024).  Grids this
  small are the ones fa_fwd gives a key-range split, so the draw covers
  many split plans next to unsplit ones; each case prints its plan, and
  fa_fwd_ws on a workspace filled with 0xff must match fa_fwd bit for bit.
- fa_fwd_varlen: packed batches of one to five sequences of 0..700 tokens,
  key lengths equal to or independent of the query lengths.
- fa_bwd: small random shapes at the elementwise backward bar of
  test_parity_backward.py.
- fa_decode_splitkv / fa_decode_paged: random contexts, split counts, page
  sizes, absent pages and clamped lengths; where every sequence has the
  same context and no page is absent, paged and contiguous decoding must
  agree bit for bit.
Bar as for every forward: max |dO| <= 2e-3, max |dLSE| <= 1e-3.
"""
import math

import numpy as np
import pytest

import oracle
from test_parity_backward import check as backward_check, term_magnitudes
from workloads import make_qkv, make_varlen, paged_layout, to_pages

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


def draw_splitd_shapes(n, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return [(1, int(g.integers(1, 3)), int(g.integers(1, 601)), int(g.integers(1, 601)),
             int(g.choice([512, 1024])), bool(g.random() < 0.5)) for _ in range(n)]


SHAPES += draw_splitd_shapes(10, 2025)


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
    nbytes = fa.fa_fwd_workspace_bytes(B, H, Sq, Sk, D, causal, cus)
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device=dev) if nbytes else None
    o2, lse2 = fa.fa_fwd_ws(qd, kd, vd, ws, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "fa_fwd_ws differs from fa_fwd"
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    O, L = oracle.attention(q, k, v, causal, scale)
    parts = fa.fa_fwd_key_splits(B, H, Sq, Sk, D, causal, cus)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    eo = float(np.abs(o - O).max())
    el = float(np.abs(lse - L).max())
    print(f"{shape} key parts {parts}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= O_TOL and el <= LSE_TOL


def draw_varlen(n, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    cases = []
    while len(cases) < n:
        B = int(g.integers(1, 6))
        lq = g.integers(0, 701, size=B)
        lk = lq if g.random() < 0.5 else g.integers(0, 701, size=B)
        if lq.sum() and lk.sum():
            cases.append((int(g.choice([32, 64, 128, 256])), int(g.integers(1, 4)), tuple(int(x) for x in lq),
                          tuple(int(x) for x in lk), bool(g.random() < 0.6)))
    return cases


VARLEN = draw_varlen(30, 2026)


@pytest.mark.parametrize("case", VARLEN, ids=[f"D{c[0]}H{c[1]}B{len(c[2])}c{int(c[4])}" for c in VARLEN])
def test_random_varlen(env, case):
    torch, dev, fa, _ = env
    D, H, lq, lk, causal = case
    q, k, v, cq, ck = make_varlen(lq, H, D, 4000 + sum(lq) + D, lengths_k=lk)
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd, cqd, ckd = (torch.from_numpy(x).to(dev) for x in (q, k, v, cq, ck))
    o, lse = fa.fa_fwd_varlen(qd, kd, vd, cqd, ckd, max(lq), max(lk), causal=causal, scale=scale)
    torch.cuda.synchronize()
    O, L = oracle.attention_varlen(q, k, v, cq, ck, causal, scale)
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    fin = np.isfinite(L)
    assert np.isfinite(o).all() and np.array_equal(np.isneginf(lse), ~fin)
    eo = float(np.abs(o - O).max())
    el = float(np.abs(lse[fin] - L[fin]).max()) if fin.any() else 0.0
    print(f"{case}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= O_TOL and el <= LSE_TOL


def draw_backward(n, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for _ in range(n):
        Sq = int(g.integers(1, 400))
        Sk = Sq if g.random() < 0.5 else int(g.integers(1, 400))
        cases.append((int(g.integers(1, 3)), int(g.integers(1, 3)), Sq, Sk, int(g.choice([32, 64, 128, 256])),
                      bool(g.random() < 0.5)))
    return cases


BACKWARD = draw_backward(20, 2027)


@pytest.mark.parametrize("shape", BACKWARD, ids=["x".join(map(str, s)) for s in BACKWARD])
def test_random_backward(env, shape):
    torch, dev, fa, _ = env
    B, H, Sq, Sk, D, causal = shape
    q, k, v = make_qkv(B, H, Sq, Sk, D, seed=5000 + Sq + 3 * Sk + D)
    do = make_qkv(B, H, Sq, 1, D, seed=6000 + Sq + D)[0]
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd, dod = (torch.from_numpy(x).to(dev) for x in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    got = [x.float().cpu().numpy() for x in (dq, dk, dv)]
    backward_check(got, oracle.attention_backward(q, k, v, do, causal, scale),
                   term_magnitudes(q, k, v, do, causal, scale), f"{shape}")


def draw_decode(n, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for _ in range(n):
        S = int(g.integers(1, 2500))
        bs = int(2 ** g.integers(0, 9))
        ns = int(g.choice([0, 1, 2, 3, 5, 8, 17, 64]))
        cases.append((int(g.choice([32, 64, 128, 256])), int(g.integers(1, 4)), int(g.integers(1, 4)), S, bs,
                      min(ns, S), bool(g.random() < 0.5), int(g.integers(1 << 30))))
    return cases


DECODE = draw_decode(60, 2028)


@pytest.mark.parametrize("case", DECODE, ids=[f"D{c[0]}S{c[3]}bs{c[4]}ns{c[5]}" for c in DECODE])
def test_random_decode(env, case):
    torch, dev, fa, _ = env
    D, B, H, S, bs, ns, same, seed = case
    g = np.random.Generator(np.random.PCG64(seed))
    q, k, v = make_qkv(B, H, 1, S, D, seed % 100000)
    max_blocks = -(-S // bs)
    tables, nb = paged_layout(B, max_blocks, seed % 99991, spare=2)
    kc, vc = to_pages(k, tables, nb, bs), to_pages(v, tables, nb, bs)
    if same:
        lens = np.full(B, S, np.int32)
    else:
        # contexts stay within the S keys the pages hold (later rows are
        # NaN); a huge length is clamped to the table's reach, which is S
        # only when S fills its last page; one page may be absent
        lens = g.integers(-2, S + 1, size=B).astype(np.int32)
        if S % bs == 0:
            lens[g.integers(0, B)] = 10 ** 6
        tables = tables.copy()
        tables[g.integers(0, B), g.integers(0, max_blocks)] = int(g.choice([-1, nb, 2 ** 30]))
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd, kcd, vcd, td, sd = (torch.from_numpy(np.ascontiguousarray(x)).to(dev)
                                    for x in (q, k, v, kc, vc, tables, lens))
    op, lp = fa.fa_decode_paged(qd, kcd, vcd, td, sd, scale=scale, num_splits=ns)
    torch.cuda.synchronize()
    O, L = oracle.decode_paged(q, kc, vc, tables, lens, scale)
    o, lse = op.float().cpu().numpy(), lp.cpu().numpy()
    fin = np.isfinite(L)
    assert np.isfinite(o).all() and np.array_equal(np.isneginf(lse), ~fin)
    eo = float(np.abs(o - O).max())
    el = float(np.abs(lse[fin] - L[fin]).max()) if fin.any() else 0.0
    print(f"{case}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= O_TOL and el <= LSE_TOL
    if same:
        oc, lc = fa.fa_decode_splitkv(qd, kd, vd, scale=scale, num_splits=ns)
        torch.cuda.synchronize()
        assert torch.equal(oc, op) and torch.equal(lc, lp), "paged and contiguous decoding differ"
