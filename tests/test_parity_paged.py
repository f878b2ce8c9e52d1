"""GPU parity of paged decoding (fa_decode_paged) against the CPU fp64 oracle.

Same bar as the other parity tests: max |O - O_oracle| <= 2e-3 and
max |LSE - LSE_oracle| <= 1e-3 on the same seeded inputs.  Pages that no
table entry names, and the rows of a page past a sequence's context, hold
NaN or unrelated data, so a read outside the context shows in the result.
The full 8K shape (16 sequences x 32 heads x 8192 tokens, 16-token pages in
random physical order) is checked on sampled (sequence, head) rows against
the oracle and bit for bit against contiguous split-KV decoding of the same
K / V with the same split count.
"""
import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, PAGED_BLOCK_SIZE, PAGED_PERM_SEED, make_qkv, paged_layout, to_pages

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


def gpu_paged(torch_dev, fa, q, kc, vc, tables, seq_lens, scale, ns):
    torch, _ = torch_dev
    qd, kd, vd, td, sd = to_dev(torch_dev, q, kc, vc, tables.astype(np.int32), seq_lens.astype(np.int32))
    o, lse = fa.fa_decode_paged(qd, kd, vd, td, sd, scale=scale, num_splits=ns)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def check(o, lse, O, L, what):
    fin = np.isfinite(L)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    assert np.array_equal(np.isneginf(lse), ~fin), f"{what}: -inf pattern of lse differs"
    eo = float(np.abs(o - O).max())
    el = float(np.abs(lse[fin] - L[fin]).max()) if fin.any() else 0.0
    print(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= O_TOL, f"{what}: max|dO| = {eo:.3e}"
    assert el <= LSE_TOL, f"{what}: max|dLSE| = {el:.3e}"


def case(B, H, S, D, bs, seed, spare=5):
    q, k, v = make_qkv(B, H, 1, S, D, seed)
    max_blocks = -(-S // bs)
    tables, nb = paged_layout(B, max_blocks, seed + 1000, spare=spare)
    return q, to_pages(k, tables, nb, bs), to_pages(v, tables, nb, bs), tables


CASES = [
    # B, H, S (table reach), block_size, seq_lens
    (3, 4, 200, 16, [200, 1, 17]),
    (2, 2, 333, 1, [333, 100]),
    (4, 3, 256, 64, [256, 64, 65, 3]),
    (2, 5, 1000, 32, [999, 512]),
    (1, 2, 64, 1024, [40]),
]


@pytest.mark.parametrize("D", [32, 64, 128, 256])
@pytest.mark.parametrize("cs", CASES, ids=[f"B{c[0]}H{c[1]}S{c[2]}bs{c[3]}" for c in CASES])
@pytest.mark.parametrize("ns", [0, 1, 3, 8])
def test_paged_parity(torch_dev, fa, D, cs, ns):
    B, H, S, bs, lens = cs
    q, kc, vc, tables = case(B, H, S, D, bs, 21 + D + B)
    seq_lens = np.array(lens, dtype=np.int32)
    scale = 1.0 / np.sqrt(D)
    o, lse = gpu_paged(torch_dev, fa, q, kc, vc, tables, seq_lens, scale, ns)
    O, L = oracle.decode_paged(q, kc, vc, tables, seq_lens, scale)
    check(o, lse, O, L, f"paged D={D} {cs} ns={ns}")


def test_paged_long_partition_segments(torch_dev, fa):
    # one-token pages and one partition of 3000 keys: the table of the
    # partition is staged through LDS in three segments
    B, H, S, D, bs = 2, 2, 3000, 128, 1
    q, kc, vc, tables = case(B, H, S, D, bs, 31)
    seq_lens = np.array([3000, 2047], dtype=np.int32)
    o, lse = gpu_paged(torch_dev, fa, q, kc, vc, tables, seq_lens, 0.1, 1)
    O, L = oracle.decode_paged(q, kc, vc, tables, seq_lens, 0.1)
    check(o, lse, O, L, "segments")


@pytest.mark.parametrize("ns", [0, 1, 3])   # 1: the single-kernel form merges in LDS
@pytest.mark.parametrize("D", [64, 128])     # 16-token pages: 2 and 1 pages per wavefront iteration
def test_paged_absent_and_out_of_range_pages(torch_dev, fa, ns, D):
    B, H, S, bs = 3, 2, 96, 16
    q, kc, vc, tables = case(B, H, S, D, bs, 41)
    tables = tables.copy()
    tables[0, 1] = -1
    tables[1, 0] = kc.shape[0]       # one past the last page
    tables[2, :] = 2 ** 30           # every page of sequence 2 absent -> empty
    seq_lens = np.array([96, 80, 96], dtype=np.int32)
    o, lse = gpu_paged(torch_dev, fa, q, kc, vc, tables, seq_lens, 0.125, ns)
    O, L = oracle.decode_paged(q, kc, vc, tables, seq_lens, 0.125)
    check(o, lse, O, L, f"absent pages ns={ns}")
    assert (o[2] == 0).all() and np.isneginf(lse[2]).all()


@pytest.mark.parametrize("ns", [1, 3])
def test_paged_empty_and_clamped_contexts(torch_dev, fa, ns):
    B, H, S, D, bs = 4, 2, 48, 128, 16
    q, kc, vc, tables = case(B, H, S, D, bs, 51)
    seq_lens = np.array([0, -7, 10 ** 6, 48], dtype=np.int32)
    o, lse = gpu_paged(torch_dev, fa, q, kc, vc, tables, seq_lens, 0.2, ns)
    O, L = oracle.decode_paged(q, kc, vc, tables, seq_lens, 0.2)
    check(o, lse, O, L, f"empty / clamped ns={ns}")
    assert (o[:2] == 0).all() and np.isneginf(lse[:2]).all()


@pytest.fixture(scope="module")
def paged_8k(torch_dev):
    """The 8K decode inputs on the GPU, contiguous and in 16-token pages."""
    torch, dev = torch_dev
    w = WORKLOADS["decode_8k"]
    q, k, v = make_qkv(w.B, w.H, w.Sq, w.Sk, w.D, w.seed)
    bs = PAGED_BLOCK_SIZE
    max_blocks = w.Sk // bs
    tables, nb = paged_layout(w.B, max_blocks, PAGED_PERM_SEED)
    qd, kd, vd, td = to_dev(torch_dev, q, k, v, tables)
    # pages built on the GPU: logical block j of sequence b -> page tables[b, j]
    idx = td.reshape(-1).long()
    kc = torch.empty((nb, w.H, bs, w.D), dtype=torch.float16, device=dev)
    vc = torch.empty_like(kc)
    kc[idx] = kd.view(w.B, w.H, max_blocks, bs, w.D).permute(0, 2, 1, 3, 4).reshape(-1, w.H, bs, w.D)
    vc[idx] = vd.view(w.B, w.H, max_blocks, bs, w.D).permute(0, 2, 1, 3, 4).reshape(-1, w.H, bs, w.D)
    sl = torch.full((w.B,), w.Sk, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    return w, (q, k, v, tables), (qd, kd, vd, kc, vc, td, sl)


def test_paged_8k_matches_contiguous_bitwise(torch_dev, fa, paged_8k):
    torch, _ = torch_dev
    w, _, (qd, kd, vd, kc, vc, td, sl) = paged_8k
    for ns in (4, 0):
        op, lp = fa.fa_decode_paged(qd, kc, vc, td, sl, scale=w.scale, num_splits=ns)
        oc, lc = fa.fa_decode_splitkv(qd, kd, vd, scale=w.scale, num_splits=ns)
        torch.cuda.synchronize()
        assert torch.equal(op, oc), f"ns={ns}: O differs from contiguous decoding"
        assert torch.equal(lp, lc), f"ns={ns}: LSE differs from contiguous decoding"


def test_paged_8k_sampled_against_oracle(torch_dev, fa, paged_8k):
    torch, _ = torch_dev
    w, (q, k, v, tables), (qd, kd, vd, kc, vc, td, sl) = paged_8k
    o, lse = fa.fa_decode_paged(qd, kc, vc, td, sl, scale=w.scale)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    gen = np.random.Generator(np.random.PCG64(77))
    picks = {(0, 0), (w.B - 1, w.H - 1)} | {(int(gen.integers(w.B)), int(gen.integers(w.H))) for _ in range(10)}
    for b, h in sorted(picks):
        # the oracle on the pages of this (sequence, head), rebuilt on the host
        kc_h = to_pages(k[b : b + 1, h : h + 1], tables[b : b + 1], int(tables.max()) + 1, PAGED_BLOCK_SIZE)
        vc_h = to_pages(v[b : b + 1, h : h + 1], tables[b : b + 1], int(tables.max()) + 1, PAGED_BLOCK_SIZE)
        O, L = oracle.decode_paged(q[b : b + 1, h : h + 1], kc_h, vc_h, tables[b : b + 1],
                                   np.array([w.Sk], dtype=np.int32), w.scale)
        check(o[b : b + 1, h : h + 1], lse[b : b + 1, h : h + 1], O, L, f"8k paged b={b} h={h}")


# (D, block_size, context, ns): pages holding a whole wavefront group of keys
# (16 keys at D = 128 and 256, 32 at D = 64, 64 at D = 32) take the
# per-group translation, smaller pages the per-key one; ns > 1 with a context
# that ns does not divide starts partitions between groups; 40000 / 70000
# keys at 16-token pages and 5000 at 1-token pages stage the table in
# several segments.
BITWISE_CASES = [
    (128, 16, 1000, 3),
    (128, 4, 1000, 3),
    (64, 32, 1000, 3),
    (64, 16, 1000, 5),
    (32, 64, 777, 3),
    (32, 16, 777, 1),
    (256, 16, 1000, 3),
    (256, 8, 1000, 1),
    (128, 16, 40000, 1),
    (128, 16, 70000, 2),
    (128, 1, 5000, 1),
    (128, 1, 5000, 2),
]


@pytest.mark.parametrize("cs", BITWISE_CASES, ids=[f"D{c[0]}bs{c[1]}S{c[2]}ns{c[3]}" for c in BITWISE_CASES])
def test_paged_matches_contiguous_bitwise(torch_dev, fa, cs):
    # the same keys in the same order per lane: paged and contiguous decoding
    # of one K / V agree bit for bit at any split count and page size
    torch, _ = torch_dev
    D, bs, S, ns = cs
    B, H = 2, 2
    q, k, v = make_qkv(B, H, 1, S, D, 81 + D + bs)
    max_blocks = -(-S // bs)
    tables, nb = paged_layout(B, max_blocks, 91 + bs, spare=3)
    kc, vc = to_pages(k, tables, nb, bs), to_pages(v, tables, nb, bs)
    qd, kd, vd, kcd, vcd, td = to_dev(torch_dev, q, k, v, kc, vc, tables)
    sd = torch.full((B,), S, dtype=torch.int32, device=qd.device)
    scale = 1.0 / np.sqrt(D)
    op, lp = fa.fa_decode_paged(qd, kcd, vcd, td, sd, scale=scale, num_splits=ns)
    oc, lc = fa.fa_decode_splitkv(qd, kd, vd, scale=scale, num_splits=ns)
    torch.cuda.synchronize()
    assert torch.equal(op, oc), f"{cs}: O differs from contiguous decoding"
    assert torch.equal(lp, lc), f"{cs}: LSE differs from contiguous decoding"
    if S <= 1000:
        O, L = oracle.decode_paged(q, kc, vc, tables, np.full(B, S, dtype=np.int32), scale)
        check(op.float().cpu().numpy(), lp.cpu().numpy(), O, L, f"bitwise case {cs}")


@pytest.mark.parametrize("D", [32, 128, 256])
def test_paged_many_partitions(torch_dev, fa, D):
    # 64 partitions per slice: the merge runs its 1024-thread form (more
    # than 4 partitions per group at 256 threads for D >= 64)
    B, H, S, bs = 2, 3, 3000, 16
    q, kc, vc, tables = case(B, H, S, D, bs, 71 + D)
    seq_lens = np.array([3000, 1777], dtype=np.int32)
    scale = 1.0 / np.sqrt(D)
    o, lse = gpu_paged(torch_dev, fa, q, kc, vc, tables, seq_lens, scale, 64)
    O, L = oracle.decode_paged(q, kc, vc, tables, seq_lens, scale)
    check(o, lse, O, L, f"paged D={D} ns=64")


def test_paged_bitwise_repeatable(torch_dev, fa):
    torch, _ = torch_dev
    q, kc, vc, tables = case(2, 3, 500, 128, 16, 61)
    seq_lens = np.array([500, 123], dtype=np.int32)
    qd, kd, vd, td, sd = to_dev(torch_dev, q, kc, vc, tables, seq_lens)
    o1, l1 = fa.fa_decode_paged(qd, kd, vd, td, sd, num_splits=4)
    o2, l2 = fa.fa_decode_paged(qd, kd, vd, td, sd, num_splits=4)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_errors_raise(torch_dev, fa):
    torch, dev = torch_dev
    q, kc, vc, tables = case(1, 2, 32, 64, 16, 71)
    qd, kd, vd, td = to_dev(torch_dev, q, kc, vc, tables)
    sd = torch.tensor([32], dtype=torch.int32, device=dev)
    with pytest.raises(fa.FAError) as e:
        fa.fa_decode_paged(qd, kd, vd, td, sd, num_splits=10 ** 6)
    assert e.value.status == fa.FA_ERR_INVALID_ARG
    bad = torch.zeros((kc.shape[0], 2, 12, 64), dtype=torch.float16, device=dev)  # block_size 12
    with pytest.raises(fa.FAError) as e:
        fa.fa_decode_paged(qd, bad, bad, td, sd)
    assert e.value.status == fa.FA_ERR_INVALID_ARG
    q96 = torch.zeros((1, 2, 1, 96), dtype=torch.float16, device=dev)
    c96 = torch.zeros((kc.shape[0], 2, 16, 96), dtype=torch.float16, device=dev)
    with pytest.raises(fa.FAError) as e:
        fa.fa_decode_paged(q96, c96, c96, td, sd)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
