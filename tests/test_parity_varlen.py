"""GPU parity of packed variable-length prefill (fa_fwd_varlen) against the
CPU fp64 oracle.

Same bar as the other parity tests: max |O - O_oracle| <= 2e-3 and
max |LSE - LSE_oracle| <= 1e-3.  Batches mix lengths that hit every tile
edge (1, a partial tile, exact tiles, many tiles), unequal query and key
lengths, empty sequences and both mask settings.  Rows that no sequence
covers are pre-filled with a sentinel that must survive.  The full ragged
LLaMA-shaped batch (16 sequences of 256..4096 tokens, 32 heads, D = 128) is
checked on sampled rows and on whole heads of its longest and shortest
sequences, and against dense fa_fwd on each sequence alone, bit for bit.
"""
import numpy as np
import pytest

import oracle
from workloads import (VARLEN_B, VARLEN_D, VARLEN_H, VARLEN_LEN_SEED, VARLEN_MAX, VARLEN_MIN, VARLEN_SEED,
                       make_varlen, varlen_lengths)

pytestmark = pytest.mark.gpu

O_TOL = 2e-3
LSE_TOL = 1e-3
SENTINEL = 7.0


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


def gpu_varlen(torch_dev, fa, q, k, v, cu_q, cu_k, max_q, max_k, causal, scale):
    torch, dev = torch_dev
    qd, kd, vd, cqd, ckd = to_dev(torch_dev, q, k, v, cu_q.astype(np.int32), cu_k.astype(np.int32))
    o = torch.full(qd.shape, SENTINEL, dtype=torch.float16, device=dev)
    lse = torch.full((q.shape[1], q.shape[0]), SENTINEL, dtype=torch.float32, device=dev)
    fa.fa_fwd_varlen(qd, kd, vd, cqd, ckd, max_q, max_k, o=o, lse=lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def check(o, lse, O, L, what):
    covered = ~np.isnan(L)                  # [H, total_q]
    rows = covered.any(axis=0)
    assert (o[~rows] == SENTINEL).all() and (lse[:, ~rows] == SENTINEL).all(), f"{what}: uncovered rows written"
    o, O, lse, L = o[rows], O[rows], lse[:, rows], L[:, rows]
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    fin = np.isfinite(L)
    assert np.array_equal(np.isneginf(lse), ~fin), f"{what}: -inf pattern of lse differs"
    eo = float(np.abs(o - O).max()) if o.size else 0.0
    el = float(np.abs(lse[fin] - L[fin]).max()) if fin.any() else 0.0
    print(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= O_TOL, f"{what}: max|dO| = {eo:.3e}"
    assert el <= LSE_TOL, f"{what}: max|dLSE| = {el:.3e}"


BATCHES = [
    # query lengths, key lengths (None = same), heads
    ([1, 65, 300, 128, 257], None, 3),
    ([1000, 1], None, 2),
    ([77, 0, 333, 64], [100, 5, 333, 0], 2),     # cross lengths, an empty query and an empty key sequence
    ([256] * 6, None, 4),
    ([513, 2, 1024, 31], [600, 2, 1000, 31], 2),
]


@pytest.mark.parametrize("D", [32, 64, 128, 256])
@pytest.mark.parametrize("bt", BATCHES, ids=[f"b{i}" for i in range(len(BATCHES))])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_parity(torch_dev, fa, D, bt, causal):
    lq, lk, H = bt
    q, k, v, cu_q, cu_k = make_varlen(lq, H, D, 500 + D + len(lq), lengths_k=lk)
    scale = 1.0 / np.sqrt(D)
    max_q = max(lq)
    max_k = max(lk if lk is not None else lq)
    o, lse = gpu_varlen(torch_dev, fa, q, k, v, cu_q, cu_k, max_q, max_k, causal, scale)
    O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, causal, scale)
    check(o, lse, O, L, f"varlen D={D} {bt} causal={causal}")


def test_varlen_untrusted_cumulative_lengths(torch_dev, fa):
    # starts below 0 and ends past the tensors are clamped; max_seqlen_q cuts
    # query rows (those rows stay untouched); a gap between sequences stays
    # untouched as well
    q, k, v, _, _ = make_varlen([10, 20, 30], 2, 128, 601)
    cu_q = np.array([-5, 10, 25, 10 ** 6], dtype=np.int64)   # rows 25.. of seq 1 never covered
    cu_k = np.array([0, 10, 30, 60], dtype=np.int64)
    for max_q in (60, 12):
        o, lse = gpu_varlen(torch_dev, fa, q, k, v, cu_q, cu_k, max_q, 60, True, 0.1)
        O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, True, 0.1, max_q=max_q, max_k=60)
        check(o, lse, O, L, f"clamps max_q={max_q}")


@pytest.fixture(scope="module")
def ragged_llama(torch_dev, fa):
    torch, _ = torch_dev
    lens = varlen_lengths(VARLEN_B, VARLEN_MIN, VARLEN_MAX, VARLEN_LEN_SEED)
    q, k, v, cu_q, cu_k = make_varlen(lens, VARLEN_H, VARLEN_D, VARLEN_SEED)
    qd, kd, vd, cqd, ckd = to_dev(torch_dev, q, k, v, cu_q, cu_k)
    scale = 1.0 / np.sqrt(VARLEN_D)
    o, lse = fa.fa_fwd_varlen(qd, kd, vd, cqd, ckd, int(lens.max()), int(lens.max()), causal=True, scale=scale)
    torch.cuda.synchronize()
    return lens, (q, k, v, cu_q), (qd, kd, vd), (o, lse), scale


def test_ragged_llama_sampled_rows(ragged_llama):
    lens, (q, k, v, cu), _, (o, lse), scale = ragged_llama
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    gen = np.random.Generator(np.random.PCG64(88))
    picks = [(0, 0, 0), (VARLEN_B - 1, VARLEN_H - 1, int(lens[-1]) - 1)]
    picks += [(int(b), int(gen.integers(VARLEN_H)), int(gen.integers(lens[b]))) for b in gen.integers(VARLEN_B, size=40)]
    for b, h, i in picks:
        s0, n = int(cu[b]), int(lens[b])
        tb = lambda x: np.transpose(x[s0 : s0 + n], (1, 0, 2))[None]
        O, L = oracle.attention_rows(tb(q), tb(k), tb(v), True, scale, [(0, h, i)])
        eo = float(np.abs(o[s0 + i, h] - O[0]).max())
        el = abs(float(lse[h, s0 + i]) - float(L[0]))
        assert eo <= O_TOL and el <= LSE_TOL, f"seq {b} head {h} row {i}: {eo:.3e} {el:.3e}"


@pytest.mark.parametrize("which", ["longest", "shortest"])
def test_ragged_llama_whole_head(ragged_llama, which):
    lens, (q, k, v, cu), _, (o, lse), scale = ragged_llama
    b = int(np.argmax(lens) if which == "longest" else np.argmin(lens))
    s0, n = int(cu[b]), int(lens[b])
    h = 5
    tb = lambda x: np.transpose(x[s0 : s0 + n, h : h + 1], (1, 0, 2))[None]
    O, L = oracle.attention(tb(q), tb(k), tb(v), True, scale)
    oo = o[s0 : s0 + n, h].float().cpu().numpy()
    ll = lse[h, s0 : s0 + n].cpu().numpy()
    eo = float(np.abs(oo - O[0, 0]).max())
    el = float(np.abs(ll - L[0, 0]).max())
    print(f"{which} seq {b} (len {n}) head {h}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= O_TOL and el <= LSE_TOL


def test_ragged_llama_matches_dense_per_sequence(torch_dev, fa, ragged_llama):
    # each sequence alone through fa_fwd ([1, H, n, D]) gives the same bits
    torch, _ = torch_dev
    lens, (q, k, v, cu), (qd, kd, vd), (o, lse), scale = ragged_llama
    for b in (0, int(np.argmax(lens)), VARLEN_B - 1):
        s0, n = int(cu[b]), int(lens[b])
        sl = lambda x: x[s0 : s0 + n].permute(1, 0, 2).unsqueeze(0).contiguous()
        od, ld = fa.fa_fwd(sl(qd), sl(kd), sl(vd), causal=True, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(od[0].permute(1, 0, 2), o[s0 : s0 + n]), f"sequence {b}: O differs from dense"
        assert torch.equal(ld[0], lse[:, s0 : s0 + n]), f"sequence {b}: LSE differs from dense"


def test_varlen_errors_raise(torch_dev, fa):
    torch, dev = torch_dev
    q = torch.zeros((10, 2, 96), dtype=torch.float16, device=dev)
    cu = torch.tensor([0, 10], dtype=torch.int32, device=dev)
    with pytest.raises(fa.FAError) as e:
        fa.fa_fwd_varlen(q, q, q, cu, cu, 10, 10)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    q = torch.zeros((10, 2, 64), dtype=torch.float16, device=dev)
    with pytest.raises(fa.FAError) as e:
        fa.fa_fwd_varlen(q, q, q, cu, cu, 0, 10)
    assert e.value.status == fa.FA_ERR_INVALID_ARG
    with pytest.raises(fa.FAError) as e:
        fa.fa_fwd_varlen(q, q, q, cu, cu, 2 ** 30, 10)
    assert e.value.status == fa.FA_ERR_INVALID_ARG
