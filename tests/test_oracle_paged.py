"""Pins for the paged-decoding oracle (no GPU).

``oracle.paged.decode_paged`` gathers each sequence's context out of the
pages and applies the dense definition.  It is pinned against:
  * an independent scalar-loop evaluation that looks every token up in the
    block table itself (``oracle.brute.decode_paged_brute``);
  * the already-pinned dense oracle on the contiguous K / V the pages were
    cut from (identity of content, any physical order);
  * truncation (a shorter context equals dense attention on a key prefix),
    invariance under relabelling the physical pages, NaN in pages no table
    entry names, and the empty-context convention.
The last test plants plausible gather mistakes and checks a pin catches each.
"""
import numpy as np
import pytest

import oracle
from oracle import dense as od
from oracle import paged as op
from workloads import make_qkv, paged_layout, to_pages


def _paged_case(B, H, S, D, bs, seed, spare=3):
    """Contiguous draws, their pages, and the tables (distinct random pages)."""
    q, k, v = make_qkv(B, H, 1, S, D, seed)
    max_blocks = -(-S // bs)
    tables, nb = paged_layout(B, max_blocks, seed + 100, spare=spare)
    return q, k, v, to_pages(k, tables, nb, bs), to_pages(v, tables, nb, bs), tables


# ---------------------------------------------------------------- pin suite

def pin_brute():
    # ragged contexts incl. 0, 1, a block boundary and the full reach; an
    # absent page (-1) and an out-of-range page id; block sizes 1, 2, 4
    for (B, H, S, D, bs, seed) in [(3, 2, 9, 4, 2, 1), (2, 3, 8, 3, 4, 2), (2, 1, 5, 8, 1, 3)]:
        q, k, v, kc, vc, tables = _paged_case(B, H, S, D, bs, seed)
        tables = tables.copy()
        nb = kc.shape[0]
        seq_lens = np.array([S, 1, 0][:B] if B == 3 else [S - 1, bs + 1][:B], dtype=np.int32)
        tables[0, 1] = -1          # tokens bs .. 2bs-1 of sequence 0 absent
        if tables.shape[1] > 2:
            tables[0, 2] = nb + 5  # out of range: absent as well
        scale = 0.4
        O, L = op.decode_paged(q, kc, vc, tables, seq_lens, scale)
        Ob, Lb = oracle.decode_paged_brute(q.astype(np.float64).tolist(), kc.astype(np.float64).tolist(),
                                           vc.astype(np.float64).tolist(), tables.tolist(), seq_lens.tolist(), scale)
        np.testing.assert_allclose(O, np.array(Ob), rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(np.isinf(L), np.isinf(np.array(Lb)))
        fin = np.isfinite(L)
        np.testing.assert_allclose(L[fin], np.array(Lb)[fin], rtol=1e-12, atol=1e-12)


def pin_contiguous_equivalence():
    # full contexts: paged decoding = dense attention on the contiguous K / V
    for (B, H, S, D, bs, seed) in [(2, 3, 37, 8, 4, 4), (3, 2, 64, 16, 16, 5), (1, 4, 7, 5, 8, 6)]:
        q, k, v, kc, vc, tables = _paged_case(B, H, S, D, bs, seed)
        seq_lens = np.full(B, S, dtype=np.int32)
        O, L = op.decode_paged(q, kc, vc, tables, seq_lens, 0.3)
        Od, Ld = od.attention(q, k, v, False, 0.3)
        np.testing.assert_allclose(O, Od, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(L, Ld, rtol=1e-12, atol=1e-12)


def pin_truncation():
    B, H, S, D, bs = 3, 2, 50, 8, 8
    q, k, v, kc, vc, tables = _paged_case(B, H, S, D, bs, 7)
    seq_lens = np.array([50, 17, 8], dtype=np.int32)
    O, L = op.decode_paged(q, kc, vc, tables, seq_lens, 0.25)
    for b, n in enumerate(seq_lens):
        Od, Ld = od.attention(q[b : b + 1], k[b : b + 1, :, :n], v[b : b + 1, :, :n], False, 0.25)
        np.testing.assert_allclose(O[b : b + 1], Od, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(L[b : b + 1], Ld, rtol=1e-12, atol=1e-12)


def pin_page_relabelling():
    # moving the pages to other physical slots (and fixing the tables) changes nothing
    B, H, S, D, bs = 2, 2, 30, 4, 4
    q, k, v, kc, vc, tables = _paged_case(B, H, S, D, bs, 8, spare=0)
    perm = np.random.Generator(np.random.PCG64(9)).permutation(kc.shape[0])
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    seq_lens = np.array([30, 13], dtype=np.int32)
    O1, L1 = op.decode_paged(q, kc, vc, tables, seq_lens, 0.5)
    O2, L2 = op.decode_paged(q, kc2, vc2, perm[tables].astype(np.int32), seq_lens, 0.5)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)


def pin_unnamed_pages_unread():
    B, H, S, D, bs = 2, 2, 20, 4, 4
    q, k, v, kc, vc, tables = _paged_case(B, H, S, D, bs, 10, spare=4)
    named = set(tables.ravel().tolist())
    unnamed = [p for p in range(kc.shape[0]) if p not in named]
    assert unnamed and np.isnan(kc[unnamed]).all()  # to_pages left them NaN
    O, L = op.decode_paged(q, kc, vc, tables, np.array([20, 20], dtype=np.int32), 0.5)
    assert np.isfinite(O).all() and np.isfinite(L).all()


def pin_empty_context():
    B, H, S, D, bs = 2, 3, 8, 4, 4
    q, k, v, kc, vc, tables = _paged_case(B, H, S, D, bs, 11)
    O, L = op.decode_paged(q, kc, vc, tables, np.array([0, -5], dtype=np.int32), 0.5)
    assert (O == 0).all() and np.isneginf(L).all()
    # a context longer than the table's reach is clamped to it
    O1, L1 = op.decode_paged(q, kc, vc, tables, np.array([S, S], dtype=np.int32), 0.5)
    O2, L2 = op.decode_paged(q, kc, vc, tables, np.array([10 ** 6, S], dtype=np.int32), 0.5)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)


PINS = [
    pin_brute,
    pin_contiguous_equivalence,
    pin_truncation,
    pin_page_relabelling,
    pin_unnamed_pages_unread,
    pin_empty_context,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def test_layout_helpers():
    tables, nb = paged_layout(3, 4, 1, spare=2)
    assert tables.dtype == np.int32 and tables.shape == (3, 4) and nb == 14
    assert len(set(tables.ravel().tolist())) == 12 and tables.min() >= 0 and tables.max() < nb
    x = np.arange(3 * 2 * 10 * 4, dtype=np.float32).reshape(3, 2, 10, 4).astype(np.float16)
    pages = to_pages(x, tables, nb, 4)
    # token t of sequence b is at page tables[b, t // 4], row t % 4
    for b in range(3):
        for t in range(10):
            np.testing.assert_array_equal(pages[tables[b, t // 4], :, t % 4, :], x[b, :, t, :])


# -------------------------------------------------- planted mistakes (mutants)

def _mut_row_block_swapped(orig):
    # page index from t % bs and row from t // bs
    def f(table_row, seq_len, block_size, num_blocks):
        L = int(min(max(int(seq_len), 0), len(table_row) * block_size))
        toks, pages, rows = [], [], []
        for t in range(L):
            j, r = t % len(table_row), min(t // len(table_row), block_size - 1)
            p = int(table_row[j])
            if 0 <= p < num_blocks:
                toks.append(t)
                pages.append(p)
                rows.append(r)
        return toks, pages, rows
    return f


def _mut_off_by_one_context(orig):
    return lambda table_row, seq_len, block_size, num_blocks: orig(table_row, int(seq_len) + 1, block_size,
                                                                    num_blocks)


def _mut_physical_not_translated(orig):
    # uses the logical block number as the page
    def f(table_row, seq_len, block_size, num_blocks):
        L = int(min(max(int(seq_len), 0), len(table_row) * block_size))
        toks = list(range(L))
        return toks, [t // block_size for t in toks], [t % block_size for t in toks]
    return f


def _mut_absent_read_as_zero_page(orig):
    # treats an absent entry as page 0 instead of skipping it
    def f(table_row, seq_len, block_size, num_blocks):
        fixed = [p if 0 <= int(p) < num_blocks else 0 for p in table_row]
        return orig(fixed, seq_len, block_size, num_blocks)
    return f


MUTANTS = [
    ("context_tokens", _mut_row_block_swapped),
    ("context_tokens", _mut_off_by_one_context),
    ("context_tokens", _mut_physical_not_translated),
    ("context_tokens", _mut_absent_read_as_zero_page),
]


@pytest.mark.parametrize("target,mutant", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(op, target, mutant(getattr(op, target)))
    failed = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {mutant.__name__}"
