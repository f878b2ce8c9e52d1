"""C-ABI checks that need no GPU: the library loads, exports every function
include/fa.h declares, and rejects invalid arguments before any HIP call
(the fake pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

from exact_attention_54_amd import _capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

A = 0x10000  # 16-byte aligned fake device addresses
P = [A, A + 0x1000, A + 0x2000, A + 0x3000, A + 0x4000]
GOOD = dict(B=2, H=3, Sq=5, Sk=7, D=64, causal=0, scale=0.125)


@pytest.fixture(scope="module")
def lib():
    return _capi.load()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(fa_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function(lib):
    names = header_functions()
    assert names == sorted(_capi.SIGNATURES), names
    for n in names:
        assert getattr(lib, n) is not None


def fwd(lib, p=P, **kw):
    a = dict(GOOD, **kw)
    return lib.fa_fwd(p[0], p[1], p[2], p[3], p[4], a["B"], a["H"], a["Sq"], a["Sk"], a["D"], a["causal"],
                      a["scale"], None)


def dec(lib, p=P, ns=2, **kw):
    a = dict(GOOD, Sq=1)
    a.update(kw)
    return lib.fa_decode_splitkv(p[0], p[1], p[2], p[3], p[4], a["B"], a["H"], a["Sq"], a["Sk"], a["D"],
                                 a["causal"], a["scale"], None, ns)


def dec_ws(lib, ws=A + 0x8000, nbytes=1 << 20, p=P, ns=2, **kw):
    a = dict(GOOD, Sq=1)
    a.update(kw)
    return lib.fa_decode_splitkv_ws(p[0], p[1], p[2], p[3], p[4], a["B"], a["H"], a["Sq"], a["Sk"], a["D"],
                                    a["causal"], a["scale"], None, ns, ws, nbytes)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), _capi.FA_ERR_INVALID_ARG),
    (dict(H=-1), _capi.FA_ERR_INVALID_ARG),
    (dict(Sq=0), _capi.FA_ERR_INVALID_ARG),
    (dict(Sk=0), _capi.FA_ERR_INVALID_ARG),
    (dict(D=0), _capi.FA_ERR_INVALID_ARG),
    (dict(D=96), _capi.FA_ERR_UNSUPPORTED),
    (dict(D=16), _capi.FA_ERR_UNSUPPORTED),
    (dict(D=2048), _capi.FA_ERR_UNSUPPORTED),
    (dict(D=384), _capi.FA_ERR_UNSUPPORTED),
    (dict(causal=2), _capi.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), _capi.FA_ERR_INVALID_ARG),
    (dict(scale=-0.5), _capi.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _capi.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), _capi.FA_ERR_INVALID_ARG),
    (dict(B=1 << 20, H=1 << 20, Sq=1 << 10, D=64), _capi.FA_ERR_INVALID_ARG),
])
def test_fwd_rejects(lib, kw, code):
    assert fwd(lib, **kw) == code
    assert _capi.last_error() != ""


@pytest.mark.parametrize("idx", range(5))
def test_fwd_rejects_null(lib, idx):
    p = list(P)
    p[idx] = None
    assert fwd(lib, p=p) == _capi.FA_ERR_INVALID_ARG
    assert "null" in _capi.last_error()


@pytest.mark.parametrize("idx,off", [(0, 8), (1, 4), (2, 2), (3, 8), (4, 2)])
def test_fwd_rejects_misaligned(lib, idx, off):
    p = list(P)
    p[idx] += off
    assert fwd(lib, p=p) == _capi.FA_ERR_INVALID_ARG
    assert "aligned" in _capi.last_error()


def test_lse_needs_only_4_byte_alignment_check(lib):
    # lse at +4 passes alignment; use an invalid D so no HIP call happens
    p = list(P)
    p[4] += 4
    assert fwd(lib, p=p, D=96) == _capi.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,ns", [
    (dict(Sq=2), 2),
    (dict(causal=1), 2),
    (dict(Sk=7), 8),
    (dict(D=96), 2),
    (dict(scale=-1.0), 2),
])
def test_decode_rejects(lib, kw, ns):
    code = _capi.FA_ERR_UNSUPPORTED if kw.get("D") == 96 else _capi.FA_ERR_INVALID_ARG
    a = dict(kw)
    sq = a.pop("Sq", 1)
    assert lib.fa_decode_splitkv(P[0], P[1], P[2], P[3], P[4], GOOD["B"], GOOD["H"], sq, a.get("Sk", GOOD["Sk"]),
                                 a.get("D", 64), a.get("causal", 0), a.get("scale", 0.125), None, ns) == code


def test_decode_ws_rejects(lib):
    need = lib.fa_decode_workspace_bytes(2, 3, 64, 2)
    assert dec_ws(lib, ws=None) == _capi.FA_ERR_INVALID_ARG
    assert dec_ws(lib, ws=A + 0x8008) == _capi.FA_ERR_INVALID_ARG
    assert dec_ws(lib, nbytes=need - 1) == _capi.FA_ERR_INVALID_ARG
    assert "workspace" in _capi.last_error()
    assert dec_ws(lib, Sq=3) == _capi.FA_ERR_INVALID_ARG


def test_workspace_bytes(lib):
    assert lib.fa_decode_workspace_bytes(16, 32, 128, 4) == 16 * 32 * 4 * 129 * 4
    assert lib.fa_decode_workspace_bytes(1, 1, 64, 3) == 1024  # 195 floats -> 780 B -> 1024
    assert lib.fa_decode_workspace_bytes(0, 1, 64, 3) == 0
    assert lib.fa_decode_workspace_bytes(1, 1, 64, 0) == 0


@pytest.mark.parametrize("B,H,Sk,cus,want", [
    (16, 32, 8192, 256, 1),     # 512 slices: two 1024-thread workgroups per CU, no split
    (8, 32, 8192, 256, 8),      # 256 slices x 8 = 2048 workgroups of 256 threads = 8 per CU
    (1, 1, 8192, 256, 32),      # capped so each partition keeps >= 256 keys
    (1, 1, 100, 256, 1),
    (1, 1, 1, 256, 1),
    (64, 64, 8192, 256, 1),     # already 16 slices per CU
    (2, 8, 4096, 304, 16),
    (0, 1, 10, 256, 0),
    (1, 1, 10, 0, 0),
])
def test_auto_splits(lib, B, H, Sk, cus, want):
    assert lib.fa_decode_auto_splits(B, H, Sk, cus) == want


@pytest.mark.parametrize("B,H,Sq,Sk,D,causal,cus,want", [
    (1, 32, 4096, 4096, 128, 1, 256, 1),   # 8-wavefront grid (every CU has a workgroup): never split
    (1, 4, 4096, 4096, 128, 1, 256, 4),    # one GPU's 4 heads of it: 128 tiles, heaviest 32x the lightest
    (1, 2, 8192, 8192, 128, 1, 256, 4),
    (1, 1, 4096, 4096, 64, 1, 256, 4),
    (8, 16, 2048, 2048, 32, 1, 256, 1),    # D = 32 (always 128-row workgroups): 2048 tiles
    (1, 8, 2048, 2048, 128, 0, 256, 1),    # D <= 128 non-causal: measured no gain, never split
    (2, 8, 1024, 1024, 128, 1, 256, 1),    # short tiles: the merge costs what the balance saves
    (1, 16, 2048, 2048, 256, 1, 256, 2),   # D = 256 runs, one per CU: every heavy tile cut once
    (1, 16, 2048, 2048, 256, 0, 256, 1),   # full key range everywhere: every CU equally loaded
    (1, 16, 1024, 1024, 256, 1, 256, 1),   # 128 short tiles: the merge would cost more than it saves
    (1, 8, 4096, 4096, 256, 1, 256, 2),    # heaviest tiles twice the mean: every heavy tile cut once
    (1, 4, 2048, 2048, 256, 0, 256, 4),    # 64 tiles on 256 CUs: four runs each
    (1, 2, 1000, 1000, 256, 1, 256, 8),    # 16 tiles on 256 CUs: runs of 5 key tiles
    (8, 32, 2048, 2048, 256, 1, 256, 1),   # 4096 tiles: more than two per CU, never split
    (1, 4, 512, 512, 1024, 0, 256, 4),     # Split-D: 64 work items -> runs of a quarter tile
    (1, 8, 1024, 1024, 512, 0, 256, 1),    # Split-D: 256 work items fill the CUs
    (1, 8, 1024, 1024, 512, 1, 256, 2),    # Split-D causal: runs, every heavy tile cut once
    (0, 1, 16, 16, 256, 0, 256, 0),        # invalid sizes
    (1, 1, 16, 16, 96, 0, 256, 0),
    (1, 1, 16, 16, 256, 2, 256, 0),
    (1, 1, 16, 16, 256, 0, 0, 0),
])
def test_fwd_key_splits(lib, B, H, Sq, Sk, D, causal, cus, want):
    assert lib.fa_fwd_key_splits(B, H, Sq, Sk, D, causal, cus) == want


def test_fwd_key_splits_stays_within_sensible_bounds(lib):
    # any valid size: at most 8 parts at D = 256, none when the grid already
    # holds more than two workgroups per CU
    for B, H, S, causal in [(1, 1, 1, 0), (1, 1, 129, 1), (1, 3, 777, 1), (2, 5, 3000, 0), (1, 64, 1024, 1)]:
        ns = lib.fa_fwd_key_splits(B, H, S, S, 256, causal, 256)
        assert 1 <= ns <= 8
        if B * H * -(-S // 128) > 512:
            assert ns == 1


def test_fwd_key_splits_properties_on_random_shapes(lib):
    # invariants of the split choice over 2000 seeded shapes: parts in 1..8
    # (D <= 256) or 1..16 (Split-D); non-causal D <= 128 grids and grids
    # with a 256-row tile per CU are never split; invalid sizes give 0
    import numpy as np

    g = np.random.Generator(np.random.PCG64(5))
    for _ in range(2000):
        B, H = int(g.integers(1, 5)), int(g.integers(1, 65))
        Sq, Sk = int(g.integers(1, 20000)), int(g.integers(1, 20000))
        D = int(g.choice([32, 64, 128, 256, 512, 1024]))
        causal = int(g.integers(0, 2))
        cus = int(g.choice([80, 256, 304]))
        ns = lib.fa_fwd_key_splits(B, H, Sq, Sk, D, causal, cus)
        assert 1 <= ns <= (16 if D >= 512 else 8), (B, H, Sq, Sk, D, causal, cus, ns)
        if Sq == 1 and not causal and D <= 256:
            # a decode step: the decode's partitions
            assert ns == lib.fa_decode_auto_splits(B, H, Sk, cus), (B, H, Sk, D, cus, ns)
            continue
        if D in (64, 128) and (not causal or B * H * -(-Sq // 256) >= cus):
            assert ns == 1, (B, H, Sq, Sk, D, causal, cus, ns)
        if D <= 256 and B * H * -(-Sq // 128) > 2 * cus:
            assert ns == 1, (B, H, Sq, Sk, D, causal, cus, ns)
    assert lib.fa_fwd_key_splits(1, 1, 0, 5, 128, 1, 256) == 0
    assert lib.fa_fwd_key_splits(1, 1, 5, 5, 48, 1, 256) == 0


def test_fwd_plan_cache_is_transparent(lib):
    # plans are cached per size tuple in a table of 256 slots: 1200 shapes
    # (every slot reused several times) queried in one order and again in
    # another give identical answers
    import numpy as np

    g = np.random.Generator(np.random.PCG64(11))
    shapes = []
    for _ in range(1200):
        shapes.append((int(g.integers(1, 5)), int(g.integers(1, 33)), int(g.integers(1, 9000)),
                       int(g.integers(1, 9000)), int(g.choice([32, 64, 128, 256, 512, 1024])),
                       int(g.integers(0, 2)), int(g.choice([80, 256, 304]))))

    def answers(order):
        return {shapes[i]: (lib.fa_fwd_key_splits(*shapes[i]), lib.fa_fwd_workspace_bytes(*shapes[i]))
                for i in order}

    first = answers(range(len(shapes)))
    again = answers(g.permutation(len(shapes)))
    assert first == again


def test_fwd_plan_is_cheap_once_cached(lib):
    # the key-split planner simulates its candidate dispatches; a repeated
    # size tuple must not pay for that again (uncached: hundreds of us here)
    import time

    args = (1, 16, 2048, 2048, 256, 1, 256)
    lib.fa_fwd_workspace_bytes(*args)
    t0 = time.perf_counter()
    for _ in range(200):
        lib.fa_fwd_workspace_bytes(*args)
    per_call_us = (time.perf_counter() - t0) / 200 * 1e6
    assert per_call_us < 50, per_call_us


def rup256(n):
    return -(-n // 256) * 256


@pytest.mark.parametrize("B,H,Sq,Sk,D,causal,cus", [
    (1, 32, 4096, 4096, 128, 1, 256),
    (1, 4, 4096, 4096, 128, 1, 256),
    (1, 2, 8192, 8192, 128, 1, 256),
    (1, 16, 1024, 1024, 256, 1, 256),
    (1, 4, 2048, 2048, 256, 0, 256),
    (1, 16, 2048, 2048, 256, 1, 256),
    (1, 4, 512, 512, 1024, 0, 256),
    (1, 8, 1024, 1024, 512, 1, 256),
    (1, 8, 1, 32768, 128, 0, 256),     # a decode step with many partitions
    (16, 32, 1, 8192, 128, 0, 256),    # a decode step with one partition
    (1, 1, 1, 9, 64, 1, 256),          # causal single row: the tile kernel
])
def test_fwd_workspace_bytes(lib, B, H, Sq, Sk, D, causal, cus):
    # the workspace follows the split choice: none without a split; otherwise
    # the fp32 partial rows (D values and one LSE per part) of the split tiles
    ns = lib.fa_fwd_key_splits(B, H, Sq, Sk, D, causal, cus)
    ws = lib.fa_fwd_workspace_bytes(B, H, Sq, Sk, D, causal, cus)
    if ns == 1:
        assert ws == 0
    elif Sq == 1 and not causal:
        assert ws == lib.fa_decode_workspace_bytes(B, H, D, ns) == rup256(B * H * ns * (D + 1) * 4)
    elif D >= 256:
        # runs (32-row tiles for Split-D, 128-row at D = 256): partial O and
        # log2-sum-exp slots for two segments of each of G runs; or, for
        # Split-D, equal key parts of every query row
        bm = 32 if D >= 512 else 128
        runs = any(ws == rup256(g * 2 * bm * D * 4) + rup256(g * 2 * bm * 4) for g in range(1, 2 * cus + 9))
        parts = D >= 512 and ws == rup256(B * H * Sq * ns * (D + 1) * 4)
        assert runs or parts, ws
    else:
        # rows of the split 128-row query tiles: a whole number of tiles per slice
        assert ws % 256 == 0 and ws > 0
        tiles = -(-Sq // 128)
        per_tile = 128 * ns * (D + 1) * 4
        assert any(ws == rup256(B * H * t * per_tile) for t in range(1, tiles + 1)), ws


def test_fwd_workspace_bytes_invalid(lib):
    assert lib.fa_fwd_workspace_bytes(0, 1, 16, 16, 128, 0, 256) == 0
    assert lib.fa_fwd_workspace_bytes(1, 1, 16, 16, 96, 0, 256) == 0
    assert lib.fa_fwd_workspace_bytes(1, 1, 16, 16, 128, 2, 256) == 0
    assert lib.fa_fwd_workspace_bytes(1, 1, 16, 16, 128, 0, 0) == 0


def test_fwd_ws_rejects_before_any_hip_call(lib):
    a = GOOD

    def call(ws, nbytes=1 << 20, **kw):
        b = dict(a, **kw)
        return lib.fa_fwd_ws(P[0], P[1], P[2], P[3], P[4], b["B"], b["H"], b["Sq"], b["Sk"], b["D"], b["causal"],
                             b["scale"], None, ws, nbytes)

    assert call(A + 0x8008) == _capi.FA_ERR_INVALID_ARG    # misaligned workspace
    assert "workspace" in _capi.last_error()
    assert call(A + 0x8000, D=96) == _capi.FA_ERR_UNSUPPORTED
    assert call(A + 0x8000, scale=0.0) == _capi.FA_ERR_INVALID_ARG


def test_status_strings(lib):
    assert _capi.status_name(0) == "ok"
    assert _capi.status_name(1) == "invalid argument"
    assert _capi.status_name(2) == "unsupported head dimension"
    assert _capi.status_name(3) == "HIP error"
    assert _capi.status_name(99) == "unknown status"


def test_python_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    import exact_attention_54_amd as fa

    q = torch.zeros(1, 1, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        fa.fa_fwd(q, q, q)
    with pytest.raises(TypeError):
        fa.fa_fwd(q.float(), q, q)


# ------------------------------------------------ packed (ragged) prefill

VGOOD = dict(B=2, H=3, total_q=9, total_k=11, max_q=5, max_k=6, D=64, causal=1, scale=0.125)
CU = [A + 0x5000, A + 0x6000]  # fake cumulative-length arrays


def varlen(lib, p=P, cu=CU, **kw):
    a = dict(VGOOD, **kw)
    return lib.fa_fwd_varlen(p[0], p[1], p[2], p[3], p[4], cu[0], cu[1], a["B"], a["H"], a["total_q"],
                             a["total_k"], a["max_q"], a["max_k"], a["D"], a["causal"], a["scale"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), _capi.FA_ERR_INVALID_ARG),
    (dict(H=0), _capi.FA_ERR_INVALID_ARG),
    (dict(total_q=0), _capi.FA_ERR_INVALID_ARG),
    (dict(total_k=-3), _capi.FA_ERR_INVALID_ARG),
    (dict(max_q=0), _capi.FA_ERR_INVALID_ARG),
    (dict(max_k=0), _capi.FA_ERR_INVALID_ARG),
    (dict(D=96), _capi.FA_ERR_UNSUPPORTED),
    (dict(causal=3), _capi.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _capi.FA_ERR_INVALID_ARG),
    (dict(max_q=1 << 24, H=64, D=128), _capi.FA_ERR_INVALID_ARG),   # one sequence past 2 GiB
    (dict(max_k=(1 << 24) - 200, H=32, D=128), _capi.FA_ERR_INVALID_ARG),
])
def test_varlen_rejects(lib, kw, code):
    assert varlen(lib, **kw) == code
    assert _capi.last_error() != ""


@pytest.mark.parametrize("idx", range(7))
def test_varlen_rejects_null_and_misaligned(lib, idx):
    ptrs = list(P) + list(CU)
    ptrs[idx] = 0
    assert varlen(lib, p=ptrs[:5], cu=ptrs[5:]) == _capi.FA_ERR_INVALID_ARG
    ptrs = list(P) + list(CU)
    ptrs[idx] += 2  # below every alignment the entry point asks for
    assert varlen(lib, p=ptrs[:5], cu=ptrs[5:]) == _capi.FA_ERR_INVALID_ARG


# ------------------------------------------------------ paged decoding

PGOOD = dict(B=2, H=3, D=64, num_blocks=10, block_size=16, max_blocks=4, scale=0.125, ns=2)
TBL = [A + 0x5000, A + 0x6000]  # fake block table and context lengths


def paged(lib, p=P, t=TBL, **kw):
    a = dict(PGOOD, **kw)
    return lib.fa_decode_paged(p[0], p[1], p[2], t[0], t[1], p[3], p[4], a["B"], a["H"], a["D"],
                               a["num_blocks"], a["block_size"], a["max_blocks"], a["scale"], None, a["ns"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), _capi.FA_ERR_INVALID_ARG),
    (dict(H=0), _capi.FA_ERR_INVALID_ARG),
    (dict(num_blocks=0), _capi.FA_ERR_INVALID_ARG),
    (dict(max_blocks=0), _capi.FA_ERR_INVALID_ARG),
    (dict(block_size=0), _capi.FA_ERR_INVALID_ARG),
    (dict(block_size=12), _capi.FA_ERR_INVALID_ARG),     # not a power of two
    (dict(block_size=2048), _capi.FA_ERR_INVALID_ARG),   # above 1024
    (dict(D=16), _capi.FA_ERR_UNSUPPORTED),
    (dict(scale=-1.0), _capi.FA_ERR_INVALID_ARG),
    (dict(ns=65), _capi.FA_ERR_INVALID_ARG),             # more splits than the table reaches (4 * 16)
    (dict(max_blocks=1 << 21, block_size=1024), _capi.FA_ERR_INVALID_ARG),
])
def test_paged_rejects(lib, kw, code):
    assert paged(lib, **kw) == code
    assert _capi.last_error() != ""


@pytest.mark.parametrize("idx", range(7))
def test_paged_rejects_null_and_misaligned(lib, idx):
    ptrs = list(P[:3]) + list(TBL) + list(P[3:])
    ptrs[idx] = 0
    assert paged(lib, p=ptrs[:3] + ptrs[5:], t=ptrs[3:5]) == _capi.FA_ERR_INVALID_ARG
    ptrs = list(P[:3]) + list(TBL) + list(P[3:])
    ptrs[idx] += 2
    assert paged(lib, p=ptrs[:3] + ptrs[5:], t=ptrs[3:5]) == _capi.FA_ERR_INVALID_ARG


def bwd(lib, **kw):
    a = dict(GOOD, **kw)
    return lib.fa_bwd(P[0], P[1], P[2], P[3], P[4], A + 0x5000, A + 0x6000, A + 0x7000, A + 0x8000, a["B"], a["H"],
                      a["Sq"], a["Sk"], a["D"], a["causal"], a["scale"], None)


@pytest.mark.parametrize("D", [16, 48, 96, 512, 1024])
def test_bwd_rejects_head_dims_without_a_kernel(lib, D):
    # every head dim the backward has no kernel for is refused before any HIP
    # call (the fake pointers are never touched)
    assert bwd(lib, D=D) == _capi.FA_ERR_UNSUPPORTED
    assert "head dim" in _capi.last_error()


@pytest.mark.parametrize("B,H,Sq,D", [(1, 32, 4096, 128), (2, 3, 5, 64), (1, 2, 129, 32), (1, 16, 2048, 256)])
def test_bwd_workspace_bytes(lib, B, H, Sq, D):
    # one fp32 D and one fp32 LSE (log2 units) per query row
    assert lib.fa_bwd_workspace_bytes(B, H, Sq, D) == rup256(B * H * Sq * 8)


def test_bwd_workspace_bytes_invalid(lib):
    assert lib.fa_bwd_workspace_bytes(0, 1, 16, 64) == 0
    assert lib.fa_bwd_workspace_bytes(1, 1, 16, 96) == 0
    assert lib.fa_bwd_workspace_bytes(1, 1, 16, 512) == 0


def test_bwd_ws_rejects_before_any_hip_call(lib):
    a = GOOD
    need = lib.fa_bwd_workspace_bytes(a["B"], a["H"], a["Sq"], a["D"])

    def call(ws, nbytes, **kw):
        b = dict(a, **kw)
        return lib.fa_bwd_ws(P[0], P[1], P[2], P[3], P[4], A + 0x5000, A + 0x6000, A + 0x7000, A + 0x8000, b["B"],
                             b["H"], b["Sq"], b["Sk"], b["D"], b["causal"], b["scale"], None, ws, nbytes)

    assert call(None, need) == _capi.FA_ERR_INVALID_ARG          # no workspace
    assert call(A + 0x9008, need) == _capi.FA_ERR_INVALID_ARG    # misaligned workspace
    assert call(A + 0x9000, need - 1) == _capi.FA_ERR_INVALID_ARG  # one byte short
    assert "workspace" in _capi.last_error()
    assert call(A + 0x9000, need, D=512) == _capi.FA_ERR_UNSUPPORTED
    assert call(A + 0x9000, need, scale=0.0) == _capi.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("D", [512, 1024])
def test_large_heads_only_through_fa_fwd(lib, D):
    # Split-D serves fa_fwd; decoding, paged decoding, packed prefill and the
    # backward refuse head dims above 256 before any HIP call
    assert dec(lib, D=D) == _capi.FA_ERR_UNSUPPORTED
    assert paged(lib, D=D) == _capi.FA_ERR_UNSUPPORTED
    assert varlen(lib, D=D) == _capi.FA_ERR_UNSUPPORTED
    a = dict(GOOD, D=D)
    assert lib.fa_bwd(P[0], P[1], P[2], P[3], P[4], A + 0x5000, A + 0x6000, A + 0x7000, A + 0x8000, a["B"], a["H"],
                      a["Sq"], a["Sk"], D, a["causal"], a["scale"], None) == _capi.FA_ERR_UNSUPPORTED


def test_decode_noalloc_rejects_partials_beyond_its_scratch(lib):
    # 64 * 64 * 4 * 257 * 4 bytes of partials > the 16 MiB static scratch:
    # refused before any HIP call (fake pointers, explicit split count)
    a = dict(GOOD, Sq=1)
    st = lib.fa_decode_splitkv_noalloc(P[0], P[1], P[2], P[3], P[4], 64, 64, 1, 4096, 256, 0, a["scale"], None, 4)
    assert st == _capi.FA_ERR_INVALID_ARG
    assert "scratch" in _capi.last_error()
    # the usual argument checks come first
    assert lib.fa_decode_splitkv_noalloc(P[0], P[1], P[2], P[3], P[4], 2, 3, 2, 7, 64, 0, 0.125, None, 2) == \
        _capi.FA_ERR_INVALID_ARG
    assert lib.fa_decode_splitkv_noalloc(P[0], P[1], P[2], P[3], P[4], 2, 3, 1, 7, 96, 0, 0.125, None, 2) == \
        _capi.FA_ERR_UNSUPPORTED
