"""MI355X (gfx950) exact-attention forward: Python binding of libfa_hip.so.

The functions below carry the C-ABI names of include/fa.h and only marshal
arguments: torch tensors supply device memory and the current HIP stream,
the HIP kernels do all of the work.  There is no fallback path: if the
library is missing or the tensors are not on a GPU, the call raises.

    o, lse = fa_fwd(q, k, v, causal=True)                  # q,k,v fp16 [B,H,S,D]
    o, lse = fa_fwd_ws(q, k, v, workspace, causal=True)    # caller-owned workspace
    o, lse = fa_decode_splitkv(q, k, v, num_splits=0)      # Sq == 1, 0 = auto
    o, lse = fa_decode_paged(q, k_cache, v_cache, block_tables, seq_lens)
    o, lse = fa_fwd_varlen(q, k, v, cu_q, cu_k, max_q, max_k)  # packed [total, H, D]
    dq, dk, dv = fa_bwd(q, k, v, o, lse, do, causal=True)
"""
from __future__ import annotations

import math

from . import _capi
from ._capi import FA_ERR_HIP, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_OK, FAError, LIB_PATH

__all__ = [
    "fa_fwd",
    "fa_fwd_ws",
    "fa_fwd_workspace_bytes",
    "fa_fwd_varlen",
    "fa_bwd",
    "fa_bwd_ws",
    "fa_bwd_workspace_bytes",
    "fa_decode_splitkv",
    "fa_decode_splitkv_ws",
    "fa_decode_paged",
    "fa_decode_workspace_bytes",
    "fa_decode_auto_splits",
    "fa_fwd_key_splits",
    "fa_status_string",
    "fa_last_error",
    "FAError",
    "LIB_PATH",
    "FA_OK",
    "FA_ERR_INVALID_ARG",
    "FA_ERR_UNSUPPORTED",
    "FA_ERR_HIP",
]


_TORCH = None
_F16 = None
_F32 = None


def _torch():
    global _TORCH, _F16, _F32
    if _TORCH is None:
        import torch

        _F16, _F32 = torch.float16, torch.float32
        _TORCH = torch
    return _TORCH


def _check_qkv(q, k, v):
    """(B, H, Sq, Sk, D) of fp16, contiguous, 4-d q, k, v on one GPU.  The
    common valid case is settled by one chain of cheap attribute tests; any
    failure re-runs the checks one by one for a precise message."""
    _torch()
    try:
        qs, ks = q.shape, k.shape
        dev = q.get_device()
        if (len(qs) == 4 and len(ks) == 4 and dev >= 0
                and q.dtype is _F16 and k.dtype is _F16 and v.dtype is _F16
                and k.get_device() == dev and v.get_device() == dev
                and q.is_contiguous() and k.is_contiguous() and v.is_contiguous()
                and v.shape == ks and ks[0] == qs[0] and ks[1] == qs[1] and ks[3] == qs[3]):
            return qs[0], qs[1], qs[2], ks[2], qs[3]
    except (AttributeError, TypeError):
        pass
    return _check_qkv_slow(q, k, v)


def _check_qkv_slow(q, k, v):
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.float16:
            raise TypeError(f"{name} must be float16 (got {t.dtype})")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, S, D] tensor")
    if q.device != k.device or q.device != v.device:
        raise ValueError("q, k, v must be on one device")
    B, H, Sq, D = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    return B, H, Sq, k.shape[2], D


def _outputs(q, o, lse):
    torch = _torch()
    qs = q.shape
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((qs[0], qs[1], qs[2]), dtype=_F32, device=q.device)
    try:
        dev = q.get_device()
        ls = lse.shape
        if (o.dtype is _F16 and lse.dtype is _F32 and o.shape == qs and len(ls) == 3
                and ls[0] == qs[0] and ls[1] == qs[1] and ls[2] == qs[2]
                and o.get_device() == dev and lse.get_device() == dev
                and o.is_contiguous() and lse.is_contiguous()):
            return o, lse
    except (AttributeError, TypeError):
        pass
    return _outputs_slow(q, o, lse)


def _outputs_slow(q, o, lse):
    torch = _torch()
    B, H, Sq, D = q.shape
    if not isinstance(o, torch.Tensor) or o.dtype != torch.float16 or tuple(o.shape) != tuple(q.shape) \
            or not o.is_contiguous() or o.device != q.device:
        raise ValueError("o must be a contiguous fp16 tensor shaped like q on its device")
    if not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Sq) \
            or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 [B, H, Sq] tensor on q's device")
    return o, lse


def _stream(q, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(q.get_device())
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def fa_fwd(q, k, v, o=None, lse=None, causal=False, scale=None, stream=None):
    """Exact attention forward; returns (o, lse).  See fa_fwd in include/fa.h."""
    B, H, Sq, Sk, D = _check_qkv(q, k, v)
    o, lse = _outputs(q, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lib = _capi.load()
    st = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    B, H, Sq, Sk, D, int(bool(causal)), float(scale), _stream(q, stream))
    _capi.check(st, "fa_fwd")
    return o, lse


def fa_fwd_ws(q, k, v, workspace, o=None, lse=None, causal=False, scale=None, stream=None):
    """fa_fwd with a caller-owned workspace tensor (any dtype, contiguous, on q's device; None when
    fa_fwd_workspace_bytes is 0).  Nothing is allocated.  See fa_fwd_ws in include/fa.h."""
    B, H, Sq, Sk, D = _check_qkv(q, k, v)
    o, lse = _outputs(q, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    ptr, nbytes = 0, 0
    if workspace is not None:
        if not workspace.is_contiguous() or workspace.get_device() != q.get_device():
            raise ValueError("workspace must be contiguous and on q's device")
        ptr, nbytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    lib = _capi.load()
    st = lib.fa_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       B, H, Sq, Sk, D, int(bool(causal)), float(scale), _stream(q, stream), ptr or None, nbytes)
    _capi.check(st, "fa_fwd_ws")
    return o, lse


def fa_fwd_workspace_bytes(B, H, Sq, Sk, D, causal, num_cus):
    """Workspace bytes fa_fwd / fa_fwd_ws use for these sizes on num_cus CUs (0: none)."""
    return int(_capi.load().fa_fwd_workspace_bytes(B, H, Sq, Sk, D, int(bool(causal)), num_cus))


def fa_bwd(q, k, v, o, lse, do, dq=None, dk=None, dv=None, causal=False, scale=None, stream=None):
    """Gradients (dq, dk, dv) of exact attention from fa_fwd's o and lse.  See fa_bwd in include/fa.h."""
    return _bwd(q, k, v, o, lse, do, dq, dk, dv, causal, scale, stream, None, False)


def fa_bwd_ws(q, k, v, o, lse, do, workspace, dq=None, dk=None, dv=None, causal=False, scale=None, stream=None):
    """fa_bwd with a caller-owned workspace tensor (contiguous, on q's device) of at least
    fa_bwd_workspace_bytes(B, H, Sq, D) bytes.  Nothing is allocated.  See fa_bwd_ws in include/fa.h."""
    return _bwd(q, k, v, o, lse, do, dq, dk, dv, causal, scale, stream, workspace, True)


def fa_bwd_workspace_bytes(B, H, Sq, D):
    """Workspace bytes of fa_bwd / fa_bwd_ws for these sizes (0: invalid sizes)."""
    return int(_capi.load().fa_bwd_workspace_bytes(B, H, Sq, D))


def _bwd(q, k, v, o, lse, do, dq, dk, dv, causal, scale, stream, workspace, with_ws):
    torch = _torch()
    B, H, Sq, Sk, D = _check_qkv(q, k, v)
    for name, t, shape in (("o", o, q.shape), ("do", do, q.shape)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or tuple(t.shape) != tuple(shape) \
                or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous fp16 tensor shaped like q on its device")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Sq) or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 [B, H, Sq] tensor on q's device")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.dtype != torch.float16 or t.shape != ref.shape or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous fp16 tensor shaped like its input")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lib = _capi.load()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Sq, Sk, D, int(bool(causal)), float(scale),
            _stream(q, stream))
    if with_ws:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous() or workspace.device != q.device:
            raise ValueError("workspace must be a contiguous tensor on q's device")
        st = lib.fa_bwd_ws(*args, workspace.data_ptr(), workspace.numel() * workspace.element_size())
        _capi.check(st, "fa_bwd_ws")
    else:
        _capi.check(lib.fa_bwd(*args), "fa_bwd")
    return dq, dk, dv


def fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, o=None, lse=None,
                  causal=False, scale=None, stream=None):
    """Exact attention over a packed variable-length batch; returns (o, lse).

    q fp16 [total_q, H, D]; k, v fp16 [total_k, H, D]; cu_seqlens_q / _k int32
    [B + 1] on q's device; o fp16 like q; lse fp32 [H, total_q].  See
    fa_fwd_varlen in include/fa.h.
    """
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or not t.is_cuda:
            raise TypeError(f"{name} must be a float16 torch.Tensor on a GPU")
        if t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [total, H, D] tensor")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or not t.is_contiguous() or t.dim() != 1:
            raise TypeError(f"{name} must be a contiguous 1-d int32 torch.Tensor")
    for t in (k, v, cu_seqlens_q, cu_seqlens_k):
        if t.device != q.device:
            raise ValueError("all tensors must be on q's device")
    total_q, H, D = q.shape
    total_k = k.shape[0]
    if k.shape[1:] != (H, D) or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    B = cu_seqlens_q.shape[0] - 1
    if B < 1 or cu_seqlens_k.shape[0] != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 >= 2 entries")
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    if o.dtype != torch.float16 or tuple(o.shape) != tuple(q.shape) or not o.is_contiguous() or o.device != q.device:
        raise ValueError("o must be a contiguous fp16 tensor shaped like q on its device")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (H, total_q) or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 [H, total_q] tensor on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lib = _capi.load()
    st = lib.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, H, total_q, total_k,
                           int(max_seqlen_q), int(max_seqlen_k), D, int(bool(causal)), float(scale),
                           _stream(q, stream))
    _capi.check(st, "fa_fwd_varlen")
    return o, lse


def fa_decode_splitkv(q, k, v, o=None, lse=None, causal=False, scale=None, stream=None, num_splits=0):
    """Split-KV single-query decoding; returns (o, lse).

    num_splits <= 0 picks the split count automatically; 1 runs one kernel
    whose 16 wavefronts per (batch, head) split the keys and merge in LDS
    (no workspace); more partitions write partials that a merge kernel
    combines.  See fa_decode_splitkv in include/fa.h.
    """
    B, H, Sq, Sk, D = _check_qkv(q, k, v)
    o, lse = _outputs(q, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lib = _capi.load()
    st = lib.fa_decode_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                               B, H, Sq, Sk, D, int(bool(causal)), float(scale), _stream(q, stream),
                               int(num_splits))
    _capi.check(st, "fa_decode_splitkv")
    return o, lse


def fa_decode_splitkv_ws(q, k, v, workspace, o=None, lse=None, causal=False, scale=None, stream=None,
                         num_splits=0):
    """fa_decode_splitkv with a caller-owned workspace tensor (any dtype, contiguous)."""
    B, H, Sq, Sk, D = _check_qkv(q, k, v)
    o, lse = _outputs(q, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if not workspace.is_contiguous() or workspace.device != q.device:
        raise ValueError("workspace must be contiguous and on q's device")
    nbytes = workspace.numel() * workspace.element_size()
    lib = _capi.load()
    st = lib.fa_decode_splitkv_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  B, H, Sq, Sk, D, int(bool(causal)), float(scale), _stream(q, stream),
                                  int(num_splits), workspace.data_ptr(), nbytes)
    _capi.check(st, "fa_decode_splitkv_ws")
    return o, lse


def fa_decode_paged(q, k_cache, v_cache, block_tables, seq_lens, o=None, lse=None, scale=None, stream=None,
                    num_splits=0):
    """Split-KV decoding over a paged KV cache; returns (o, lse).  See fa_decode_paged in include/fa.h.

    q fp16 [B, H, 1, D]; k_cache / v_cache fp16 [num_blocks, H, block_size, D];
    block_tables int32 [B, max_blocks]; seq_lens int32 [B] (all on q's device).
    """
    torch = _torch()
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or not t.is_cuda:
            raise TypeError(f"{name} must be a float16 torch.Tensor on a GPU")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-d tensor")
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous int32 torch.Tensor")
    for t in (k_cache, v_cache, block_tables, seq_lens):
        if t.device != q.device:
            raise ValueError("all tensors must be on q's device")
    B, H, Sq, D = q.shape
    num_blocks, Hc, block_size, Dc = k_cache.shape
    if Sq != 1 or Hc != H or Dc != D or v_cache.shape != k_cache.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k_cache {tuple(k_cache.shape)} "
                         f"v_cache {tuple(v_cache.shape)}")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_tables must be [B, max_blocks] and seq_lens [B]")
    o, lse = _outputs(q, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lib = _capi.load()
    st = lib.fa_decode_paged(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                             seq_lens.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, D, num_blocks, block_size,
                             block_tables.shape[1], float(scale), _stream(q, stream), int(num_splits))
    _capi.check(st, "fa_decode_paged")
    return o, lse


def fa_decode_workspace_bytes(B, H, D, num_splits):
    return int(_capi.load().fa_decode_workspace_bytes(B, H, D, num_splits))


def fa_decode_auto_splits(B, H, Sk, num_cus):
    return int(_capi.load().fa_decode_auto_splits(B, H, Sk, num_cus))


def fa_fwd_key_splits(B, H, Sq, Sk, D, causal, num_cus):
    """Key-range parts fa_fwd gives the heaviest query tiles (1: no split)."""
    return int(_capi.load().fa_fwd_key_splits(B, H, Sq, Sk, D, int(bool(causal)), num_cus))


def fa_status_string(status):
    return _capi.status_name(status)


def fa_last_error():
    return _capi.last_error()
