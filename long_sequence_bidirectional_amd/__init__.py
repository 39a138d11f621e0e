"""MI355X-native per-rank attention for context-parallel diffusion transformers.

Python binding of libcpattn (include/cpattn.h).  Every function only checks
and marshals torch tensors (device pointers, sizes, the current HIP stream)
and calls the C ABI; all computation runs in the library's HIP kernels.
torch provides device memory and streams.

  attn_fwd(q, k, v, o=None, lse=None, scale=None)        -> (o, lse)
  attn_fwd_ex(q, k, v, o, lse, workspace=..., accumulate=False) -> (o, lse)
  attn_fwd_ex_static(q, k, v, o, lse, scratch_bytes=None, ...) -> (o, lse)
  attn_fwd_workspace_size(B, H, Sq, Skv, D, ...)          -> bytes
  attn_fwd_split_plan(B, H, Sq, Skv, D, slots, ws_bytes)  -> (split_tiles, pieces, bytes)
  attn_merge(o_a, lse_a, o_b, lse_b, o_out=None, lse_out=None) -> (o_out, lse_out)
  ring_attn_fwd(q, k_chunks, v_chunks, ...)               -> (o, lse)
  attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, ...) -> (o, lse)
  qk_rmsnorm(x, w, eps=1e-6, post_scale=1.0, out=None)   -> out
  ulysses_pack(src, P, direction, dst=None)               -> dst
  ulysses_unpack(src, P, direction, dst=None)             -> dst
  ulysses_pack_n / ulysses_unpack_n(srcs, P, direction, dsts=None) -> dsts (one launch)
"""
from __future__ import annotations

import ctypes
import math

from ._lib import (BF16, E4M3, F16, F32, FLAG_ACCUMULATE, FLAG_K_SEQ_LAST, FLAG_SEQ_MAJOR, HEAD_TO_SEQ, SEQ_TO_HEAD,
                   STATIC_SCRATCH_BYTES,
                   CpattnError, check, lib)

__all__ = ["attn_fwd", "attn_fwd_ex", "attn_fwd_ex_static", "attn_fwd_workspace_size", "attn_fwd_split_plan", "attn_merge",
           "qk_rmsnorm", "attn_fwd_fp8", "ring_attn_fwd", "ulysses_pack", "ulysses_unpack",
           "ulysses_pack_n", "ulysses_unpack_n", "MAX_RELAYOUT_TENSORS",
           "SEQ_TO_HEAD", "HEAD_TO_SEQ", "CpattnError", "lib"]


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16, float16 or float32)")


def _dev(t, name, device=None):
    """Device pointer of a contiguous device tensor (on `device` when given).  The C ABI cannot
    tell a host or strided buffer from a device one, so every pointer passes through here."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _launch(fn, device, *args, stream=None):
    """Call C entry point `fn` with `args` and the stream, with the tensors' device current (the
    library's per-device lookups use the current device).  The stream defaults to that device's
    current stream; a stream given must belong to that device."""
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    if s.device != device:
        raise ValueError(f"stream is on {s.device}, the tensors on {device}")
    with torch.cuda.device(device):
        st = getattr(lib(), fn)(*args, s.cuda_stream)
    check(fn, st)


def _attn_operands(q, k, v, o, lse, scale, out_dtype, seq_major=False, k_seq_last=False):
    """Shapes, defaults and the C argument tuple of an attention call.  Head-major tensors are
    [B, H, S, D]; sequence-major ones [B, S, H, D]; with k_seq_last k is [B, H, D, Skv]; lse is
    [B, H, Sq] in every layout."""
    torch = _torch()
    if seq_major and k_seq_last:
        raise ValueError("k_seq_last takes head-major q, v and o")
    if seq_major:
        B, Sq, H, D = q.shape
        Skv = k.shape[1]
        kv_shape, o_shape = (B, Skv, H, D), (B, Sq, H, D)
    else:
        B, H, Sq, D = q.shape
        Skv = v.shape[2]
        kv_shape, o_shape = (B, H, Skv, D), (B, H, Sq, D)
    k_shape = (B, H, D, Skv) if k_seq_last else kv_shape
    if tuple(k.shape) != k_shape or tuple(v.shape) != kv_shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if o is None:
        o = torch.empty(o_shape, dtype=out_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if tuple(o.shape) != o_shape or lse.shape != (B, H, Sq) or lse.dtype != torch.float32:
        raise ValueError(f"o must be {o_shape} and lse float32 [B,H,Sq]")
    dv = q.device
    args = (_dev(q, "q"), _dev(k, "k", dv) if Skv else None, _dev(v, "v", dv) if Skv else None,
            _dev(o, "o", dv), _dev(lse, "lse", dv), B, H, Sq, Skv, D, float(scale), _dtype_code(q), _dtype_code(o))
    return o, lse, args, dv


def attn_fwd(q, k, v, o=None, lse=None, scale=None, out_dtype=None, stream=None):
    """Non-causal attention with per-row LSE.  q [B,H,Sq,D], k/v [B,H,Skv,D]."""
    o, lse, args, dv = _attn_operands(q, k, v, o, lse, scale, out_dtype)
    _launch("cpattn_attn_fwd", dv, *args, stream=stream)
    return o, lse


def attn_fwd_ex(q, k, v, o=None, lse=None, scale=None, out_dtype=None, workspace=None, accumulate=False,
                seq_major=False, stream=None, k_seq_last=False):
    """attn_fwd with a workspace (uint8 device tensor, key-range split of the last wave), an
    accumulate mode that folds the result into the f32 (o, lse) already there, a
    sequence-major layout (q [B,Sq,H,D], k/v [B,Skv,H,D], o [B,Sq,H,D]) and a sequence-last K
    (k_seq_last: k [B,H,D,Skv] with head-major q, v, o; Skv a multiple of 8)."""
    if accumulate and (o is None or lse is None):
        raise ValueError("accumulate needs the existing o and lse")
    o, lse, args, dv = _attn_operands(q, k, v, o, lse, scale, out_dtype, seq_major, k_seq_last)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None and workspace.numel() > 0:
        ws_ptr, ws_bytes = _dev(workspace, "workspace", dv), workspace.numel() * workspace.element_size()
    flags = ((FLAG_ACCUMULATE if accumulate else 0) | (FLAG_SEQ_MAJOR if seq_major else 0)
             | (FLAG_K_SEQ_LAST if k_seq_last else 0))
    _launch("cpattn_attn_fwd_ex", dv, *args, flags, ws_ptr, ws_bytes, stream=stream)
    return o, lse


def attn_fwd_ex_static(q, k, v, o=None, lse=None, scale=None, out_dtype=None, scratch_bytes=None, accumulate=False,
                       seq_major=False, stream=None):
    """attn_fwd_ex with the split workspace taken from the library's static per-device scratch
    (the library allocates nothing; pass o and lse to allocate nothing here either).
    scratch_bytes: how much of the scratch the split may use (default: the best plan's size,
    at most STATIC_SCRATCH_BYTES)."""
    if accumulate and (o is None or lse is None):
        raise ValueError("accumulate needs the existing o and lse")
    o, lse, args, dv = _attn_operands(q, k, v, o, lse, scale, out_dtype, seq_major)
    if scratch_bytes is None:
        B, H, Sq, Skv, D = args[5], args[6], args[7], args[8], args[9]
        with _torch().cuda.device(dv):
            scratch_bytes = min(attn_fwd_workspace_size(B, H, Sq, Skv, D, args[11], args[12]),
                                STATIC_SCRATCH_BYTES)
    flags = (FLAG_ACCUMULATE if accumulate else 0) | (FLAG_SEQ_MAJOR if seq_major else 0)
    _launch("cpattn_attn_fwd_ex_static", dv, *args, flags, int(scratch_bytes), stream=stream)
    return o, lse


def attn_fwd_fp8(q, k, v, q_scale=1.0, k_scale=1.0, v_scale=1.0, o=None, lse=None, scale=None,
                 out_dtype=None, seq_major=False, workspace=None, accumulate=False, stream=None):
    """Attention of E4M3 inputs (uint8 codes or torch.float8_e4m3fn) with per-tensor scales;
    O in bf16 (default) or f32.  Shapes as attn_fwd_ex (head- or sequence-major), D = 128;
    workspace (uint8 device tensor, size from attn_fwd_workspace_size(..., in_dtype=E4M3)) and
    accumulate (f32 O) as for attn_fwd_ex."""
    torch = _torch()
    for t in (q, k, v):
        if t.dtype not in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)):
            raise TypeError("fp8 attention takes E4M3 codes (uint8 or float8_e4m3fn)")
    if seq_major:
        B, Sq, H, D = q.shape
        Skv = k.shape[1]
        kv_shape, o_shape = (B, Skv, H, D), (B, Sq, H, D)
    else:
        B, H, Sq, D = q.shape
        Skv = k.shape[2]
        kv_shape, o_shape = (B, H, Skv, D), (B, H, Sq, D)
    if tuple(k.shape) != kv_shape or tuple(v.shape) != kv_shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if accumulate and (o is None or lse is None):
        raise ValueError("accumulate needs the existing o and lse")
    if o is None:
        o = torch.empty(o_shape, dtype=out_dtype or torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if tuple(o.shape) != o_shape or lse.shape != (B, H, Sq) or lse.dtype != torch.float32:
        raise ValueError(f"o must be {o_shape} and lse float32 [B,H,Sq]")
    flags = (FLAG_SEQ_MAJOR if seq_major else 0) | (FLAG_ACCUMULATE if accumulate else 0)
    dv = q.device
    ws_ptr, ws_bytes = None, 0
    if workspace is not None and workspace.numel() > 0:
        ws_ptr, ws_bytes = _dev(workspace, "workspace", dv), workspace.numel() * workspace.element_size()
    _launch("cpattn_attn_fwd_fp8", dv, _dev(q, "q"), _dev(k, "k", dv) if Skv else None,
            _dev(v, "v", dv) if Skv else None, _dev(o, "o", dv), _dev(lse, "lse", dv),
            B, H, Sq, Skv, D, float(scale), float(q_scale), float(k_scale), float(v_scale), _dtype_code(o), flags,
            ws_ptr, ws_bytes, stream=stream)
    return o, lse


def attn_fwd_workspace_size(B, H, Sq, Skv, D, in_dtype=BF16, o_dtype=BF16):
    """Workspace bytes attn_fwd_ex uses for this problem on the current device."""
    n = ctypes.c_uint64(0)
    check("cpattn_attn_fwd_workspace_size",
          lib().cpattn_attn_fwd_workspace_size(B, H, Sq, Skv, D, in_dtype, o_dtype, ctypes.byref(n)))
    return n.value


def attn_fwd_split_plan(B, H, Sq, Skv, D, slots, workspace_bytes=2**64 - 1):
    """(split_tiles, pieces, bytes_used) of attn_fwd_ex on a device holding `slots` workgroups."""
    t, p, b = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_uint64(0)
    check("cpattn_attn_fwd_split_plan",
          lib().cpattn_attn_fwd_split_plan(B, H, Sq, Skv, D, slots, workspace_bytes, ctypes.byref(t),
                                           ctypes.byref(p), ctypes.byref(b)))
    return t.value, p.value, b.value


def attn_merge(o_a, lse_a, o_b, lse_b, o_out=None, lse_out=None, stream=None):
    """Merge two partial results over disjoint key sets; o_out may be o_a (in place)."""
    torch = _torch()
    B, H, S, D = o_a.shape
    if o_b.shape != o_a.shape or lse_a.shape != (B, H, S) or lse_b.shape != (B, H, S):
        raise ValueError("merge operands must share shapes")
    if o_b.dtype != o_a.dtype:
        raise TypeError("o_a and o_b must share a dtype")
    if o_out is None:
        o_out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    if o_out.dtype != o_a.dtype or o_out.shape != o_a.shape or lse_out.shape != lse_a.shape:
        raise ValueError("outputs must match the operands")
    for t in (lse_a, lse_b, lse_out):
        if t.dtype != torch.float32:
            raise TypeError("lse tensors must be float32")
    dv = o_a.device
    _launch("cpattn_attn_merge", dv, _dev(o_a, "o_a"), _dev(lse_a, "lse_a", dv), _dev(o_b, "o_b", dv),
            _dev(lse_b, "lse_b", dv), _dev(o_out, "o_out", dv), _dev(lse_out, "lse_out", dv), B, H, S, D,
            _dtype_code(o_a), stream=stream)
    return o_out, lse_out


def ring_attn_fwd(q, k_chunks, v_chunks, o=None, lse=None, o_work=None, lse_work=None, scale=None,
                  stream=None, use_work=True):
    """Ring attention over K/V chunks [n, B, H, Skv_chunk, D] (bf16); f32 O and LSE out."""
    torch = _torch()
    B, H, Sq, D = q.shape
    n, B2, H2, Skv_c, D2 = k_chunks.shape
    if (B2, H2, D2) != (B, H, D) or v_chunks.shape != k_chunks.shape:
        raise ValueError("chunk shapes must be [n, B, H, Skv_chunk, D]")
    if q.dtype != torch.bfloat16 or k_chunks.dtype != torch.bfloat16 or v_chunks.dtype != torch.bfloat16:
        raise TypeError("ring_attn_fwd takes bfloat16 q and chunks")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dev = q.device
    o = o if o is not None else torch.empty((B, H, Sq, D), dtype=torch.float32, device=dev)
    lse = lse if lse is not None else torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    if (o_work is None) != (lse_work is None):
        raise ValueError("give both o_work and lse_work, or neither")
    if o_work is None and use_work:   # scratch for the key-range split of partial waves
        o_work, lse_work = torch.empty_like(o), torch.empty_like(lse)
    _launch("cpattn_ring_attn_fwd", dev, _dev(q, "q"), _dev(k_chunks, "k_chunks", dev) if Skv_c else None,
            _dev(v_chunks, "v_chunks", dev) if Skv_c else None, _dev(o, "o", dev), _dev(lse, "lse", dev),
            _dev(o_work, "o_work", dev) if o_work is not None else None,
            _dev(lse_work, "lse_work", dev) if lse_work is not None else None,
            B, H, Sq, Skv_c, n, D, float(scale), stream=stream)
    return o, lse


def qk_rmsnorm(x, w, eps=1e-6, post_scale=1.0, out=None, stream=None):
    """RMSNorm over the last dim of x (bf16 or fp16) times w, rounded to x's type, then times the
    16-bit constant post_scale and rounded again; out may be x (in place)."""
    D = x.shape[-1]
    if w.shape != (D,) or w.dtype != x.dtype:
        raise ValueError(f"w must be [{D}] of {x.dtype}")
    if out is None:
        out = _torch().empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x")
    rows = x.numel() // D
    dv = x.device
    _launch("cpattn_qk_rmsnorm", dv, _dev(x, "x"), _dev(w, "w", dv), _dev(out, "out", dv), rows, D, float(eps),
            float(post_scale), _dtype_code(x), stream=stream)
    return out


def _relayout_shapes(src, P, direction, pack):
    """((B, S_local, H, D), dst shape) of a relayout; refuses shapes the index maps do not cover
    (the C ABI sees only S_local and H, so a full sequence that P does not divide must be caught
    here)."""
    if P < 1:
        raise ValueError(f"P must be >= 1, got {P}")
    if pack and direction == SEQ_TO_HEAD:
        B, S_l, H, D = src.shape
        if H % P:
            raise ValueError(f"heads ({H}) must be divisible by P ({P})")
        return (B, S_l, H, D), (B, P, S_l, H // P, D)
    if pack and direction == HEAD_TO_SEQ:
        B, Hp, S, D = src.shape
        if S % P:
            raise ValueError(f"sequence length ({S}) must be divisible by P ({P})")
        return (B, S // P, Hp * P, D), (B, P, S // P, Hp, D)
    B, P2, S_l, Hp, D = src.shape
    if P2 != P:
        raise ValueError("src chunk dim must equal P")
    if direction == SEQ_TO_HEAD:
        return (B, S_l, Hp * P, D), (B, Hp, P * S_l, D)
    return (B, S_l, Hp * P, D), (B, S_l, Hp * P, D)


def _relayout(fn, src, P, direction, dst, pack, stream):
    torch = _torch()
    (B, S_l, H, D), out_shape = _relayout_shapes(src, P, direction, pack)
    if dst is None:
        dst = torch.empty(out_shape, dtype=src.dtype, device=src.device)
    if tuple(dst.shape) != tuple(out_shape) or dst.dtype != src.dtype:
        raise ValueError(f"dst must be {out_shape} of {src.dtype}")
    dv = src.device
    _launch(fn, dv, _dev(src, "src"), _dev(dst, "dst", dv), B, S_l, H, D, P, _dtype_code(src), direction,
            stream=stream)
    return dst


def ulysses_pack(src, P, direction, dst=None, stream=None):
    """seq->head: [B,S_l,H,D] -> [B,P,S_l,H/P,D]; head->seq: [B,Hp,S,D] -> [B,P,S/P,Hp,D]."""
    return _relayout("cpattn_ulysses_pack", src, P, direction, dst, True, stream)


def ulysses_unpack(src, P, direction, dst=None, stream=None):
    """seq->head: [B,P,S_l,Hp,D] -> [B,Hp,P*S_l,D]; head->seq: [B,P,S_l,Hp,D] -> [B,S_l,P*Hp,D]."""
    return _relayout("cpattn_ulysses_unpack", src, P, direction, dst, False, stream)


MAX_RELAYOUT_TENSORS = 8     # CPATTN_MAX_RELAYOUT_TENSORS


def _relayout_n(fn, srcs, P, direction, dsts, pack, stream):
    torch = _torch()
    srcs = list(srcs)
    if not 1 <= len(srcs) <= MAX_RELAYOUT_TENSORS:
        raise ValueError(f"1 to {MAX_RELAYOUT_TENSORS} tensors, got {len(srcs)}")
    (B, S_l, H, D), out_shape = _relayout_shapes(srcs[0], P, direction, pack)
    for t in srcs[1:]:
        if tuple(t.shape) != tuple(srcs[0].shape) or t.dtype != srcs[0].dtype:
            raise ValueError("every source must have the first one's shape and dtype")
    if dsts is None:
        dsts = [torch.empty(out_shape, dtype=srcs[0].dtype, device=srcs[0].device) for _ in srcs]
    dsts = list(dsts)
    if len(dsts) != len(srcs):
        raise ValueError("one destination per source")
    for t in dsts:
        if tuple(t.shape) != tuple(out_shape) or t.dtype != srcs[0].dtype:
            raise ValueError(f"every dst must be {out_shape} of {srcs[0].dtype}")
    n = len(srcs)
    dv = srcs[0].device
    src_ptrs = (ctypes.c_void_p * n)(*(_dev(t, f"srcs[{i}]", dv) for i, t in enumerate(srcs)))
    dst_ptrs = (ctypes.c_void_p * n)(*(_dev(t, f"dsts[{i}]", dv) for i, t in enumerate(dsts)))
    _launch(fn, dv, src_ptrs, dst_ptrs, n, B, S_l, H, D, P, _dtype_code(srcs[0]), direction, stream=stream)
    return dsts


def ulysses_pack_n(srcs, P, direction, dsts=None, stream=None):
    """ulysses_pack of up to 8 same-shaped tensors (e.g. Q, K, V) in one launch; returns the list
    of destinations."""
    return _relayout_n("cpattn_ulysses_pack_n", srcs, P, direction, dsts, True, stream)


def ulysses_unpack_n(srcs, P, direction, dsts=None, stream=None):
    """ulysses_unpack of up to 8 same-shaped tensors in one launch; returns the destinations."""
    return _relayout_n("cpattn_ulysses_unpack_n", srcs, P, direction, dsts, False, stream)
