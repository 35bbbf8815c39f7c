"""token_level_sparse_hs_amd: token-level hybrid sparse attention with KV Reuse on MI355X.

Thin Python front-end over the C ABI of libhysparse (include/hysparse.h):

    full_attn_select   full-attention layer: causal GQA attention plus per-row,
                       per-KV-group top-k token indices (forced window implicit)
    sparse_attn_reuse  sparse layer reusing the full layer's cache and indices
    decode_step        decode full layer: append, attend, select once
    kv_to_fp8          FP8 (e4m3) copy of the cache for the sparse layers

All tensors live on the GPU; the cache layout is [B][Hkv][capacity][2][128]
bf16 (K row then V row per token) unless explicit strides are given.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (HS_FLAG_BLOCK_SELECT, HS_FLAG_EXACT_RESCAN, HS_FLAG_FP8_KV, HS_FLAG_HEAD_UNION,  # noqa: F401
                   HS_FLAG_PROB_SCORE, HsError, HsShape)

__all__ = ["full_attn_select", "sparse_attn_reuse", "decode_step", "make_shape", "HsError",
           "HS_FLAG_EXACT_RESCAN", "HS_FLAG_PROB_SCORE", "HS_FLAG_FP8_KV", "HS_FLAG_BLOCK_SELECT", "HS_FLAG_HEAD_UNION", "kv_to_fp8", "version",
           "select_diagnostics", "kv_bridge", "decode_step_noalloc"]


def version() -> int:
    return _lib.load().hs_version()


def make_shape(*, batch, n_q, n_kv, kv_capacity, q_heads, kv_heads, top_k, window, scale=0.0,
               kv_strides=None, flags=0, head_dim=128) -> HsShape:
    s = HsShape()
    s.batch, s.n_q, s.n_kv, s.kv_capacity = batch, n_q, n_kv, kv_capacity
    s.q_heads, s.kv_heads, s.head_dim = q_heads, kv_heads, head_dim
    s.top_k, s.window, s.scale = top_k, window, scale
    if kv_strides is not None:
        s.kv_stride_b, s.kv_stride_h, s.kv_stride_t, s.kv_v_offset = kv_strides
    s.flags = flags
    s.reserved = 0
    return s


def _check_bf16(name, t, dims):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda:
        raise TypeError(f"{name} must be a bf16 CUDA/HIP tensor")
    if t.dim() != dims or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dims}-d tensor (got shape {tuple(t.shape)})")


def _kv_dims(kv, kv_strides):
    if kv_strides is None:
        _check_bf16("kv", kv, 5)
        if kv.shape[3] != 2 or kv.shape[4] != 128:
            raise ValueError("kv must be [B][Hkv][capacity][2][128]")
        return kv.shape[1], kv.shape[2]
    raise ValueError("explicit kv_strides need kv_heads and kv_capacity arguments")


def _idx_row(flags, top_k, q_heads, kv_heads):
    """Entries per index row: G * top_k under the per-head union."""
    return top_k * (q_heads // kv_heads) if flags & _lib.HS_FLAG_HEAD_UNION else top_k


def full_attn_select(q, kv, n_kv, *, top_k, window, scale=0.0, with_lse=True, flags=0,
                     kv_heads=None, kv_capacity=None, kv_strides=None, workspace=None):
    """Full-attention layer with token selection over a prefill chunk.

    q: bf16 [B][n_q][Hq][128] (the chunk's rows sit at the end of the n_kv-token
    cache). Returns (o bf16 [B][n_q][Hq][128], lse fp32 [B][Hq][n_q] or None,
    idx int32 [B][n_q][Hkv][top_k], or [..][G*top_k] with HS_FLAG_HEAD_UNION).
    """
    _check_bf16("q", q, 4)
    B, n_q, Hq, d = q.shape
    if kv_strides is None:
        kv_heads, kv_capacity = _kv_dims(kv, None)
    shape = make_shape(batch=B, n_q=n_q, n_kv=n_kv, kv_capacity=kv_capacity, q_heads=Hq, kv_heads=kv_heads,
                       top_k=top_k, window=window, scale=scale, kv_strides=kv_strides, flags=flags, head_dim=d)
    dev = q.device
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, n_q), dtype=torch.float32, device=dev) if with_lse else None
    idx = torch.empty((B, n_q, kv_heads, _idx_row(flags, top_k, Hq, kv_heads)), dtype=torch.int32, device=dev)
    nbytes = _lib.workspace_size(_lib.HS_OP_FULL_ATTN_SELECT, shape)
    ws = workspace if workspace is not None else _lib.alloc_workspace(nbytes, dev)
    lib = _lib.load()
    _lib.check(lib.hs_full_attn_select(ctypes.byref(shape), _lib.ptr(q), _lib.ptr(kv), _lib.ptr(o), _lib.ptr(lse),
                                       _lib.ptr(idx) if top_k > 0 else None, _lib.ptr(ws),
                                       0 if ws is None else ws.numel(), _lib.stream_handle(dev)))
    return o, lse, idx


def sparse_attn_reuse(q, kv, idx, *, top_k, window, n_kv=None, seq_lens=None, scale=0.0,
                      kv_heads=None, kv_capacity=None, kv_strides=None, workspace=None, kv_fp8=None, flags=0):
    """Sparse layer reusing the full layer's cache and selection.

    Prefill: q bf16 [B][n_q][Hq][128], idx [B][n_q][Hkv][k], n_kv given.
    Decode:  q bf16 [B][Hq][128], idx [B][Hkv][k], seq_lens int32 [B] on device.
    kv_fp8: the cache's FP8 copy from kv_to_fp8 to gather from instead of kv
    (kv then only gives the shape). flags: HS_FLAG_HEAD_UNION when idx came
    from a full layer with that flag (rows of G*k entries). Returns o with
    q's shape.
    """
    decode = seq_lens is not None
    _check_bf16("q", q, 3 if decode else 4)
    if decode:
        B, Hq, d = q.shape
        n_q = 1
    else:
        B, n_q, Hq, d = q.shape
    if kv_strides is None:
        kv_heads, kv_capacity = _kv_dims(kv, None)
    if idx is not None and (idx.dtype != torch.int32 or not idx.is_contiguous()):
        raise TypeError("idx must be a contiguous int32 tensor")
    if decode and (seq_lens.dtype != torch.int32 or not seq_lens.is_cuda):
        raise TypeError("seq_lens must be an int32 device tensor")
    shape = make_shape(batch=B, n_q=n_q, n_kv=0 if decode else n_kv, kv_capacity=kv_capacity, q_heads=Hq,
                       kv_heads=kv_heads, top_k=top_k, window=window, scale=scale, kv_strides=kv_strides,
                       flags=(flags & _lib.HS_FLAG_HEAD_UNION) | (_lib.HS_FLAG_FP8_KV if kv_fp8 is not None else 0),
                       head_dim=d)
    dev = q.device
    o = torch.empty_like(q)
    nbytes = _lib.workspace_size(_lib.HS_OP_SPARSE_ATTN_REUSE, shape, 1 if decode else 0)
    ws = workspace if workspace is not None else _lib.alloc_workspace(nbytes, dev)
    lib = _lib.load()
    _lib.check(lib.hs_sparse_attn_reuse(ctypes.byref(shape), _lib.ptr(q), _lib.ptr(kv if kv_fp8 is None else kv_fp8),
                                        _lib.ptr(idx) if top_k > 0 else None, _lib.ptr(seq_lens), _lib.ptr(o),
                                        _lib.ptr(ws), 0 if ws is None else ws.numel(), _lib.stream_handle(dev)))
    return o


def decode_step(q, kv_new, kv, seq_lens, max_seq_len, *, top_k, window, scale=0.0, with_lse=True, flags=0,
                kv_heads=None, kv_capacity=None, kv_strides=None, workspace=None, kv_fp8=None):
    """Decode full-attention layer: append kv_new at seq_lens[b]-1, attend, select once.

    q bf16 [B][Hq][128]; kv_new bf16 [B][Hkv][2][128]; seq_lens int32 [B] (device,
    including the new token). Returns (o [B][Hq][128], lse [B][Hq] or None,
    idx int32 [B][Hkv][top_k], or [B][Hkv][G*top_k] with HS_FLAG_HEAD_UNION).
    kv_fp8: the cache's FP8 copy (from kv_to_fp8) to append to and read
    instead of kv, which then only gives the shape and is left unchanged.
    """
    _check_bf16("q", q, 3)
    _check_bf16("kv_new", kv_new, 4)
    B, Hq, d = q.shape
    if kv_strides is None:
        kv_heads, kv_capacity = _kv_dims(kv, None)
    if seq_lens.dtype != torch.int32 or not seq_lens.is_cuda:
        raise TypeError("seq_lens must be an int32 device tensor")
    if kv_fp8 is not None:
        flags |= _lib.HS_FLAG_FP8_KV
    shape = make_shape(batch=B, n_q=1, n_kv=0, kv_capacity=kv_capacity, q_heads=Hq, kv_heads=kv_heads,
                       top_k=top_k, window=window, scale=scale, kv_strides=kv_strides, flags=flags, head_dim=d)
    dev = q.device
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if with_lse else None
    idx = torch.empty((B, kv_heads, _idx_row(flags, top_k, Hq, kv_heads)), dtype=torch.int32, device=dev)
    nbytes = _lib.workspace_size(_lib.HS_OP_DECODE_STEP, shape, max_seq_len)
    ws = workspace if workspace is not None else _lib.alloc_workspace(nbytes, dev)
    lib = _lib.load()
    _lib.check(lib.hs_decode_step(ctypes.byref(shape), _lib.ptr(q), _lib.ptr(kv_new),
                                  _lib.ptr(kv if kv_fp8 is None else kv_fp8),
                                  _lib.ptr(seq_lens), max_seq_len, _lib.ptr(o), _lib.ptr(lse),
                                  _lib.ptr(idx) if top_k > 0 else None, _lib.ptr(ws),
                                  0 if ws is None else ws.numel(), _lib.stream_handle(dev)))
    return o, lse, idx


def decode_step_noalloc(q, kv_new, kv, seq_lens, max_seq_len, *, top_k, window, scale=0.0, with_lse=True, flags=0,
                        kv_fp8=None):
    """decode_step with the library's own static scratch instead of a
    workspace (include/hysparse.h, hs_decode_step_noalloc): no device memory
    is allocated for the step itself (outputs excepted). Steps that need more
    than the 64 MiB scratch raise HsError (HS_ERR_WORKSPACE)."""
    _check_bf16("q", q, 3)
    _check_bf16("kv_new", kv_new, 4)
    B, Hq, d = q.shape
    kv_heads, kv_capacity = _kv_dims(kv, None)
    if seq_lens.dtype != torch.int32 or not seq_lens.is_cuda:
        raise TypeError("seq_lens must be an int32 device tensor")
    if kv_fp8 is not None:
        flags |= _lib.HS_FLAG_FP8_KV
    shape = make_shape(batch=B, n_q=1, n_kv=0, kv_capacity=kv_capacity, q_heads=Hq, kv_heads=kv_heads,
                       top_k=top_k, window=window, scale=scale, flags=flags, head_dim=d)
    dev = q.device
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if with_lse else None
    idx = torch.empty((B, kv_heads, _idx_row(flags, top_k, Hq, kv_heads)), dtype=torch.int32, device=dev)
    _lib.check(_lib.load().hs_decode_step_noalloc(ctypes.byref(shape), _lib.ptr(q), _lib.ptr(kv_new),
                                                  _lib.ptr(kv if kv_fp8 is None else kv_fp8), _lib.ptr(seq_lens),
                                                  max_seq_len, _lib.ptr(o), _lib.ptr(lse),
                                                  _lib.ptr(idx) if top_k > 0 else None, _lib.stream_handle(dev)))
    return o, lse, idx


def kv_bridge(hidden, w_kv, kv, n_kv, *, kv_strides=None, kv_heads=None, kv_capacity=None):
    """KV Bridging: writes cache rows [n_kv - n_q, n_kv) of every (b, KV head)
    of kv from the self-decoder's hidden states (include/hysparse.h,
    hs_kv_bridge): K = hidden W[g][0]^T, V = hidden W[g][1]^T, bf16.

    hidden: bf16 [B][n_q][d_model]; w_kv: bf16 [Hkv][2][128][d_model]; kv: the
    cache [B][Hkv][capacity][2][128] (or kv_new [B][Hkv][2][128] viewed as a
    cache of capacity 1 with n_kv = 1). Returns kv."""
    _check_bf16("hidden", hidden, 3)
    _check_bf16("w_kv", w_kv, 4)
    B, n_q, d_model = hidden.shape
    if kv_strides is None:
        kv_heads, kv_capacity = _kv_dims(kv, None)
    if tuple(w_kv.shape) != (kv_heads, 2, 128, d_model):
        raise ValueError(f"w_kv must be [{kv_heads}][2][128][{d_model}] (got {tuple(w_kv.shape)})")
    shape = make_shape(batch=B, n_q=n_q, n_kv=n_kv, kv_capacity=kv_capacity, q_heads=kv_heads, kv_heads=kv_heads,
                       top_k=0, window=1, kv_strides=kv_strides)
    _lib.check(_lib.load().hs_kv_bridge(ctypes.byref(shape), _lib.ptr(hidden), d_model, _lib.ptr(w_kv), _lib.ptr(kv),
                                        _lib.stream_handle(hidden.device)))
    return kv


def select_diagnostics(q, kv, n_kv, workspace, *, top_k, window, flags=0):
    """Records of the token-level selection that full_attn_select(q, kv, n_kv,
    ..., workspace=workspace) left in `workspace` (include/hysparse.h,
    hs_select_diagnostics): {"deferred_rows": int64 tensor of the rows
    (b*n_q + t)*Hkv + g that took the block-wide path, "rescans": rows whose
    scores were recomputed exactly}. Synchronises the device."""
    B, n_q, Hq, d = q.shape
    kv_heads, kv_capacity = _kv_dims(kv, None)
    shape = make_shape(batch=B, n_q=n_q, n_kv=n_kv, kv_capacity=kv_capacity, q_heads=Hq, kv_heads=kv_heads,
                       top_k=top_k, window=window, flags=flags, head_dim=d)
    a, b, c = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    _lib.check(_lib.load().hs_select_diagnostics(ctypes.byref(shape), ctypes.byref(a), ctypes.byref(b),
                                                 ctypes.byref(c)))
    torch.cuda.synchronize(workspace.device)
    words = workspace[b.value:c.value + 4].view(torch.int32).cpu()
    n = int(words[0])
    rows = workspace[a.value:a.value + 4 * n].view(torch.int32).to(torch.int64).cpu()
    return {"deferred_rows": rows, "rescans": int(words[-1])}


def kv_to_fp8(kv, *, n_kv=None, seq_lens=None, out=None):
    """FP8 (e4m3) copy of the bf16 cache kv [B][Hkv][capacity][2][128] for
    the sparse layers (include/hysparse.h, hs_kv_fp8_convert).

    Prefill form (n_kv given): per-KV-head power-of-two scales from rows
    [0, n_kv), those rows converted into a new (or the given) copy. Decode
    form (seq_lens given, int32 [B] on the device): row seq_lens[b]-1 of
    `out` refreshed with its stored scales. Returns the copy (uint8 tensor).
    """
    B, Hkv, cap = kv.shape[0], kv.shape[1], kv.shape[2]
    _kv_dims(kv, None)
    shape = make_shape(batch=B, n_q=1, n_kv=n_kv or 0, kv_capacity=cap, q_heads=Hkv, kv_heads=Hkv, top_k=0,
                       window=1)
    lib = _lib.load()
    if out is None:
        if seq_lens is not None:
            raise ValueError("the decode form refreshes an existing copy: pass out")
        n = ctypes.c_size_t(0)
        _lib.check(lib.hs_kv_fp8_size(ctypes.byref(shape), ctypes.byref(n)))
        out = torch.empty(n.value, dtype=torch.uint8, device=kv.device)
    _lib.check(lib.hs_kv_fp8_convert(ctypes.byref(shape), _lib.ptr(kv), _lib.ptr(out), _lib.ptr(seq_lens),
                                     _lib.stream_handle(kv.device)))
    return out


from .graph import DecodeStepGraph, length_bucket  # noqa: E402  (uses the calls above)

__all__ += ["DecodeStepGraph", "length_bucket"]
