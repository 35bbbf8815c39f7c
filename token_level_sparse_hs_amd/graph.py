"""One decode step as one HIP graph: append, full layer, selection and the
sparse layers that reuse its selection, replayed with a single launch.

Decode with KV Reuse runs, per generated token, the full layer (which appends
the token's K/V and selects once) and then every sparse layer on that one
selection ("HySparse2 od Xiaomi zkracuje zpracovani dlouheho kontextu",
section "Proc neni nutne znovu zpracovat cely dlouhy vstup"). At a long
context with a small batch the sparse layers read only a few MB each and take
microseconds, so per-launch overhead dominates them ("Simplified Sparse
Attention via Gist Tokens", section 3.6, on launch overhead once kernels
take microseconds). Every call of the library enqueues kernels only (no
allocation, copy, memset or host wait), so a step can be captured once and
replayed.

What the capture fixes: the full layer's split plan and score-row workspace
follow the host bound on the sequence lengths. Lengths themselves are read on
the device, so one graph serves every step whose longest sequence stays within
the bound it was captured with. Bounds are taken in buckets of at most 1/8 of
an octave (at least 4096 tokens), and the step is captured again when a
sequence outgrows its bucket.
"""
from __future__ import annotations

import torch

from . import _lib
from . import decode_step, kv_to_fp8, make_shape, sparse_attn_reuse

__all__ = ["DecodeStepGraph", "length_bucket"]


def length_bucket(max_seq_len: int) -> int:
    """Smallest bucket bound >= max_seq_len: a multiple of 2^max(12, floor(log2 L) - 3)."""
    if max_seq_len < 1:
        raise ValueError("max_seq_len must be >= 1")
    g = 1 << max(12, max_seq_len.bit_length() - 1 - 3)
    return -(-max_seq_len // g) * g


class DecodeStepGraph:
    """Replays append + full layer + selection + `sparse_layers` sparse layers.

    Write the step's inputs into the static tensors `q` [B][Hq][128],
    `kv_new` [B][Hkv][2][128], `q_sparse[i]` [B][Hq][128] and `seq_lens` [B]
    (int32, each sequence's length including the new token), then call
    `step(max_seq_len)`. Outputs land in `o`, `lse`, `idx` and `o_sparse[i]`,
    which the next replay overwrites. `kv` is the caller's cache, written at
    slot seq_lens[b]-1 by every replay.
    """

    def __init__(self, kv, *, batch, q_heads, sparse_layers, top_k, window, scale=0.0, with_lse=True, flags=0,
                 kv_fp8=None, fp8_full_layer=False):
        if not isinstance(kv, torch.Tensor) or kv.dim() != 5:
            raise ValueError("kv must be the [B][Hkv][capacity][2][128] cache tensor")
        self.kv = kv
        dev = kv.device
        B, Hkv, cap = batch, kv.shape[1], kv.shape[2]
        if kv.shape[0] != B:
            raise ValueError("kv batch does not match")
        self.B, self.Hq, self.Hkv, self.cap = B, q_heads, Hkv, cap
        self.top_k, self.window, self.scale, self.with_lse = top_k, window, scale, with_lse
        # options: selection flags of the full layer; an FP8 copy of the cache
        # (from kv_to_fp8) that the step refreshes at the appended row and the
        # sparse layers gather from; with fp8_full_layer the full layer also
        # reads the copy (and appends to it; the bf16 cache is then untouched)
        if fp8_full_layer and kv_fp8 is None:
            raise ValueError("fp8_full_layer needs the FP8 copy kv_fp8")
        self.flags, self.kv_fp8, self.fp8_full_layer = flags, kv_fp8, fp8_full_layer
        self.q = torch.zeros((B, q_heads, 128), dtype=torch.bfloat16, device=dev)
        self.kv_new = torch.zeros((B, Hkv, 2, 128), dtype=torch.bfloat16, device=dev)
        self.q_sparse = [torch.zeros_like(self.q) for _ in range(sparse_layers)]
        self.seq_lens = torch.ones((B,), dtype=torch.int32, device=dev)
        shape = make_shape(batch=B, n_q=1, n_kv=0, kv_capacity=cap, q_heads=q_heads, kv_heads=Hkv,
                           top_k=top_k, window=window, scale=scale,
                           flags=flags | (_lib.HS_FLAG_FP8_KV if fp8_full_layer else 0))
        self.ws_sparse = _lib.alloc_workspace(_lib.workspace_size(_lib.HS_OP_SPARSE_ATTN_REUSE, shape, 1), dev)
        self._shape = shape
        self.graph = None
        self.bound = 0
        self.captures = 0

    def _capture(self, bound: int) -> None:
        dev = self.kv.device
        self.graph = None
        ws_full = _lib.alloc_workspace(_lib.workspace_size(_lib.HS_OP_DECODE_STEP, self._shape, bound), dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            o, lse, idx = decode_step(self.q, self.kv_new, self.kv, self.seq_lens, bound, top_k=self.top_k,
                                      window=self.window, scale=self.scale, with_lse=self.with_lse,
                                      flags=self.flags, workspace=ws_full,
                                      kv_fp8=self.kv_fp8 if self.fp8_full_layer else None)
            if self.kv_fp8 is not None and not self.fp8_full_layer:
                kv_to_fp8(self.kv, seq_lens=self.seq_lens, out=self.kv_fp8)
            o_sp = [sparse_attn_reuse(x, self.kv, idx, top_k=self.top_k, window=self.window, scale=self.scale,
                                      seq_lens=self.seq_lens, workspace=self.ws_sparse, kv_fp8=self.kv_fp8,
                                      flags=self.flags)
                    for x in self.q_sparse]
        self.graph, self.ws_full, self.bound = g, ws_full, bound
        self.o, self.lse, self.idx, self.o_sparse = o, lse, idx, o_sp
        self.captures += 1

    def step(self, max_seq_len: int):
        """Runs one step whose longest sequence (new token included) is max_seq_len."""
        if max_seq_len > self.cap:
            raise ValueError(f"max_seq_len {max_seq_len} exceeds the cache capacity {self.cap}")
        if self.graph is None or max_seq_len > self.bound:
            self._capture(min(length_bucket(max_seq_len), self.cap))
        self.graph.replay()
        return self.o, self.lse, self.idx, self.o_sparse
