"""Seeded synthetic inputs for the five long-context workloads (inputs only).

This module holds no attention or selection arithmetic: it only draws i.i.d.
N(0, 1) values (rounded to bf16), plants "needle" keys and draws decode
context lengths. Tests, the smoke check and the benchmark feed the same
tensors to the HIP library and to the CPU oracle.

Workloads (shapes of the pages' long-context agent scenario: long tool
responses prefilled into a growing cache, then decoding):
  tiny        B=1, N=2048, 4 q heads / 1 KV head, k=256, W=128, 1 sparse layer
  prefill32k  B=1, N=32768, 32/4 heads, k=2048, W=512, 3 sparse layers, 64 needles
  chunk128k   131072 cached + 8192-token chunk, 32/4, k=2048, W=1024, 3 sparse, 64 needles
  decode64    64 sequences, contexts U{65536..262144}, 32/4, k=2048, W=512, 32 steps
  ctx1m       1048576 cached + 16384-token chunk, 32/4, k=4096, W=1024, 3 sparse,
              256 needles, then 16 decode steps

Needles: key row of KV head g at a planted position = 0.8*u + 0.6*eps, with u
the mean query (over a 16-row span of later query rows and the group's heads)
rescaled to norm sqrt(128), eps ~ N(0, I). Seeds: 0x48530000 + 4096*config +
64*tensor + step.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

D = 128
SPAN = 16

T_K, T_V, T_QFULL, T_QS1, T_QS2, T_QS3, T_NEEDLE, T_CTX, T_KVNEW, T_QDEC = 0, 1, 2, 3, 4, 5, 6, 7, 8, 9


@dataclass
class Workload:
    name: str
    cid: int
    B: int
    n_q: int
    n_kv: int
    Hq: int
    Hkv: int
    top_k: int
    window: int
    sparse_layers: int
    needles: int = 0
    needle_mode: str = "uniform"      # uniform | spread
    decode_steps: int = 0
    ctx_lo: int = 0
    ctx_hi: int = 0
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 2048, 2048, 4, 1, 256, 128, 1),
    "prefill32k": Workload("prefill32k", 1, 1, 32768, 32768, 32, 4, 2048, 512, 3, needles=64),
    "chunk128k": Workload("chunk128k", 2, 1, 8192, 131072 + 8192, 32, 4, 2048, 1024, 3, needles=64),
    "decode64": Workload("decode64", 3, 64, 1, 0, 32, 4, 2048, 512, 3, decode_steps=32, ctx_lo=65536,
                         ctx_hi=262144),
    "ctx1m": Workload("ctx1m", 4, 1, 16384, 1048576 + 16384, 32, 4, 4096, 1024, 3, needles=256,
                      needle_mode="spread", decode_steps=16),
}


def seed_for(cid: int, tensor: int, step: int = 0) -> int:
    return 0x48530000 + 4096 * cid + 64 * tensor + step


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn_bf16(shape, seed: int, device, chunk_elems: int = 1 << 28) -> torch.Tensor:
    """i.i.d. N(0,1) float32 values rounded to bf16, drawn in chunks along dim 0."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    g = _gen(seed, device)
    flat = out.view(shape[0], -1) if len(shape) > 1 else out.view(-1, 1)
    per_row = flat.shape[1]
    rows = max(1, chunk_elems // max(1, per_row))
    for r0 in range(0, flat.shape[0], rows):
        r1 = min(flat.shape[0], r0 + rows)
        flat[r0:r1] = torch.randn((r1 - r0, per_row), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    return out


def fill_cache(kv: torch.Tensor, lengths, cid: int) -> None:
    """Fills rows [0, lengths[b]) of kv [B][Hkv][cap][2][D] with seeded N(0,1) bf16
    (K from seed tensor T_K, V from T_V; one generator stream per (b, g))."""
    B, Hkv = kv.shape[0], kv.shape[1]
    for b in range(B):
        L = int(lengths[b])
        for g in range(Hkv):
            step = b * Hkv + g
            kv[b, g, :L, 0] = randn_bf16((L, D), seed_for(cid, T_K) * 1000003 + step, kv.device)
            kv[b, g, :L, 1] = randn_bf16((L, D), seed_for(cid, T_V) * 1000003 + step, kv.device)


def needle_positions(w: Workload, gen_cpu: torch.Generator):
    """Planted positions and the query-row span that each needle serves."""
    off = w.n_kv - w.n_q
    pos, spans = [], []
    if w.needles == 0:
        return pos, spans
    if w.needle_mode == "spread":
        cache_len = w.n_kv - w.n_q
        pos = [int((i + 0.5) * cache_len / w.needles) for i in range(w.needles)]
    elif off > 0:      # chunk: needles in the cache, spans in the chunk
        pos = torch.randperm(off, generator=gen_cpu)[: w.needles].tolist()
    else:              # whole-sequence prefill: needles early enough to have a later span
        hi = w.n_kv - w.window - SPAN
        pos = torch.randperm(hi + 1, generator=gen_cpu)[: w.needles].tolist()
    for p in pos:
        lo_t = max(0, p + w.window - off)          # span rows at positions >= p + W
        hi_t = w.n_q - SPAN
        t0 = lo_t + int(torch.randint(0, max(1, hi_t - lo_t + 1), (1,), generator=gen_cpu))
        spans.append(min(t0, hi_t))
    return pos, spans


def plant_needles(w: Workload, kv: torch.Tensor, q_full: torch.Tensor):
    """Overwrites needle key rows (all KV heads) in kv [1][Hkv][cap][2][D]."""
    gen_cpu = torch.Generator()
    gen_cpu.manual_seed(seed_for(w.cid, T_NEEDLE))
    pos, spans = needle_positions(w, gen_cpu)
    G = w.Hq // w.Hkv
    for i, (p, t0) in enumerate(zip(pos, spans)):
        for g in range(w.Hkv):
            u = q_full[0, t0:t0 + SPAN, g * G:(g + 1) * G].float().mean(dim=(0, 1))
            u = u * (math.sqrt(D) / u.norm().clamp_min(1e-12))
            eps = randn_bf16((D,), seed_for(w.cid, T_NEEDLE) * 1000003 + 1 + i * w.Hkv + g, kv.device).float()
            kv[0, g, p, 0] = (0.8 * u + 0.6 * eps).to(torch.bfloat16)
    return pos, spans


def make_prefill_case(w: Workload, device, kv_capacity=None, sparse_layers=None):
    """Returns dict(kv, q_full, q_sparse list, needles) for a prefill workload."""
    cap = kv_capacity or w.n_kv
    nsl = w.sparse_layers if sparse_layers is None else sparse_layers
    kv = torch.zeros((w.B, w.Hkv, cap, 2, D), dtype=torch.bfloat16, device=device)
    fill_cache(kv, [w.n_kv] * w.B, w.cid)
    q_full = randn_bf16((w.B, w.n_q, w.Hq, D), seed_for(w.cid, T_QFULL), device)
    q_sparse = [randn_bf16((w.B, w.n_q, w.Hq, D), seed_for(w.cid, T_QS1 + i), device) for i in range(nsl)]
    needles = plant_needles(w, kv, q_full) if w.needles else ([], [])
    return {"kv": kv, "q_full": q_full, "q_sparse": q_sparse, "needles": needles}


def decode_lengths(w: Workload, B=None):
    g = torch.Generator()
    g.manual_seed(seed_for(w.cid, T_CTX))
    B = w.B if B is None else B
    return torch.randint(w.ctx_lo, w.ctx_hi + 1, (B,), generator=g).tolist()


def make_decode_case(w: Workload, device, lengths, steps, sparse_layers=None):
    """Cache with `lengths[b]` seeded rows (capacity max(lengths)+steps) and, per
    step, q_full [B][Hq][D], q_sparse list, kv_new [B][Hkv][2][D]."""
    nsl = w.sparse_layers if sparse_layers is None else sparse_layers
    B = len(lengths)
    cap = max(lengths) + steps
    kv = torch.zeros((B, w.Hkv, cap, 2, D), dtype=torch.bfloat16, device=device)
    fill_cache(kv, lengths, w.cid)
    per_step = []
    for s in range(steps):
        per_step.append({
            "q_full": randn_bf16((B, w.Hq, D), seed_for(w.cid, T_QDEC, s), device),
            "q_sparse": [randn_bf16((B, w.Hq, D), seed_for(w.cid, T_QDEC + 1 + i, s), device) for i in range(nsl)],
            "kv_new": randn_bf16((B, w.Hkv, 2, D), seed_for(w.cid, T_KVNEW, s), device),
        })
    return {"kv": kv, "steps": per_step, "cap": cap}
