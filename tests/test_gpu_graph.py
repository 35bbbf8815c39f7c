"""Decode steps captured as one HIP graph (append, full layer, selection and
the sparse layers) must reproduce the eager calls bit for bit on every replay,
with eager work and synchronisations between replays, including the replays
right after a re-capture for a larger length bucket."""
import pytest
import torch

import token_level_sparse_hs_amd as hs
from token_level_sparse_hs_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("option", ["default", "prob_score", "fp8_cache", "block_select", "head_union"])
def test_decode_graph_matches_eager(option):
    lengths = [4093, 700, 64, 2500, 1, 3000]  # the longest crosses 4096 -> a second bucket
    B, Hq, Hkv, k, W, nsl, steps = len(lengths), 32, 4, 256, 64, 2, 6
    print(f"[case] decode graph B={B} steps={steps} option={option}", flush=True)
    cap = max(lengths) + steps
    kv_a = torch.zeros((B, Hkv, cap, 2, 128), dtype=torch.bfloat16, device=DEV)
    for b, L in enumerate(lengths):
        kv_a[b, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), 700 + b, DEV)
    kv_b = kv_a.clone()
    flags = {"prob_score": hs.HS_FLAG_PROB_SCORE, "block_select": hs.HS_FLAG_BLOCK_SELECT,
             "head_union": hs.HS_FLAG_HEAD_UNION}.get(option, 0)
    f8_a = hs.kv_to_fp8(kv_a, n_kv=cap) if option == "fp8_cache" else None
    f8_b = f8_a.clone() if f8_a is not None else None
    g = hs.DecodeStepGraph(kv_b, batch=B, q_heads=Hq, sparse_layers=nsl, top_k=k, window=W, flags=flags,
                           kv_fp8=f8_b)
    for s in range(steps):
        q = synth.randn_bf16((B, Hq, 128), 710 + s, DEV)
        kv_new = synth.randn_bf16((B, Hkv, 2, 128), 720 + s, DEV)
        qs = [synth.randn_bf16((B, Hq, 128), 730 + 8 * s + i, DEV) for i in range(nsl)]
        cur = [L + s + 1 for L in lengths]
        seq = torch.tensor(cur, dtype=torch.int32, device=DEV)
        g.q.copy_(q)
        g.kv_new.copy_(kv_new)
        for dst, src in zip(g.q_sparse, qs):
            dst.copy_(src)
        g.seq_lens.copy_(seq)
        o_g, lse_g, idx_g, osp_g = g.step(max(cur))
        torch.cuda.synchronize()
        # eager calls with the bound the graph was captured with (same plan)
        o, lse, idx = hs.decode_step(q, kv_new, kv_a, seq, g.bound, top_k=k, window=W, flags=flags)
        if f8_a is not None:
            hs.kv_to_fp8(kv_a, seq_lens=seq, out=f8_a)
        osp = [hs.sparse_attn_reuse(x, kv_a, idx, top_k=k, window=W, seq_lens=seq, kv_fp8=f8_a, flags=flags)
               for x in qs]
        torch.cuda.synchronize()
        assert torch.equal(idx_g, idx), s
        assert torch.equal(o_g, o), s
        assert torch.equal(lse_g, lse), s
        for a, b in zip(osp_g, osp):
            assert torch.equal(a, b), s
        print(f"[case] step {s} bound {g.bound} captures {g.captures}: identical", flush=True)
    assert torch.equal(kv_a, kv_b)
    if f8_a is not None:
        assert torch.equal(f8_a, f8_b)
    assert g.captures == 2
