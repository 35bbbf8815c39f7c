"""Decode steps captured as one HIP graph (append, full layer, selection and
the sparse layers). Every replay must reproduce the eager calls bit for bit,
with eager work and synchronisations between replays, including the replays
right after a re-capture for a larger length bucket; and every replay's
outputs (o, lse, idx, the sparse layers' o) must match the oracle's decode
step under the acceptance rules, for the default path and every option."""
import numpy as np
import pytest
import torch

import oracle as orc
import token_level_sparse_hs_amd as hs
from token_level_sparse_hs_amd import synth
from parity import OutStats, check_block_row, check_idx_row, check_union_row, f32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def fp8_exponents(K, V):
    """Per-KV-head exponents of the oracle's FP8 quantiser for host caches
    [Hkv][n][d] (K and V separately)."""
    return [(orc.fp8_scale_exponent(np.abs(K[g]).max()), orc.fp8_scale_exponent(np.abs(V[g]).max()))
            for g in range(K.shape[0])]


def dequantised(X, exps, which):
    """The oracle's dequantised FP8 values of a host cache [Hkv][n][d]."""
    out = np.empty_like(X)
    for g in range(X.shape[0]):
        out[g] = orc.quantize_fp8(X[g], exps[g][which])[1]
    return out


@pytest.mark.parametrize("option", ["default", "prob_score", "fp8_cache", "fp8_full_layer", "block_select",
                                    "head_union"])
def test_decode_graph_matches_eager_and_oracle(option):
    lengths = [4093, 700, 64, 2500, 1, 3000]  # the longest crosses 4096 -> a second bucket
    B, Hq, Hkv, k, W, nsl, steps = len(lengths), 32, 4, 256, 64, 2, 6
    print(f"[case] decode graph B={B} steps={steps} option={option}", flush=True)
    cap = max(lengths) + steps
    kv_a = torch.zeros((B, Hkv, cap, 2, 128), dtype=torch.bfloat16, device=DEV)
    for b, L in enumerate(lengths):
        kv_a[b, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), 700 + b, DEV)
    kv_b = kv_a.clone()
    host = [(kv_a[b, :, :, 0].double().cpu().numpy(), kv_a[b, :, :, 1].double().cpu().numpy()) for b in range(B)]
    flags = {"prob_score": hs.HS_FLAG_PROB_SCORE, "block_select": hs.HS_FLAG_BLOCK_SELECT,
             "head_union": hs.HS_FLAG_HEAD_UNION}.get(option, 0)
    fp8_full = option == "fp8_full_layer"
    f8_a = hs.kv_to_fp8(kv_a, n_kv=cap) if option in ("fp8_cache", "fp8_full_layer") else None
    f8_b = f8_a.clone() if f8_a is not None else None
    exps = [fp8_exponents(*host[b]) for b in range(B)] if f8_a is not None else None
    if fp8_full:  # the whole step reads the copy: the oracle runs on its dequantised cache
        host = [(dequantised(K, e, 0), dequantised(V, e, 1)) for (K, V), e in zip(host, exps)]
    g = hs.DecodeStepGraph(kv_b, batch=B, q_heads=Hq, sparse_layers=nsl, top_k=k, window=W, flags=flags,
                           kv_fp8=f8_b, fp8_full_layer=fp8_full)
    scale = orc.default_scale(128)
    score = "prob" if option == "prob_score" else "logit"
    full, sparse = OutStats(), OutStats()
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
        o, lse, idx = hs.decode_step(q, kv_new, kv_a, seq, g.bound, top_k=k, window=W, flags=flags,
                                     kv_fp8=f8_a if fp8_full else None)
        if f8_a is not None and not fp8_full:
            hs.kv_to_fp8(kv_a, seq_lens=seq, out=f8_a)
        osp = [hs.sparse_attn_reuse(x, kv_a, idx, top_k=k, window=W, seq_lens=seq, kv_fp8=f8_a, flags=flags)
               for x in qs]
        torch.cuda.synchronize()
        assert torch.equal(idx_g, idx), s
        assert torch.equal(o_g, o), s
        assert torch.equal(lse_g, lse), s
        for a, b in zip(osp_g, osp):
            assert torch.equal(a, b), s
        # the replay against the oracle's decode step of every sequence
        idx_np, o_np, lse_np = idx_g.cpu().numpy(), f32(o_g), lse_g.cpu().numpy()
        for b in range(B):
            K, V = host[b]
            new_row = f32(kv_new[b]).astype(np.float64)
            if fp8_full:
                new_row = np.stack([dequantised(new_row[:, h2][:, None], exps[b], h2)[:, 0] for h2 in range(2)], 1)
            ref = orc.decode_step(f32(q[b]), [], new_row, K, V, cur[b], k, W, scale, score=score,
                                  blocks=option == "block_select", union=option == "head_union")
            full.add(o_np[b], ref["o_full"])
            assert np.abs(lse_np[b] - ref["lse_full"]).max() <= 1e-3, (s, b)
            p = cur[b] - 1
            for gg in range(Hkv):
                where = f"step{s} b{b} g{gg}"
                if option == "head_union":
                    check_union_row(idx_np[b, gg], ref["idx"][gg], ref["heads"][gg], p, W, k, where)
                elif option == "block_select":
                    check_block_row(idx_np[b, gg], ref["idx"][gg], ref["sigma"][gg], ref["tau"][gg], p, W, k, where)
                else:
                    check_idx_row(idx_np[b, gg], ref["idx"][gg], ref["sigma"][gg], ref["tau"][gg], p, W, k, where)
            if exps is not None and not fp8_full:  # the sparse layers read the oracle's dequantised copy
                Ks, Vs = dequantised(K[:, :cur[b]], exps[b], 0), dequantised(V[:, :cur[b]], exps[b], 1)
            else:
                Ks, Vs = K, V
            for x, osx in zip(qs, osp_g):
                r, _ = orc.sparse_attention_rows(f32(x[b])[None], Ks, Vs, idx_np[b][None], np.array([p]), W, scale)
                sparse.add(f32(osx[b]), r[0])
        print(f"[case] step {s} bound {g.bound} captures {g.captures}: identical to eager, oracle ok", flush=True)
    full.check("graph decode full o")
    sparse.check("graph decode sparse o")
    assert torch.equal(kv_a, kv_b)
    if f8_a is not None:
        assert torch.equal(f8_a, f8_b)
    assert g.captures == 2


def test_decode_graph_bucketed_bound_matches_oracle():
    """The eager step with the graph's bucketed bound (max_seq_len rounded up
    to its bucket, so more splits than rows need and score rows longer than
    any sequence) against the oracle."""
    lengths = [3000, 70000, 5, 40000]
    B, Hq, Hkv, k, W = len(lengths), 32, 4, 512, 128
    bound = hs.length_bucket(max(lengths) + 1)
    assert bound > max(lengths) + 1
    print(f"[case] bucketed bound {bound} lengths {lengths}", flush=True)
    kv = torch.zeros((B, Hkv, bound, 2, 128), dtype=torch.bfloat16, device=DEV)
    for b, L in enumerate(lengths):
        kv[b, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), 760 + b, DEV)
    q = synth.randn_bf16((B, Hq, 128), 770, DEV)
    kv_new = synth.randn_bf16((B, Hkv, 2, 128), 771, DEV)
    qs = synth.randn_bf16((B, Hq, 128), 772, DEV)
    cur = [L + 1 for L in lengths]
    seq = torch.tensor(cur, dtype=torch.int32, device=DEV)
    host = [(kv[b, :, :, 0].double().cpu().numpy(), kv[b, :, :, 1].double().cpu().numpy()) for b in range(B)]
    o, lse, idx = hs.decode_step(q, kv_new, kv, seq, bound, top_k=k, window=W)
    osp = hs.sparse_attn_reuse(qs, kv, idx, top_k=k, window=W, seq_lens=seq)
    torch.cuda.synchronize()
    scale = orc.default_scale(128)
    full, sparse = OutStats(), OutStats()
    idx_np = idx.cpu().numpy()
    for b in range(B):
        K, V = host[b]
        ref = orc.decode_step(f32(q[b]), [], f32(kv_new[b]), K, V, cur[b], k, W, scale)
        full.add(f32(o[b]), ref["o_full"])
        for gg in range(Hkv):
            check_idx_row(idx_np[b, gg], ref["idx"][gg], ref["sigma"][gg], ref["tau"][gg], cur[b] - 1, W, k)
        r, _ = orc.sparse_attention_rows(f32(qs[b])[None], K, V, idx_np[b][None], np.array([cur[b] - 1]), W, scale)
        sparse.add(f32(osp[b]), r[0])
    full.check("bucketed full o")
    sparse.check("bucketed sparse o")
