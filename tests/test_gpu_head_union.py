"""GPU parity of the union of per-head top-k sets (grouped unfolding for
GQA) with the oracle: each query head keeps its own top k by its scaled
logit, the group's row is the union, G*k entries ascending, -1 padded; the
sparse layers read those rows. Outputs o / lse are the full layer's."""
import numpy as np
import pytest
import torch

import oracle as orc
import token_level_sparse_hs_amd as hs
from token_level_sparse_hs_amd import synth
from parity import OutStats, check_prefill, check_union_row, f32
from test_gpu_fp8 import split_copy

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
UNI = hs.HS_FLAG_HEAD_UNION


def prefill(B, n_q, n_kv, Hq, Hkv, k, W, seed, with_lse=True):
    print(f"[case] union prefill B={B} n_q={n_q} n_kv={n_kv} Hq={Hq} Hkv={Hkv} k={k} W={W}", flush=True)
    kv = torch.zeros((B, Hkv, n_kv + 3, 2, 128), dtype=torch.bfloat16, device=DEV)
    kv[:, :, :n_kv] = synth.randn_bf16((B, Hkv, n_kv, 2, 128), seed, DEV)
    q = synth.randn_bf16((B, n_q, Hq, 128), seed + 1, DEV)
    qs = synth.randn_bf16((B, n_q, Hq, 128), seed + 2, DEV)
    o, lse, idx = hs.full_attn_select(q, kv, n_kv, top_k=k, window=W, flags=UNI, with_lse=with_lse)
    assert idx.shape[-1] == (Hq // Hkv) * k
    osp = hs.sparse_attn_reuse(qs, kv, idx, top_k=k, window=W, n_kv=n_kv, flags=UNI)
    torch.cuda.synchronize()
    return check_prefill(q, kv, n_kv, k, W, o, lse, idx, q_sparse=[qs], o_sparse=[osp], union=True)


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (32, 4), (4, 2), (2, 2)])
def test_union_prefill_small(Hq, Hkv):
    # n_kv - W + 1 > 3k + 256: each one-head pass filters by a sampled threshold
    prefill(1, 260, 700, Hq, Hkv, 64, 24, seed=3100 + Hq)


def test_union_prefill_chunk_batch_no_lse():
    prefill(2, 90, 610, 8, 2, 40, 17, seed=3200, with_lse=False)


def decode(lengths, Hq, Hkv, k, W, seed):
    B = len(lengths)
    print(f"[case] union decode lengths={lengths} Hq={Hq} Hkv={Hkv} k={k}", flush=True)
    cap = max(lengths) + 1
    kv = torch.zeros((B, Hkv, cap, 2, 128), dtype=torch.bfloat16, device=DEV)
    for b, L in enumerate(lengths):
        kv[b, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), seed + b, DEV)
    seq = torch.tensor([L + 1 for L in lengths], dtype=torch.int32, device=DEV)
    q = synth.randn_bf16((B, Hq, 128), seed + 50, DEV)
    qs = synth.randn_bf16((B, Hq, 128), seed + 51, DEV)
    kv_new = synth.randn_bf16((B, Hkv, 2, 128), seed + 52, DEV)
    o, lse, idx = hs.decode_step(q, kv_new, kv, seq, max(lengths) + 1, top_k=k, window=W, flags=UNI)
    osp = hs.sparse_attn_reuse(qs, kv, idx, top_k=k, window=W, seq_lens=seq, flags=UNI)
    torch.cuda.synchronize()
    full, sparse = OutStats(), OutStats()
    idx_np = idx.cpu().numpy()
    for b, L in enumerate(lengths):
        K = kv[b, :, :, 0].float().cpu().numpy()
        V = kv[b, :, :, 1].float().cpu().numpy()
        K[:, L] = 0.0  # the oracle appends kv_new itself
        ref = orc.decode_step(f32(q[b]), [], f32(kv_new[b]), K, V, L + 1, k, W, orc.default_scale(128), union=True)
        full.add(f32(o[b]), ref["o_full"])
        assert np.abs(lse[b].cpu().numpy() - ref["lse_full"]).max() <= 1e-3
        for g in range(Hkv):
            check_union_row(idx_np[b, g], ref["idx"][g], ref["heads"][g], L, W, k, where=f"b{b} g{g}")
        so, _ = orc.sparse_attention_rows(f32(qs[b])[None], K, V, idx_np[b][None], np.array([L]), W,
                                          orc.default_scale(128))
        sparse.add(f32(osp[b]), so[0])
    full.check("decode full o")
    sparse.check("decode sparse o")


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (32, 4), (8, 1)])
def test_union_decode(Hq, Hkv):
    decode([40, 300, 1200, 5000, 20000], Hq, Hkv, 64, 32, seed=3300 + Hq)


def test_union_decode_long_rows_sliced():
    """Eight head rows of 300K candidates: few rows, so the heads' top-k run
    in slices spread over the chip."""
    decode([300_000], 8, 1, 2048, 512, seed=3400)


def test_union_widens_the_selection():
    """The flag is not a no-op: with G = 8 the union holds more tokens than k."""
    n, W, k = 2000, 16, 64
    kv = synth.randn_bf16((1, 2, n, 2, 128), 3500, DEV)
    q = synth.randn_bf16((1, 64, 16, 128), 3501, DEV)
    _, _, iu = hs.full_attn_select(q, kv, n, top_k=k, window=W, flags=UNI)
    torch.cuda.synchronize()
    counts = (iu >= 0).sum(-1).cpu().numpy()
    assert counts.min() > k and counts.max() <= 8 * k


def test_union_prefill_exact_rescan():
    """The one-head passes take the flag through (forced exact rescan)."""
    print("[case] union prefill exact rescan", flush=True)
    n_kv, n_q, Hq, Hkv, k, W = 500, 150, 8, 2, 48, 16
    kv = synth.randn_bf16((1, Hkv, n_kv, 2, 128), 3600, DEV)
    q = synth.randn_bf16((1, n_q, Hq, 128), 3601, DEV)
    o, lse, idx = hs.full_attn_select(q, kv, n_kv, top_k=k, window=W, flags=UNI | hs.HS_FLAG_EXACT_RESCAN)
    torch.cuda.synchronize()
    check_prefill(q, kv, n_kv, k, W, o, lse, idx, union=True)


def test_union_decode_sparse_from_fp8_copy():
    """Sparse decode layers over union rows (8 * k entries) gathering from
    the FP8 copy, against the oracle on the dequantised copy."""
    lengths = [700, 5000]
    B, Hq, Hkv, k, W = len(lengths), 32, 4, 64, 32
    print(f"[case] union decode + fp8 sparse lengths={lengths}", flush=True)
    cap = max(lengths) + 1
    kv = torch.zeros((B, Hkv, cap, 2, 128), dtype=torch.bfloat16, device=DEV)
    for b, L in enumerate(lengths):
        kv[b, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), 3700 + b, DEV)
    seq = torch.tensor([L + 1 for L in lengths], dtype=torch.int32, device=DEV)
    q = synth.randn_bf16((B, Hq, 128), 3710, DEV)
    qs = synth.randn_bf16((B, Hq, 128), 3711, DEV)
    kv_new = synth.randn_bf16((B, Hkv, 2, 128), 3712, DEV)
    _, _, idx = hs.decode_step(q, kv_new, kv, seq, cap, top_k=k, window=W, flags=UNI)
    f8 = hs.kv_to_fp8(kv, n_kv=cap)
    o8 = hs.sparse_attn_reuse(qs, kv, idx, top_k=k, window=W, seq_lens=seq, flags=UNI, kv_fp8=f8)
    torch.cuda.synchronize()
    codes, scales = split_copy(f8, B, Hkv, cap)
    deq = codes.view(torch.float8_e4m3fn).double().cpu().numpy() * scales.double().cpu().numpy()[:, :, None, :, None]
    idx_np = idx.cpu().numpy()
    assert idx_np.shape[-1] == 8 * k
    stats = OutStats()
    for b, L in enumerate(lengths):
        ref, _ = orc.sparse_attention_rows(f32(qs[b])[None], deq[b, :, :, 0], deq[b, :, :, 1], idx_np[b][None],
                                           np.array([L]), W, orc.default_scale(128))
        stats.add(f32(o8[b]), ref[0])
    stats.check("union fp8 sparse decode o")
