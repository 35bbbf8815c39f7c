"""GPU parity of the probability (softmax-normalised) selection score with
the oracle: sigma'(j) = max over the group's heads of s_h(j) - lse_h, the
log of the largest attention probability the group gives token j. Outputs
o / lse are those of the logit path; the selection is checked against the
oracle's probability scores with the same near-tie rule."""
import numpy as np
import pytest
import torch

import oracle as orc
import token_level_sparse_hs_amd as hs
from token_level_sparse_hs_amd import synth
from parity import OutStats, check_idx_row, check_prefill, f32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PROB = hs.HS_FLAG_PROB_SCORE


def prefill(B, n_q, n_kv, Hq, Hkv, k, W, seed, flags=PROB, with_lse=True):
    print(f"[case] prob prefill B={B} n_q={n_q} n_kv={n_kv} Hq={Hq} Hkv={Hkv} k={k} W={W} flags={flags}", flush=True)
    kv = torch.zeros((B, Hkv, n_kv + 3, 2, 128), dtype=torch.bfloat16, device=DEV)
    kv[:, :, :n_kv] = synth.randn_bf16((B, Hkv, n_kv, 2, 128), seed, DEV)
    q = synth.randn_bf16((B, n_q, Hq, 128), seed + 1, DEV)
    qs = synth.randn_bf16((B, n_q, Hq, 128), seed + 2, DEV)
    o, lse, idx = hs.full_attn_select(q, kv, n_kv, top_k=k, window=W, flags=flags, with_lse=with_lse)
    osp = hs.sparse_attn_reuse(qs, kv, idx, top_k=k, window=W, n_kv=n_kv)
    torch.cuda.synchronize()
    return check_prefill(q, kv, n_kv, k, W, o, lse, idx, q_sparse=[qs], o_sparse=[osp], score="prob")


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (32, 4), (8, 2), (2, 2)])
def test_prob_prefill_small(Hq, Hkv):
    # n_kv - W + 1 > 3k + 256: the sampled threshold filters the candidates
    prefill(1, 260, 700, Hq, Hkv, 64, 24, seed=1100 + Hq)


def test_prob_prefill_chunk_batch_no_lse_buffer():
    # lse not requested: the library keeps it in the workspace for the score
    prefill(2, 90, 610, 8, 2, 40, 17, seed=1200, with_lse=False)


def test_prob_prefill_exact_rescan():
    prefill(1, 150, 500, 8, 2, 48, 16, seed=1300, flags=PROB | hs.HS_FLAG_EXACT_RESCAN)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (32, 4), (2, 2)])
def test_prob_decode(Hq, Hkv):
    lengths = [300, 1200, 5000, 20000]
    B, k, W = len(lengths), 64, 32
    print(f"[case] prob decode lengths={lengths} Hq={Hq} Hkv={Hkv}", flush=True)
    cap = max(lengths) + 1
    kv = torch.zeros((B, Hkv, cap, 2, 128), dtype=torch.bfloat16, device=DEV)
    for b, L in enumerate(lengths):
        kv[b, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), 1400 + 7 * Hq + b, DEV)
    seq = torch.tensor([L + 1 for L in lengths], dtype=torch.int32, device=DEV)
    q = synth.randn_bf16((B, Hq, 128), 1410, DEV)
    kv_new = synth.randn_bf16((B, Hkv, 2, 128), 1411, DEV)
    o, lse, idx = hs.decode_step(q, kv_new, kv, seq, max(lengths) + 1, top_k=k, window=W, flags=PROB)
    torch.cuda.synchronize()
    full = OutStats()
    idx_np = idx.cpu().numpy()
    for b, L in enumerate(lengths):
        K = kv[b, :, :, 0].float().cpu().numpy()
        V = kv[b, :, :, 1].float().cpu().numpy()
        K[:, L] = 0.0  # the oracle appends kv_new itself
        ref = orc.decode_step(f32(q[b]), [], f32(kv_new[b]), K, V, L + 1, k, W, orc.default_scale(128), score="prob")
        full.add(f32(o[b]), ref["o_full"])
        assert np.abs(lse[b].cpu().numpy() - ref["lse_full"]).max() <= 1e-3
        for g in range(Hkv):
            check_idx_row(idx_np[b, g], ref["idx"][g], ref["sigma"][g], ref["tau"][g], L, W, k, where=f"b{b} g{g}")
    full.check("decode full o")


def test_prob_score_changes_the_selection():
    """The flag is not a no-op: on random data the two scores pick different
    sets for most rows with G = 8 (they coincide only for G = 1)."""
    n, W, k = 600, 16, 32
    kv = synth.randn_bf16((1, 1, n, 2, 128), 1500, DEV)
    q = synth.randn_bf16((1, 64, 8, 128), 1501, DEV)
    _, _, a = hs.full_attn_select(q, kv, n, top_k=k, window=W)
    _, _, b = hs.full_attn_select(q, kv, n, top_k=k, window=W, flags=PROB)
    torch.cuda.synchronize()
    differ = (a != b).any(dim=-1).float().mean().item()
    assert differ > 0.5, differ
