"""GPU parity of block-level selection with the oracle: C(p) in aligned
64-token blocks, each scored by its best candidate, the top top_k/64 blocks
taken whole. Outputs o / lse are those of the token-level path; rows must be
whole ascending blocks, and the block set may differ from the oracle's only
by near-ties of the block score."""
import numpy as np
import pytest
import torch

import oracle as orc
import token_level_sparse_hs_amd as hs
from token_level_sparse_hs_amd import synth
from parity import OutStats, check_block_row, check_prefill, f32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BLK = hs.HS_FLAG_BLOCK_SELECT


def prefill(B, n_q, n_kv, Hq, Hkv, k, W, seed, with_lse=True):
    print(f"[case] block prefill B={B} n_q={n_q} n_kv={n_kv} Hq={Hq} Hkv={Hkv} k={k} W={W}", flush=True)
    kv = torch.zeros((B, Hkv, n_kv + 3, 2, 128), dtype=torch.bfloat16, device=DEV)
    kv[:, :, :n_kv] = synth.randn_bf16((B, Hkv, n_kv, 2, 128), seed, DEV)
    q = synth.randn_bf16((B, n_q, Hq, 128), seed + 1, DEV)
    qs = synth.randn_bf16((B, n_q, Hq, 128), seed + 2, DEV)
    o, lse, idx = hs.full_attn_select(q, kv, n_kv, top_k=k, window=W, flags=BLK, with_lse=with_lse)
    osp = hs.sparse_attn_reuse(qs, kv, idx, top_k=k, window=W, n_kv=n_kv)
    torch.cuda.synchronize()
    return check_prefill(q, kv, n_kv, k, W, o, lse, idx, q_sparse=[qs], o_sparse=[osp], blocks=True)


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (32, 4), (8, 2), (4, 2), (2, 2)])
def test_block_prefill_small(Hq, Hkv):
    # rows from no candidates through partial last blocks to 20 blocks
    prefill(1, 330, 1300, Hq, Hkv, 128, 24, seed=2100 + Hq)


def test_block_prefill_chunk_batch_no_lse():
    prefill(2, 90, 610, 8, 2, 64, 17, seed=2200, with_lse=False)


def test_block_prefill_k_beyond_rows():
    # top_k larger than every row's candidate count: all blocks, -1 padded
    prefill(1, 100, 300, 8, 2, 512, 8, seed=2300)


@pytest.mark.parametrize("Hq,Hkv,lengths", [
    (8, 2, [40, 300, 1200, 5000, 20000]),   # up to 1024 blocks a row: one wave per row
    (32, 4, [40, 300, 1200, 5000, 20000]),
    (8, 1, [40, 300, 1200, 5000, 20000]),
    (8, 2, [3000, 100_000]),                 # longer rows: one block per row
])
def test_block_decode(Hq, Hkv, lengths):
    B, k, W = len(lengths), 256, 32
    print(f"[case] block decode lengths={lengths} Hq={Hq} Hkv={Hkv}", flush=True)
    cap = max(lengths) + 1
    kv = torch.zeros((B, Hkv, cap, 2, 128), dtype=torch.bfloat16, device=DEV)
    for b, L in enumerate(lengths):
        kv[b, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), 2400 + 7 * Hq + b, DEV)
    seq = torch.tensor([L + 1 for L in lengths], dtype=torch.int32, device=DEV)
    q = synth.randn_bf16((B, Hq, 128), 2410, DEV)
    kv_new = synth.randn_bf16((B, Hkv, 2, 128), 2411, DEV)
    o, lse, idx = hs.decode_step(q, kv_new, kv, seq, max(lengths) + 1, top_k=k, window=W, flags=BLK)
    torch.cuda.synchronize()
    full = OutStats()
    idx_np = idx.cpu().numpy()
    for b, L in enumerate(lengths):
        K = kv[b, :, :, 0].float().cpu().numpy()
        V = kv[b, :, :, 1].float().cpu().numpy()
        K[:, L] = 0.0  # the oracle appends kv_new itself
        ref = orc.decode_step(f32(q[b]), [], f32(kv_new[b]), K, V, L + 1, k, W, orc.default_scale(128), blocks=True)
        full.add(f32(o[b]), ref["o_full"])
        assert np.abs(lse[b].cpu().numpy() - ref["lse_full"]).max() <= 1e-3
        for g in range(Hkv):
            check_block_row(idx_np[b, g], ref["idx"][g], ref["sigma"][g], ref["tau"][g], L, W, k, where=f"b{b} g{g}")
    full.check("decode full o")


def test_block_decode_long_row_filtered():
    """A row with more blocks than one block's registers rank at once
    (600K candidates: 9375 blocks), selected by the sampled filter."""
    L, Hq, Hkv, k, W = 600_000, 8, 1, 2048, 512
    print(f"[case] block decode long row L={L} k={k}", flush=True)
    kv = torch.zeros((1, Hkv, L + 1, 2, 128), dtype=torch.bfloat16, device=DEV)
    kv[0, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), 2500, DEV)
    seq = torch.tensor([L + 1], dtype=torch.int32, device=DEV)
    q = synth.randn_bf16((1, Hq, 128), 2501, DEV)
    kv_new = synth.randn_bf16((1, Hkv, 2, 128), 2502, DEV)
    o, lse, idx = hs.decode_step(q, kv_new, kv, seq, L + 1, top_k=k, window=W, flags=BLK)
    torch.cuda.synchronize()
    K = kv[0, :, :, 0].float().cpu().numpy()
    V = kv[0, :, :, 1].float().cpu().numpy()
    K[:, L] = 0.0
    ref = orc.decode_step(f32(q[0]), [], f32(kv_new[0]), K, V, L + 1, k, W, orc.default_scale(128), blocks=True)
    check_block_row(idx.cpu().numpy()[0, 0], ref["idx"][0], ref["sigma"][0], ref["tau"][0], L, W, k, where="long")
    full = OutStats()
    full.add(f32(o[0]), ref["o_full"])
    full.check("decode full o")


def test_block_select_differs_from_token_select():
    """The flag is not a no-op: block rows are whole blocks, token rows are not."""
    n, W, k = 2000, 16, 128
    kv = synth.randn_bf16((1, 2, n, 2, 128), 2600, DEV)
    q = synth.randn_bf16((1, 64, 8, 128), 2601, DEV)
    _, _, it = hs.full_attn_select(q, kv, n, top_k=k, window=W)
    _, _, ib = hs.full_attn_select(q, kv, n, top_k=k, window=W, flags=BLK)
    torch.cuda.synchronize()
    it, ib = it.cpu().numpy(), ib.cpu().numpy()
    v = ib >= 0
    assert (ib[v] % 64 == np.broadcast_to(np.arange(k), ib.shape)[v] % 64).all()
    assert not np.array_equal(it, ib)
