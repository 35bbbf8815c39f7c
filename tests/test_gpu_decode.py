"""GPU parity of the decode path: append + full attention + select once, then
sparse layers that reuse the one selection, over several steps."""
import numpy as np
import pytest
import torch

import oracle as orc
import token_level_sparse_hs_amd as hs
from token_level_sparse_hs_amd import synth
from parity import OutStats, check_idx_row, f32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_decode(lengths, steps, Hq, Hkv, k, W, seed, n_sparse=2):
    print(f"[case] decode lengths={lengths} steps={steps} Hq={Hq} Hkv={Hkv} k={k} W={W} seed={seed}", flush=True)
    B = len(lengths)
    cap = max(lengths) + steps
    kv = torch.zeros((B, Hkv, cap, 2, 128), dtype=torch.bfloat16, device=DEV)
    for b, L in enumerate(lengths):
        kv[b, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), seed + 17 * b, DEV)
    Ks = [kv[b, :, :, 0].float().cpu().numpy() for b in range(B)]
    Vs = [kv[b, :, :, 1].float().cpu().numpy() for b in range(B)]
    scale = orc.default_scale(128)
    full, sparse = OutStats(), OutStats()
    swaps = 0
    for s in range(steps):
        cur = [L + s + 1 for L in lengths]
        seq_lens = torch.tensor(cur, dtype=torch.int32, device=DEV)
        q = synth.randn_bf16((B, Hq, 128), seed + 1000 + s, DEV)
        kv_new = synth.randn_bf16((B, Hkv, 2, 128), seed + 2000 + s, DEV)
        qs = [synth.randn_bf16((B, Hq, 128), seed + 3000 + 10 * s + i, DEV) for i in range(n_sparse)]
        o, lse, idx = hs.decode_step(q, kv_new, kv, seq_lens, max(cur), top_k=k, window=W)
        osp = [hs.sparse_attn_reuse(x, kv, idx, top_k=k, window=W, seq_lens=seq_lens) for x in qs]
        torch.cuda.synchronize()
        o_np, lse_np, idx_np = f32(o), lse.cpu().numpy(), idx.cpu().numpy()
        for b in range(B):
            ref = orc.decode_step(f32(q[b]), [f32(x[b]) for x in qs], f32(kv_new[b]), Ks[b], Vs[b], cur[b], k, W, scale)
            full.add(o_np[b], ref["o_full"])
            assert np.abs(lse_np[b] - ref["lse_full"]).max() <= 1e-3
            for g in range(Hkv):
                swaps += check_idx_row(idx_np[b, g], ref["idx"][g], ref["sigma"][g], ref["tau"][g], cur[b] - 1, W, k,
                                       where=f"step{s} b{b} g{g}")
            pos = np.array([cur[b] - 1])
            for x, osx in zip(qs, osp):
                r, _ = orc.sparse_attention_rows(f32(x[b])[None], Ks[b], Vs[b], idx_np[b][None], pos, W, scale)
                sparse.add(f32(osx[b]), r[0])
        # the cache row written by the library equals kv_new
        for b in range(B):
            assert torch.equal(kv[b, :, cur[b] - 1], kv_new[b])
    full.check("decode full o")
    sparse.check("decode sparse o")
    return swaps


def test_decode_small_batch():
    run_decode([300, 1200, 5000], 3, 8, 2, 64, 32, seed=11)


def test_decode_gqa4_short_rows():
    # rows with fewer candidates than k, and a row inside the window
    run_decode([5, 40, 100, 700], 2, 4, 1, 64, 32, seed=12)


def test_decode_exact_ties():
    B, Hq, Hkv, k, W = 1, 8, 1, 4, 4
    L = 64
    kv = torch.zeros((B, Hkv, L + 1, 2, 128), dtype=torch.bfloat16, device=DEV)
    kv[0, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), 77, DEV)
    q = synth.randn_bf16((B, Hq, 128), 78, DEV)
    hot = (q[0].float().sum(0) / q[0].float().sum(0).norm() * 20).to(torch.bfloat16)
    for j in (3, 9, 10, 30, 31, 50):
        kv[0, 0, j, 0] = hot
    kv_new = synth.randn_bf16((B, Hkv, 2, 128), 79, DEV)
    seq_lens = torch.tensor([L + 1], dtype=torch.int32, device=DEV)
    o, lse, idx = hs.decode_step(q, kv_new, kv, seq_lens, L + 1, top_k=k, window=W)
    torch.cuda.synchronize()
    assert idx[0, 0].tolist() == [3, 9, 10, 30]


def test_decode_long_rows_filtered_select():
    """Rows longer than the register capacity take the sampled-threshold
    filter inside the decode select."""
    run_decode([20000, 70000], 2, 8, 1, 512, 64, seed=13, n_sparse=1)


def test_decode_sampled_threshold_overshoot():
    """Long rows are filtered by the m-th largest of their samples: every
    2^s-th candidate score, s >= 2 the smallest shift leaving at most 16384
    of them. Keys placed exactly at the sampled positions and aimed at the
    queries push that threshold above the row's k-th score, so fewer than k
    keys survive the filter: the selection must fall back to the whole row
    and still return the exact top k (most of them those planted keys)."""
    L, Hq, Hkv, k, W = 40000, 4, 1, 512, 16
    print(f"[case] decode sampled-threshold overshoot L={L} k={k}", flush=True)
    kv = torch.zeros((1, Hkv, L + 1, 2, 128), dtype=torch.bfloat16, device=DEV)
    kv[0, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), 81, DEV)
    q = synth.randn_bf16((1, Hq, 128), 82, DEV)
    u = q[0].float().sum(0)
    u = u / u.norm() * (128 ** 0.5)
    ncand = L - W + 1  # candidates of the row after the append (p = L)
    shift = 2
    while -(-ncand // (1 << shift)) > 16384:
        shift += 1
    pos = torch.arange(0, ncand, 1 << shift, device=DEV)
    noise = synth.randn_bf16((len(pos), 128), 83, DEV).float()
    kv[0, 0, pos, 0] = (0.8 * u[None] + 0.6 * noise).to(torch.bfloat16)
    kv_new = synth.randn_bf16((1, Hkv, 2, 128), 84, DEV)
    seq_lens = torch.tensor([L + 1], dtype=torch.int32, device=DEV)
    o, lse, idx = hs.decode_step(q, kv_new, kv, seq_lens, L + 1, top_k=k, window=W)
    torch.cuda.synchronize()
    Ks, Vs = kv[0, :, :, 0].float().cpu().numpy(), kv[0, :, :, 1].float().cpu().numpy()
    ref = orc.decode_step(f32(q[0]), [], f32(kv_new[0]), Ks, Vs, L + 1, k, W, orc.default_scale(128))
    check_idx_row(idx.cpu().numpy()[0, 0], ref["idx"][0], ref["sigma"][0], ref["tau"][0], L, W, k, where="overshoot")
    planted = set(pos.tolist())
    assert sum(int(j) in planted for j in ref["idx"][0]) > k // 2


@pytest.mark.parametrize("tail", [1, 2, 3])
def test_decode_filter_ragged_tail_keeps_last_keys(tail):
    """The sliced selection reads score rows in 16-byte pieces; when |C(p)| is
    not a multiple of 4 the last piece runs past the row's range. Keys planted
    at the row's last `tail` candidates, aimed at the queries, are the top of
    the row and must all be selected (and the rest must match the oracle)."""
    W, k, Hq, Hkv = 64, 256, 4, 1
    ncand = 20000 + tail
    L = ncand + W - 1  # after the append, p = L and |C(p)| = L - W + 1 = ncand
    print(f"[case] decode ragged tail ncand={ncand}", flush=True)
    kv = torch.zeros((1, Hkv, L + 1, 2, 128), dtype=torch.bfloat16, device=DEV)
    kv[0, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), 91 + tail, DEV)
    q = synth.randn_bf16((1, Hq, 128), 92 + tail, DEV)
    u = q[0].float().sum(0)
    u = u / u.norm() * (128 ** 0.5)
    planted = list(range(ncand - tail, ncand))
    kv[0, 0, planted, 0] = (2.0 * u).to(torch.bfloat16)
    kv_new = synth.randn_bf16((1, Hkv, 2, 128), 93 + tail, DEV)
    seq_lens = torch.tensor([L + 1], dtype=torch.int32, device=DEV)
    o, lse, idx = hs.decode_step(q, kv_new, kv, seq_lens, L + 1, top_k=k, window=W)
    torch.cuda.synchronize()
    Ks, Vs = kv[0, :, :, 0].float().cpu().numpy(), kv[0, :, :, 1].float().cpu().numpy()
    ref = orc.decode_step(f32(q[0]), [], f32(kv_new[0]), Ks, Vs, L + 1, k, W, orc.default_scale(128))
    got = idx.cpu().numpy()[0, 0]
    check_idx_row(got, ref["idx"][0], ref["sigma"][0], ref["tau"][0], L, W, k, where="ragged tail")
    assert set(planted) <= set(int(j) for j in got), "a planted last candidate was not selected"


def test_decode_slicewise_copy_dense_slices():
    """Rows with more than 16 survivors per thread gather the slices'
    survivors slice by slice (two per lane per pass, a loop beyond 128).
    Clusters of keys aimed at the queries put 300 and 100 survivors into two
    slices; every planted key must be selected and the rest match the oracle."""
    W, k, Hq, Hkv = 64, 4096, 4, 1
    ncand = 300000
    L = ncand + W - 1
    print(f"[case] decode slice-wise copy ncand={ncand} k={k}", flush=True)
    kv = torch.zeros((1, Hkv, L + 1, 2, 128), dtype=torch.bfloat16, device=DEV)
    kv[0, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), 171, DEV)
    q = synth.randn_bf16((1, Hq, 128), 172, DEV)
    u = q[0].float().sum(0)
    u = u / u.norm() * (128 ** 0.5)
    planted = list(range(100000, 100300)) + list(range(200000, 200100))
    kv[0, 0, planted, 0] = (2.0 * u).to(torch.bfloat16)
    kv_new = synth.randn_bf16((1, Hkv, 2, 128), 173, DEV)
    seq_lens = torch.tensor([L + 1], dtype=torch.int32, device=DEV)
    o, lse, idx = hs.decode_step(q, kv_new, kv, seq_lens, L + 1, top_k=k, window=W)
    torch.cuda.synchronize()
    Ks, Vs = kv[0, :, :, 0].float().cpu().numpy(), kv[0, :, :, 1].float().cpu().numpy()
    ref = orc.decode_step(f32(q[0]), [], f32(kv_new[0]), Ks, Vs, L + 1, k, W, orc.default_scale(128))
    got = idx.cpu().numpy()[0, 0]
    check_idx_row(got, ref["idx"][0], ref["sigma"][0], ref["tau"][0], L, W, k, where="slice-wise copy")
    assert set(planted) <= set(int(j) for j in got), "a planted key was not selected"
    stats = OutStats()
    stats.add(f32(o[0]), ref["o_full"])
    stats.check("decode full o")


def test_decode_streaming_select():
    """k close to the row length defeats the sample filter: streaming select."""
    run_decode([9000], 1, 4, 1, 8000, 16, seed=14, n_sparse=1)


def test_decode_batch_block_merge():
    """256 (b, g) rows: each sparse row is split over the four waves of one
    block, which merge their partials in LDS. Short rows leave splits with no
    kept key (all idx entries padding) or no source position at all."""
    rng = np.random.default_rng(15)
    lengths = [1, 5, 30, 63, 64, 65, 200, 319, 320, 321, 1000, 2500]
    lengths += [int(x) for x in rng.integers(1, 2500, size=64 - len(lengths))]
    run_decode(lengths, 1, 32, 4, 256, 64, seed=15, n_sparse=1)
