"""GPU parity of the prefill path (full layer + selection + sparse layers) with the oracle."""
import numpy as np
import pytest
import torch

import token_level_sparse_hs_amd as hs
from token_level_sparse_hs_amd import synth
from parity import check_prefill, f32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def make_inputs(B, n_q, n_kv, Hq, Hkv, seed, cap=None, n_sparse=1):
    cap = cap or n_kv
    kv = torch.zeros((B, Hkv, cap, 2, 128), dtype=torch.bfloat16, device=DEV)
    kv[:, :, :n_kv] = synth.randn_bf16((B, Hkv, n_kv, 2, 128), seed, DEV)
    q = synth.randn_bf16((B, n_q, Hq, 128), seed + 1, DEV)
    qs = [synth.randn_bf16((B, n_q, Hq, 128), seed + 2 + i, DEV) for i in range(n_sparse)]
    return q, kv, qs


def run(B, n_q, n_kv, Hq, Hkv, k, W, seed, rows=None, flags=0, cap=None, n_sparse=1, kv_override=None):
    print(f"[case] B={B} n_q={n_q} n_kv={n_kv} Hq={Hq} Hkv={Hkv} k={k} W={W} seed={seed} flags={flags}", flush=True)
    q, kv, qs = make_inputs(B, n_q, n_kv, Hq, Hkv, seed, cap, n_sparse)
    if kv_override is not None:
        kv = kv_override(kv)
    o, lse, idx = hs.full_attn_select(q, kv, n_kv, top_k=k, window=W, flags=flags)
    osp = [hs.sparse_attn_reuse(x, kv, idx, top_k=k, window=W, n_kv=n_kv) for x in qs]
    torch.cuda.synchronize()
    return check_prefill(q, kv, n_kv, k, W, o, lse, idx, rows=rows, q_sparse=qs, o_sparse=osp), (q, kv, o, lse, idx, osp)


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (8, 1), (8, 2), (4, 2), (2, 2)])
def test_small_full_prefill(Hq, Hkv):
    run(1, 300, 300, Hq, Hkv, 24, 16, seed=100 + Hq + Hkv)


def test_ragged_chunk_and_batch():
    # chunk of 77 rows at the end of a 517-token cache, two sequences
    run(2, 77, 517, 8, 2, 40, 33, seed=200, cap=600)


def test_tiny_workload_all_rows():
    w = synth.WORKLOADS["tiny"]
    print("[case] tiny workload", flush=True)
    case = synth.make_prefill_case(w, DEV)
    q, kv = case["q_full"], case["kv"]
    o, lse, idx = hs.full_attn_select(q, kv, w.n_kv, top_k=w.top_k, window=w.window)
    osp = [hs.sparse_attn_reuse(x, kv, idx, top_k=w.top_k, window=w.window, n_kv=w.n_kv) for x in case["q_sparse"]]
    torch.cuda.synchronize()
    res = check_prefill(q, kv, w.n_kv, w.top_k, w.window, o, lse, idx, q_sparse=case["q_sparse"], o_sparse=osp)
    print("tiny swaps", res["swaps"], "full", res["full"].max_abs, res["full"].mean_abs,
          "sparse", res["sparse"].max_abs, res["sparse"].mean_abs)


def test_exact_rescan_flag_matches():
    """The exact-rescan path (forced for every row) gives the same selection."""
    a, (q, kv, o, lse, idx, _) = run(1, 700, 700, 8, 2, 32, 8, seed=300)
    o2, lse2, idx2 = hs.full_attn_select(q, kv, 700, top_k=32, window=8, flags=hs.HS_FLAG_EXACT_RESCAN)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    # rescan scores are recomputed with fp32 VALU dot products: the sets agree
    # exactly except at near-ties, which the oracle check below bounds
    check_prefill(q, kv, 700, 32, 8, o2, lse2, idx2)


def test_k0_is_sliding_window():
    run(1, 200, 200, 8, 1, 0, 17, seed=400)


def test_budget_covers_context_equals_full():
    """k + W >= n: the sparse layer must equal full attention of its own q."""
    n, W = 256, 16
    k = n - W
    q, kv, qs = make_inputs(1, n, n, 8, 2, 500)
    o, lse, idx = hs.full_attn_select(q, kv, n, top_k=k, window=W)
    o_sp = hs.sparse_attn_reuse(qs[0], kv, idx, top_k=k, window=W, n_kv=n)
    o_full, _, _ = hs.full_attn_select(qs[0], kv, n, top_k=0, window=W)
    torch.cuda.synchronize()
    d = (o_sp.float() - o_full.float()).abs()
    assert d.max().item() <= 2e-2 and d.mean().item() <= 2e-3


def test_duplicate_keys_tie_to_lower_index():
    """Identical key rows give exactly equal scores; the lower index wins."""
    n, k, W = 160, 3, 8
    q, kv, qs = make_inputs(1, n, n, 4, 1, 600)
    t = n - 1
    d = q[0, t].float().sum(0)
    hot = (d / d.norm() * 20).to(torch.bfloat16)
    for j in (5, 40, 41, 90):
        kv[0, 0, j, 0] = hot
    o, lse, idx = hs.full_attn_select(q, kv, n, top_k=k, window=W)
    torch.cuda.synchronize()
    assert idx[0, t, 0].tolist() == [5, 40, 41]
    check_prefill(q, kv, n, k, W, o, lse, idx, rows=[t, t - 1, 100])


def test_threshold_path_long_rows():
    """Rows with many more candidates than the buffer capacity (sampled
    thresholds, filtered append, exact select), sampled rows checked."""
    n = 6000
    rows = [0, 40, 41, 42, 100, 1000, 2047, 3000, 4500, 5998, 5999]
    run(1, n, n, 8, 2, 64, 32, seed=700, rows=rows)


def test_large_k_buffer_path():
    """Buffer capacity above the register capacity (large k)."""
    n = 12000
    rows = [0, 3063, 3064, 5000, 9000, 11999]
    run(1, n, n, 8, 1, 3000, 64, seed=800, rows=rows)


def test_large_k_wave128_rows():
    """k > 2560: sampled rows keep about 1.77 k > 5120 candidates, which the
    one-wave selection takes with 128 register slots per lane (rows of up to
    8192) instead of queueing them for the block-wide path."""
    n = 16000
    rows = [9300, 10000, 11111, 12500, 14000, 15000, 15999]
    run(1, n, n, 8, 1, 3000, 64, seed=810, rows=rows)


def test_rescan_streaming_long_rows():
    """Exact rescan of rows longer than the register capacity."""
    n = 9500
    rows = [100, 8000, 9499]
    run(1, n, n, 4, 1, 64, 16, seed=900, rows=rows, flags=hs.HS_FLAG_EXACT_RESCAN)


def test_threshold_wave32_all_rows():
    """Rows of 1025..2048 samples take the one-wave threshold with 32
    register slots per lane (n = 1800, k = 64, stride 1: 1792 samples);
    every row is checked."""
    run(1, 1800, 1800, 8, 2, 64, 32, seed=1000)


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (8, 2)])
@pytest.mark.parametrize("n", [1, 5, 63, 64, 65, 129])
def test_short_contexts(n, Hq, Hkv):
    """One to three 64-key tiles: the first and the last tile of the full
    layer's pipeline (V of a tile consumed one tile after its K) meet, with
    and without tiles between them; k and W small so that rows select."""
    run(1, n, n, Hq, Hkv, 4, 2, seed=1100 + n + Hkv)


def test_short_chunk_over_two_tiles():
    """Three query rows at the end of a 70-token cache (two tiles, G = 4)."""
    run(1, 3, 70, 8, 2, 8, 4, seed=1200)
