"""hs_decode_step_noalloc (the decode step on the library's static scratch)
against hs_decode_step with a caller workspace, through the C ABI: two calls
in a row, the second with a smaller batch and shorter sequences, each must
give bit-identical o, lse, idx and cache writes (same kernels, same launch
plan; only the scratch differs). A step whose plan needs more than the
static scratch is rejected on the host."""
import ctypes

import pytest
import torch

import token_level_sparse_hs_amd as hs
from token_level_sparse_hs_amd import _lib, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def step_pair(lengths, Hq, Hkv, k, W, seed, flags=0):
    B = len(lengths)
    print(f"[case] noalloc decode lengths={lengths} Hq={Hq} Hkv={Hkv} k={k} W={W} flags={flags}", flush=True)
    cap = max(lengths) + 1
    kv_a = torch.zeros((B, Hkv, cap, 2, 128), dtype=torch.bfloat16, device=DEV)
    for b, L in enumerate(lengths):
        kv_a[b, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), seed + b, DEV)
    kv_b = kv_a.clone()
    q = synth.randn_bf16((B, Hq, 128), seed + 100, DEV)
    kv_new = synth.randn_bf16((B, Hkv, 2, 128), seed + 101, DEV)
    seq = torch.tensor([L + 1 for L in lengths], dtype=torch.int32, device=DEV)
    o1, lse1, idx1 = hs.decode_step_noalloc(q, kv_new, kv_a, seq, cap, top_k=k, window=W, flags=flags)
    o2, lse2, idx2 = hs.decode_step(q, kv_new, kv_b, seq, cap, top_k=k, window=W, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2)
    assert torch.equal(o1, o2)
    assert torch.equal(lse1, lse2)
    assert torch.equal(kv_a, kv_b)


def test_noalloc_decode_matches_workspace_call_twice():
    # first call: longer rows (sliced selection for the 200K sequence), then a smaller one
    step_pair([5000, 200000, 300, 70000], 32, 4, 2048, 512, seed=3000)
    step_pair([1000, 200], 32, 4, 256, 64, seed=3100)


def test_noalloc_decode_block_selection_and_small_batch():
    step_pair([4000, 900, 60], 16, 2, 128, 32, seed=3200, flags=hs.HS_FLAG_BLOCK_SELECT)


def test_noalloc_rejects_plans_beyond_the_static_scratch():
    """64 sequences of 256K tokens need far more score-row scratch than the
    library's 64 MiB: rejected on the host with HS_ERR_WORKSPACE."""
    lib = _lib.load()
    s = hs.make_shape(batch=64, n_q=1, n_kv=0, kv_capacity=262145, q_heads=32, kv_heads=4, top_k=2048, window=512)
    assert _lib.workspace_size(_lib.HS_OP_DECODE_STEP, s, 262145) > 64 << 20
    fake = ctypes.c_void_p(1 << 20)
    st = lib.hs_decode_step_noalloc(ctypes.byref(s), fake, fake, fake, fake, 262145, fake, None, fake, None)
    assert st == _lib.HS_ERR_WORKSPACE
    assert b"static scratch" in lib.hs_last_error()
