"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, checked on sampled rows (sequences) the oracle can compute
one by one."""
import numpy as np
import pytest
import torch

import oracle as orc
import token_level_sparse_hs_amd as hs
from token_level_sparse_hs_amd import synth
from parity import OutStats, cache_np, check_idx_row, check_prefill, f32, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_prefill_workload(name, evenly=8, flags=0):
    w = synth.WORKLOADS[name]
    score = "prob" if flags & hs.HS_FLAG_PROB_SCORE else "logit"
    blocks = bool(flags & hs.HS_FLAG_BLOCK_SELECT)
    union = bool(flags & hs.HS_FLAG_HEAD_UNION)
    print(f"[case] workload {name}: B={w.B} n_q={w.n_q} n_kv={w.n_kv} k={w.top_k} W={w.window} score={score} blocks={blocks}",
          flush=True)
    case = synth.make_prefill_case(w, DEV, kv_capacity=w.n_kv + w.decode_steps)
    q, kv, qs = case["q_full"], case["kv"], case["q_sparse"]
    o, lse, idx = hs.full_attn_select(q, kv, w.n_kv, top_k=w.top_k, window=w.window, flags=flags)
    osp = [hs.sparse_attn_reuse(x, kv, idx, top_k=w.top_k, window=w.window, n_kv=w.n_kv, flags=flags) for x in qs]
    torch.cuda.synchronize()
    pos, spans = case["needles"]
    rows = sample_rows(w.n_q, w.n_kv, w.top_k, w.window, spans, evenly)
    print(f"[case] checking rows {rows}", flush=True)
    res = check_prefill(q, kv, w.n_kv, w.top_k, w.window, o, lse, idx, rows=rows, q_sparse=qs, o_sparse=osp,
                        score=score, blocks=blocks, union=union)
    print(f"[case] {name}: near-tie swaps {res['swaps']}, full max-abs {res['full'].max_abs:.2e} "
          f"mean {res['full'].mean_abs:.2e}, sparse max-abs {res['sparse'].max_abs:.2e}", flush=True)
    # needles: the planted keys should mostly be selected by their span rows
    if pos:
        idx_np = idx.cpu().numpy()
        hit = tot = 0
        for p_, t0 in zip(pos, spans):
            for g in range(w.Hkv):
                tot += 1
                hit += int(p_ in set(idx_np[0, t0, g].tolist()))
        print(f"[case] {name}: needles selected by their span's first row: {hit}/{tot}", flush=True)
        assert hit > 0
    return w, case, idx


def test_prefill32k_full_size():
    run_prefill_workload("prefill32k")


def test_prefill32k_full_size_prob_score():
    """The probability selection score at full size (attention, then the
    sampled threshold and the QK-only candidate pass on its lse)."""
    run_prefill_workload("prefill32k", evenly=4, flags=hs.HS_FLAG_PROB_SCORE)


def test_prefill32k_full_size_block_select():
    """Block-level selection at full size: block scores from the attention
    pass, then the top top_k/64 blocks per row."""
    run_prefill_workload("prefill32k", evenly=4, flags=hs.HS_FLAG_BLOCK_SELECT)


def test_prefill32k_full_size_head_union():
    """Union of per-head top-k at full size: eight one-head passes, the
    union rows of 8 * 2048 entries, the sparse layers over them."""
    run_prefill_workload("prefill32k", evenly=3, flags=hs.HS_FLAG_HEAD_UNION)


def test_chunk128k_full_size():
    run_prefill_workload("chunk128k", evenly=4)


def decode_check(kv, lengths, steps_data, w, seqs_to_check, steps):
    """Runs `steps` decode steps on the whole batch; checks chosen sequences."""
    B = len(lengths)
    host = {b: cache_np(kv, b, lengths[b] + steps) for b in seqs_to_check}
    scale = orc.default_scale(128)
    full, sparse = OutStats(), OutStats()
    swaps = 0
    for s in range(steps):
        st = steps_data[s]
        cur = [L + s + 1 for L in lengths]
        seq_lens = torch.tensor(cur, dtype=torch.int32, device=DEV)
        o, lse, idx = hs.decode_step(st["q_full"], st["kv_new"], kv, seq_lens, max(cur), top_k=w.top_k,
                                     window=w.window)
        osp = [hs.sparse_attn_reuse(x, kv, idx, top_k=w.top_k, window=w.window, seq_lens=seq_lens)
               for x in st["q_sparse"]]
        torch.cuda.synchronize()
        idx_np = idx.cpu().numpy()
        for b in seqs_to_check:
            K, V = host[b]
            ref = orc.decode_step(f32(st["q_full"][b]), [], f32(st["kv_new"][b]), K, V, cur[b], w.top_k, w.window,
                                  scale)
            full.add(f32(o[b]), ref["o_full"])
            for g in range(w.Hkv):
                swaps += check_idx_row(idx_np[b, g], ref["idx"][g], ref["sigma"][g], ref["tau"][g], cur[b] - 1,
                                       w.window, w.top_k, where=f"step{s} b{b} g{g}")
            for x, osx in zip(st["q_sparse"], osp):
                r, _ = orc.sparse_attention_rows(f32(x[b])[None], K, V, idx_np[b][None], np.array([cur[b] - 1]),
                                                 w.window, scale)
                sparse.add(f32(osx[b]), r[0])
        print(f"[case] decode step {s} checked", flush=True)
    full.check("decode full o")
    sparse.check("decode sparse o")
    return swaps


def test_decode64_full_size():
    w = synth.WORKLOADS["decode64"]
    lengths = synth.decode_lengths(w)
    steps = 2
    print(f"[case] decode64: {len(lengths)} sequences, sum of lengths {sum(lengths)}", flush=True)
    case = synth.make_decode_case(w, DEV, lengths, steps)
    order = np.argsort(lengths)
    check = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
    decode_check(case["kv"], lengths, case["steps"], w, check, steps)


def test_ctx1m_prefill_and_decode():
    w, case, idx = run_prefill_workload("ctx1m", evenly=2)
    # decode on the same cache: the chunk's rows are in place, append after
    kv = case["kv"]
    del case["q_full"], case["q_sparse"]
    steps = 2
    steps_data = [{
        "q_full": synth.randn_bf16((1, w.Hq, 128), synth.seed_for(w.cid, synth.T_QDEC, s), DEV),
        "q_sparse": [synth.randn_bf16((1, w.Hq, 128), synth.seed_for(w.cid, synth.T_QDEC + 1 + i, s), DEV)
                     for i in range(w.sparse_layers)],
        "kv_new": synth.randn_bf16((1, w.Hkv, 2, 128), synth.seed_for(w.cid, synth.T_KVNEW, s), DEV),
    } for s in range(steps)]
    decode_check(kv, [w.n_kv], steps_data, w, [0], steps)
