"""FP8 (e4m3) copy of the cache for the sparse layers: the conversion must
equal the oracle's quantiser byte for byte (codes and scales), and the sparse
layers reading the copy must match the oracle run on the dequantised values
(which are exact bf16 values, so the usual tolerances apply)."""
import numpy as np
import pytest
import torch

import oracle as orc
import token_level_sparse_hs_amd as hs
from token_level_sparse_hs_amd import synth
from parity import OutStats, check_idx_row, f32, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def split_copy(copy, B, Hkv, cap):
    n = B * Hkv * cap * 256
    codes = copy[:n].view(B, Hkv, cap, 2, 128)
    scales = copy[n + B * Hkv * 8:n + B * Hkv * 16].view(torch.float32).view(B, Hkv, 2)
    return codes, scales


def oracle_quantise(kv, n_kv, exps=None):
    """codes [B][Hkv][n][2][128] uint8, exponents [B][Hkv][2], dequantised K, V as float64.
    The exponents come from rows [0, n_kv) unless given (the decode form keeps
    the scales of the cache it was converted from)."""
    x = kv[:, :, :n_kv].float().cpu().numpy().astype(np.float64)
    B, Hkv = x.shape[:2]
    codes = np.zeros(x.shape, np.uint8)
    deq = np.zeros(x.shape)
    if exps is None:
        exps = np.zeros((B, Hkv, 2), np.int64)
        for b in range(B):
            for g in range(Hkv):
                for s in range(2):
                    exps[b, g, s] = orc.fp8_scale_exponent(np.abs(x[b, g, :, s]).max())
    for b in range(B):
        for g in range(Hkv):
            for s in range(2):
                codes[b, g, :, s], deq[b, g, :, s] = orc.quantize_fp8(x[b, g, :, s], int(exps[b, g, s]))
    return codes, exps, deq


def test_fp8_conversion_bit_exact():
    B, Hkv, cap, n = 2, 3, 700, 650
    print(f"[case] fp8 conversion B={B} Hkv={Hkv} n={n}", flush=True)
    kv = torch.zeros((B, Hkv, cap, 2, 128), dtype=torch.bfloat16, device=DEV)
    kv[:, :, :n] = synth.randn_bf16((B, Hkv, n, 2, 128), 1600, DEV)
    kv[0, 1, :n] *= 37.5              # a head with larger values (positive exponent)
    kv[1, 2, :n, 1] *= 1e-3           # tiny V values (negative exponent, subnormal codes)
    kv[1, 0, :n, 0] = 0.0             # an all-zero K head (exponent 0)
    copy = hs.kv_to_fp8(kv, n_kv=n)
    torch.cuda.synchronize()
    codes, scales = split_copy(copy, B, Hkv, cap)
    ref_codes, exps, _ = oracle_quantise(kv, n)
    got = codes[:, :, :n].cpu().numpy()
    assert np.array_equal(got, ref_codes), int((got != ref_codes).sum())
    assert np.array_equal(scales.cpu().numpy(), np.ldexp(1.0, exps).astype(np.float32))


def test_fp8_decode_append_row():
    B, Hkv, cap = 3, 2, 300
    lengths = [100, 250, 7]
    print("[case] fp8 decode append", flush=True)
    kv = torch.zeros((B, Hkv, cap, 2, 128), dtype=torch.bfloat16, device=DEV)
    for b, L in enumerate(lengths):
        kv[b, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), 1610 + b, DEV)
    copy = hs.kv_to_fp8(kv, n_kv=cap)
    _, exps, _ = oracle_quantise(kv, cap)
    new = synth.randn_bf16((B, Hkv, 2, 128), 1620, DEV)
    new[0, 0, 0, :4] = torch.tensor([1e4, -1e4, 3.0, 0.0], dtype=torch.bfloat16)  # beyond the range: saturates
    seq = torch.tensor([L + 1 for L in lengths], dtype=torch.int32, device=DEV)
    for b, L in enumerate(lengths):
        kv[b, :, L] = new[b]
    hs.kv_to_fp8(kv, seq_lens=seq, out=copy)
    torch.cuda.synchronize()
    codes, _ = split_copy(copy, B, Hkv, cap)
    for b, L in enumerate(lengths):
        for g in range(Hkv):
            for s in range(2):
                want, _ = orc.quantize_fp8(new[b, g, s].float().cpu().numpy().astype(np.float64), int(exps[b, g, s]))
                assert np.array_equal(codes[b, g, L, s].cpu().numpy(), want), (b, g, s)


def sparse_check(q_sp, o_sp, deqK, deqV, idx_np, pos_rows, W, scale, b, stats):
    ref, _ = orc.sparse_attention_rows(q_sp, deqK, deqV, idx_np, pos_rows, W, scale)
    stats.add(o_sp, ref)


@pytest.mark.parametrize("Hq,Hkv", [(32, 4), (8, 2), (4, 1)])
def test_fp8_sparse_prefill(Hq, Hkv):
    B, n_q, n_kv, k, W = 2, 200, 600, 64, 40
    print(f"[case] fp8 sparse prefill Hq={Hq} Hkv={Hkv}", flush=True)
    kv = synth.randn_bf16((B, Hkv, n_kv, 2, 128), 1700 + Hq, DEV)
    q = synth.randn_bf16((B, n_q, Hq, 128), 1701, DEV)
    qs = synth.randn_bf16((B, n_q, Hq, 128), 1702, DEV)
    _, _, idx = hs.full_attn_select(q, kv, n_kv, top_k=k, window=W, with_lse=False)
    copy = hs.kv_to_fp8(kv, n_kv=n_kv)
    o8 = hs.sparse_attn_reuse(qs, kv, idx, top_k=k, window=W, n_kv=n_kv, kv_fp8=copy)
    torch.cuda.synchronize()
    _, _, deq = oracle_quantise(kv, n_kv)
    pos = orc.query_positions(n_q, n_kv)
    stats = OutStats()
    for b in range(B):
        sparse_check(f32(qs[b]), f32(o8[b]), deq[b, :, :, 0], deq[b, :, :, 1], idx[b].cpu().numpy(), pos, W,
                     orc.default_scale(128), b, stats)
    stats.check("fp8 sparse prefill o")


def test_fp8_sparse_decode():
    lengths = [300, 1200, 5000, 64, 2]
    B, Hq, Hkv, k, W = len(lengths), 32, 4, 256, 64
    print(f"[case] fp8 sparse decode lengths={lengths}", flush=True)
    cap = max(lengths) + 1
    kv = torch.zeros((B, Hkv, cap, 2, 128), dtype=torch.bfloat16, device=DEV)
    for b, L in enumerate(lengths):
        kv[b, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), 1800 + b, DEV)
    seq = torch.tensor([L + 1 for L in lengths], dtype=torch.int32, device=DEV)
    q = synth.randn_bf16((B, Hq, 128), 1810, DEV)
    qs = synth.randn_bf16((B, Hq, 128), 1811, DEV)
    kv_new = synth.randn_bf16((B, Hkv, 2, 128), 1812, DEV)
    copy = hs.kv_to_fp8(kv, n_kv=cap)                      # scales from the cache before the step
    _, exps, _ = oracle_quantise(kv, cap)
    _, _, idx = hs.decode_step(q, kv_new, kv, seq, cap, top_k=k, window=W)
    hs.kv_to_fp8(kv, seq_lens=seq, out=copy)               # the appended rows
    o8 = hs.sparse_attn_reuse(qs, kv, idx, top_k=k, window=W, seq_lens=seq, kv_fp8=copy)
    torch.cuda.synchronize()
    # the oracle's quantisation of the cache after the append, with the scales of the cache before it
    kv_host = kv.clone()
    for b, L in enumerate(lengths):
        kv_host[b, :, L] = kv_new[b]
    _, _, deq = oracle_quantise(kv_host, cap, exps)
    idx_np = idx.cpu().numpy()
    stats = OutStats()
    for b, L in enumerate(lengths):
        ref, _ = orc.sparse_attention_rows(f32(qs[b])[None], deq[b, :, :, 0], deq[b, :, :, 1], idx_np[b][None],
                                           np.array([L]), W, orc.default_scale(128))
        stats.add(f32(o8[b]), ref[0])
    stats.check("fp8 sparse decode o")


def test_fp8_sparse_prefill32k_full_size():
    w = synth.WORKLOADS["prefill32k"]
    print("[case] fp8 sparse layer at the 32K workload", flush=True)
    case = synth.make_prefill_case(w, DEV, sparse_layers=1)
    q, kv, qs = case["q_full"], case["kv"], case["q_sparse"][0]
    _, _, idx = hs.full_attn_select(q, kv, w.n_kv, top_k=w.top_k, window=w.window, with_lse=False)
    copy = hs.kv_to_fp8(kv, n_kv=w.n_kv)
    o8 = hs.sparse_attn_reuse(qs, kv, idx, top_k=w.top_k, window=w.window, n_kv=w.n_kv, kv_fp8=copy)
    torch.cuda.synchronize()
    _, _, deq8 = oracle_quantise(kv, w.n_kv)
    deq = deq8[0]
    rows = sample_rows(w.n_q, w.n_kv, w.top_k, w.window, case["needles"][1], 4)
    pos = orc.query_positions(w.n_q, w.n_kv)[rows]
    ref, _ = orc.sparse_attention_rows(f32(qs[0])[rows], deq[:, :, 0], deq[:, :, 1], idx[0].cpu().numpy()[rows], pos,
                                       w.window, orc.default_scale(128))
    stats = OutStats()
    stats.add(f32(o8[0])[rows], ref)
    stats.check("fp8 sparse prefill32k o")


def test_fp8_decode_full_layer():
    """hs_decode_step reading the FP8 copy: the new token is quantised into
    the copy with the stored scales (byte-exact with the oracle's quantiser),
    and the full layer, its selection and the sparse layers over the copy
    match the oracle's decode step on the oracle's dequantised cache. The
    bf16 cache is left unchanged."""
    lengths = [300, 1200, 5000, 64, 2]
    B, Hq, Hkv, k, W, steps = len(lengths), 32, 4, 256, 64, 2
    print(f"[case] fp8 decode full layer lengths={lengths}", flush=True)
    cap = max(lengths) + steps
    kv = torch.zeros((B, Hkv, cap, 2, 128), dtype=torch.bfloat16, device=DEV)
    for b, L in enumerate(lengths):
        kv[b, :, :L] = synth.randn_bf16((Hkv, L, 2, 128), 1900 + b, DEV)
    kv_before = kv.clone()
    copy = hs.kv_to_fp8(kv, n_kv=cap)
    _, exps, deq = oracle_quantise(kv, cap)
    scale = orc.default_scale(128)
    full, sparse = OutStats(), OutStats()
    for s in range(steps):
        cur = [L + s + 1 for L in lengths]
        seq = torch.tensor(cur, dtype=torch.int32, device=DEV)
        q = synth.randn_bf16((B, Hq, 128), 1910 + s, DEV)
        qs = [synth.randn_bf16((B, Hq, 128), 1920 + 4 * s + i, DEV) for i in range(2)]
        kv_new = synth.randn_bf16((B, Hkv, 2, 128), 1930 + s, DEV)
        o, lse, idx = hs.decode_step(q, kv_new, kv, seq, cap, top_k=k, window=W, kv_fp8=copy)
        osp = [hs.sparse_attn_reuse(x, kv, idx, top_k=k, window=W, seq_lens=seq, kv_fp8=copy) for x in qs]
        torch.cuda.synchronize()
        codes, _ = split_copy(copy, B, Hkv, cap)
        idx_np = idx.cpu().numpy()
        for b in range(B):
            p = cur[b] - 1
            new_deq = np.zeros((Hkv, 2, 128))
            for g in range(Hkv):
                for h2 in range(2):
                    want, new_deq[g, h2] = orc.quantize_fp8(kv_new[b, g, h2].double().cpu().numpy(),
                                                            int(exps[b, g, h2]))
                    assert np.array_equal(codes[b, g, p, h2].cpu().numpy(), want), (s, b, g, h2)
            Kd, Vd = deq[b, :, :, 0], deq[b, :, :, 1]
            ref = orc.decode_step(f32(q[b]), [], new_deq, Kd, Vd, cur[b], k, W, scale)
            full.add(f32(o[b]), ref["o_full"])
            assert np.abs(lse[b].cpu().numpy() - ref["lse_full"]).max() <= 1e-3, (s, b)
            for g in range(Hkv):
                check_idx_row(idx_np[b, g], ref["idx"][g], ref["sigma"][g], ref["tau"][g], p, W, k,
                              where=f"step{s} b{b} g{g}")
            for x, osx in zip(qs, osp):
                r, _ = orc.sparse_attention_rows(f32(x[b])[None], Kd, Vd, idx_np[b][None], np.array([p]), W, scale)
                sparse.add(f32(osx[b]), r[0])
        print(f"[case] fp8 decode step {s} checked", flush=True)
    full.check("fp8 decode full o")
    sparse.check("fp8 decode sparse o")
    assert torch.equal(kv, kv_before)


@pytest.mark.timeout(600)
def test_fp8_decode_full_layer_decode64_sequences():
    """The FP8 full layer at the batched decode workload (64 sequences of
    64K-256K tokens): one step, three sequences checked against the oracle on
    its own dequantised cache, every index row checked for structure."""
    from parity import check_idx_structure
    w = synth.WORKLOADS["decode64"]
    lengths = synth.decode_lengths(w)
    print(f"[case] fp8 decode full layer at decode64 (sum of lengths {sum(lengths)})", flush=True)
    case = synth.make_decode_case(w, DEV, lengths, 1)
    kv, st = case["kv"], case["steps"][0]
    cap = kv.shape[2]
    copy = hs.kv_to_fp8(kv, n_kv=cap)
    seq = torch.tensor([L + 1 for L in lengths], dtype=torch.int32, device=DEV)
    o, lse, idx = hs.decode_step(st["q_full"], st["kv_new"], kv, seq, cap, top_k=w.top_k, window=w.window,
                                 kv_fp8=copy)
    torch.cuda.synchronize()
    check_idx_structure(idx, seq.long() - 1, w.window, w.top_k)
    order = np.argsort(lengths)
    scale = orc.default_scale(128)
    full = OutStats()
    for b in (int(order[0]), int(order[32]), int(order[-1])):
        L = lengths[b]
        # rows [0, L] (row L still zero in the bf16 cache: the scales are those of rows [0, L))
        _, exps, deq = oracle_quantise(kv[b:b + 1, :, :L + 1].contiguous(), L + 1)
        new_deq = np.zeros((w.Hkv, 2, 128))
        for g in range(w.Hkv):
            for h2 in range(2):
                new_deq[g, h2] = orc.quantize_fp8(st["kv_new"][b, g, h2].double().cpu().numpy(), int(exps[0, g, h2]))[1]
        ref = orc.decode_step(f32(st["q_full"][b]), [], new_deq, deq[0, :, :, 0], deq[0, :, :, 1], L + 1, w.top_k,
                              w.window, scale)
        full.add(f32(o[b]), ref["o_full"])
        for g in range(w.Hkv):
            check_idx_row(idx[b, g].cpu().numpy(), ref["idx"][g], ref["sigma"][g], ref["tau"][g], L, w.window,
                          w.top_k, where=f"b{b} g{g}")
        print(f"[case] sequence {b} (length {L}) checked", flush=True)
    full.check("fp8 decode64 full o")
