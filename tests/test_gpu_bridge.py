"""KV Bridging on the GPU against the oracle: the cache rows the bridge
writes must equal the oracle's projection rounded to bf16 (except a few
values whose exact projection lies next to a rounding boundary, which may
round to the neighbouring bf16 value), rows outside the chunk must stay
untouched, strided caches and the decode form (kv_new as a one-row cache)
must work, and a prefill chunk whose whole cache comes from the bridge must
give the full layer, its selection and a sparse layer within the usual
acceptance rules of the oracle run on the oracle's own bridged cache."""
import math

import numpy as np
import pytest
import torch

import oracle as orc
import token_level_sparse_hs_amd as hs
from token_level_sparse_hs_amd import synth
from parity import check_prefill, OutStats, f32
from test_gpu_layouts import relayout

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D_MODEL = 2048


def bridge_inputs(B, n, Hkv, d_model, seed):
    h = synth.randn_bf16((B, n, d_model), seed, DEV)
    w = (synth.randn_bf16((Hkv, 2, 128, d_model), seed + 1, DEV).float() / math.sqrt(d_model)).to(torch.bfloat16)
    return h, w


def oracle_rows(h, w, b):
    """The oracle's bf16 K, V rows [Hkv][n][128] of batch entry b, the
    unrounded float64 projection, and the sums of |terms| of every dot
    product (the same projection of |h| and |w|), which bound the error of
    any fp32 accumulation order."""
    K, V = orc.kv_bridge(f32(h[b]), f32(w))
    aK, aV = orc.kv_bridge(np.abs(f32(h[b])), np.abs(f32(w)))
    return orc.bf16_round(K), orc.bf16_round(V), K, V, aK, aV


def check_rows(got, want_bf16, exact, abs_terms, d_model):
    """got (bf16 from the GPU) against the oracle: at most 1% of the values
    differ from the oracle's rounding of the exact projection, each value
    lies within one bf16 ulp plus the fp32 accumulation bound
    d_model * 2^-24 * sum|terms| of the exact projection, and the north-star
    tolerances hold against the exact values."""
    got = np.asarray(got, np.float64)
    diff = got != want_bf16
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(got), np.abs(exact)) + 1e-30)[1] - 8)
    bound = ulp + d_model * 2.0 ** -24 * abs_terms
    assert np.all(np.abs(got - exact) <= bound), "a value beyond one ulp plus the fp32 accumulation bound"
    assert diff.mean() <= 0.01, f"{diff.mean():.4f} of the values differ from the oracle's rounding"
    st = OutStats()
    st.add(got, exact)
    st.check("bridged rows")
    return int(diff.sum())


@pytest.mark.parametrize("B,n_q,n_kv,Hkv,d_model", [(2, 300, 500, 4, D_MODEL), (1, 128, 128, 1, 64),
                                                     (1, 77, 900, 2, 192)])
def test_bridge_rows_match_oracle(B, n_q, n_kv, Hkv, d_model):
    print(f"[case] bridge B={B} n_q={n_q} n_kv={n_kv} Hkv={Hkv} d_model={d_model}", flush=True)
    cap = n_kv + 20
    h, w = bridge_inputs(B, n_q, Hkv, d_model, 2100 + n_q)
    kv = torch.full((B, Hkv, cap, 2, 128), 7.0, dtype=torch.bfloat16, device=DEV)  # sentinel rows
    hs.kv_bridge(h, w, kv, n_kv)
    torch.cuda.synchronize()
    row0 = n_kv - n_q
    for b in range(B):
        Kb, Vb, K, V, aK, aV = oracle_rows(h, w, b)
        nd = check_rows(kv[b, :, row0:n_kv, 0].double().cpu().numpy(), Kb, K, aK, d_model)
        nd += check_rows(kv[b, :, row0:n_kv, 1].double().cpu().numpy(), Vb, V, aV, d_model)
        print(f"[case] b{b}: {nd} of {2 * K.size} values on the other side of a rounding boundary", flush=True)
    untouched = torch.cat([kv[:, :, :row0], kv[:, :, n_kv:]], dim=2)
    assert bool((untouched == 7.0).all()), "rows outside the chunk were written"


def test_bridge_strided_cache_and_decode_form():
    """A K-region-then-V-region cache with padded rows gets the same rows as
    the default layout; kv_new [B][Hkv][2][128] as a one-row cache gets the
    decode token's rows."""
    B, n_q, n_kv, Hkv = 2, 100, 260, 4
    print("[case] bridge strided cache + decode form", flush=True)
    h, w = bridge_inputs(B, n_q, Hkv, D_MODEL, 2200)
    kv = torch.zeros((B, Hkv, n_kv, 2, 128), dtype=torch.bfloat16, device=DEV)
    hs.kv_bridge(h, w, kv, n_kv)
    buf, strides = relayout(torch.zeros_like(kv), 24, True)
    hs.kv_bridge(h, w, buf, n_kv, kv_strides=strides, kv_heads=Hkv, kv_capacity=n_kv)
    torch.cuda.synchronize()
    sb, sh, st, voff = strides
    for b in range(B):
        for g in range(Hkv):
            base = b * sb + g * sh
            Krows = buf[base:base + n_kv * st].view(n_kv, st)[:, :128]
            Vrows = buf[voff + base:voff + base + n_kv * st].view(n_kv, st)[:, :128]
            assert torch.equal(Krows, kv[b, g, :, 0]) and torch.equal(Vrows, kv[b, g, :, 1]), (b, g)
    # decode form: one token per sequence into kv_new
    hd = h[:, -1:].contiguous()
    kv_new = torch.zeros((B, Hkv, 2, 128), dtype=torch.bfloat16, device=DEV)
    hs.kv_bridge(hd, w, kv_new.view(B, Hkv, 1, 2, 128), 1)
    torch.cuda.synchronize()
    assert torch.equal(kv_new, kv[:, :, n_kv - 1])


def test_bridged_prefill_matches_oracle():
    """Early-exit prefill of the cross-decoder: the whole cache of a chunk is
    bridged from hidden states, then the full layer selects and a sparse
    layer reuses it; the oracle runs the same layers on its own bridged
    (bf16-rounded) cache."""
    B, n, Hq, Hkv, k, W = 1, 1500, 32, 4, 128, 64
    print(f"[case] bridged prefill n={n} Hq={Hq} Hkv={Hkv} k={k} W={W}", flush=True)
    h, w = bridge_inputs(B, n, Hkv, D_MODEL, 2300)
    kv = torch.zeros((B, Hkv, n, 2, 128), dtype=torch.bfloat16, device=DEV)
    hs.kv_bridge(h, w, kv, n)
    q = synth.randn_bf16((B, n, Hq, 128), 2301, DEV)
    qs = synth.randn_bf16((B, n, Hq, 128), 2302, DEV)
    o, lse, idx = hs.full_attn_select(q, kv, n, top_k=k, window=W)
    osp = hs.sparse_attn_reuse(qs, kv, idx, top_k=k, window=W, n_kv=n)
    torch.cuda.synchronize()
    Kb, Vb = oracle_rows(h, w, 0)[:2]
    ref_kv = torch.zeros_like(kv)
    ref_kv[0, :, :, 0] = torch.from_numpy(Kb).to(torch.bfloat16).to(DEV)
    ref_kv[0, :, :, 1] = torch.from_numpy(Vb).to(torch.bfloat16).to(DEV)
    rows = [0, 63, 64, 191, 192, 500, 1000, 1499]
    res = check_prefill(q, ref_kv, n, k, W, o, lse, idx, rows=rows, q_sparse=[qs], o_sparse=[osp])
    print(f"[case] bridged prefill: swaps {res['swaps']}, full max-abs {res['full'].max_abs:.2e}", flush=True)
