"""Plain, slow CPU oracle for token-level hybrid sparse attention with KV Reuse.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this
module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark do. It shares no code with the HIP library.

Everything is evaluated in float64 with numpy. Inputs arrive as float32 arrays
that hold bf16-representable values (the caller widens bf16 exactly), so the
oracle sees the very numbers the GPU sees.

Sources (web pages; section names as printed on them):

[HS2-cs]  "HySparse2 od Xiaomi zkracuje zpracování dlouhého kontextu",
          section "Proč není nutné znovu zpracovat celý dlouhý vstup", the
          KV Reuse paragraph: the sparse layers of a hybrid block take over
          both the KV cache and the record of which tokens were selected from
          the full-attention layer before them; selection is per token, not
          per block; recent tokens are always included, so no separate
          sliding-window branch is needed and local and selected tokens share
          one cache.
[DAIR]    "DAIR.AI周报：HySparse2长上下文优化与SIFT代码Agent自改进", bullets
          "Two levels of KV sharing" (each sparse layer reuses the KV cache and
          selection indices of the preceding full-attention layer) and
          "Prefill exits early" (token-level selection; a forced window of
          recent tokens replaces the sliding-window branch).
[HS2-en]  "HySparse2 Cuts the Prefill Path for Tool-Using Agents", section
          "Tool Responses Turn Prefill Into the Bottleneck": prefill writes
          keys and values to the KV cache, which decoding then reuses.
[SSA-3.3] "Simplified Sparse Attention via Gist Tokens", section 3.3
          "Selective Unfolding and Hybrid Attention", paragraph "Grouped
          Unfolding for GQA": each query head takes its own top-k; a KV
          group unfolds the union of its heads' choices.
[SSA-3.6] "Simplified Sparse Attention via Gist Tokens", section 3.6 "Kernel
          Design": sparse kernels compute exact attention over the kept keys
          (only accumulation order may differ); softmax normalises over the
          key axis so attention does not depend on key order; split partials
          (m, l, acc) merge by the log-sum-exp correction.

Readings where the pages are silent (each one is listed with its reason in the
design notes of the repository):
  R1 selection score: sigma(t, g, j) = max over the query heads h of KV group g
     of the scaled logit scale * <q_h(t), k_g(j)>.
  R2 window: Win(p) = [max(0, p-W+1), p], the query's own position included.
  R3 candidates for top-k: C(p) = {j : 0 <= j <= p-W} (tokens older than the
     window); the attention budget is k + W.
  R4 fewer than k candidates: all of C(p) is taken, the rest padded with -1.
  R5 ties: lower token index first; -0.0 ranks as +0.0.
  R6 index rows are emitted in ascending order.
  R7 GQA: query head h reads KV head h // G, G = Hq / Hkv.
  R8 the selection decision is taken on float32 scores (float64 evaluation
     rounded once to float32), the precision the kernels decide in.
  R11 (optional, block-level selection, the ablation the pages compare
     token-level selection against): C(p) is cut into aligned blocks of 64
     tokens, a block scores the maximum sigma of its candidates, the top
     k / 64 blocks (ties: lower block first) are taken whole (the last block
     of C(p) may be partial), emitted ascending and padded with -1.
  R12 (optional, union of per-head top-k, the grouped-unfolding rule of
     [SSA-3.3]): each query head h of group g ranks C(p) by its own scaled
     logit and keeps its top k (rules R4, R5, R8 per head); the group's set
     is the union of the G head sets, emitted ascending in a row of G * k
     entries padded with -1.
  R13 KV Bridging: the cross-decoder's full-attention K and V rows of a token
     are linear projections of the self-decoder's hidden state of that token,
     K_g = h W_K,g and V_g = h W_V,g per KV head g, with no bias, norm or
     position rotation (the pages name the inputs and outputs only); the
     cache stores them in bf16, rounded to nearest even.
  R1' (optional score, score="prob"): the softmax-normalised group score
     max over h of (scale * <q_h(t), k_g(j)> - lse_h(t)), lse_h(t) the log
     of the softmax denominator of head h over keys 0..p, i.e. the log of the
     largest attention probability any head of the group gives token j.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "default_scale",
    "query_positions",
    "window_range",
    "candidate_count",
    "attention_over_set",
    "full_attention_rows",
    "selection_scores",
    "topk_select",
    "head_union_select",
    "full_attn_select_rows",
    "sparse_attention_rows",
    "decode_step",
    "lse_combine",
    "fp8_scale_exponent",
    "quantize_fp8",
    "block_select",
    "kv_bridge",
    "bf16_round",
]


def default_scale(head_dim: int) -> float:
    """Softmax scale 1/sqrt(d) of standard scaled dot-product attention."""
    return 1.0 / math.sqrt(head_dim)


def query_positions(n_q: int, n_kv: int) -> np.ndarray:
    """Absolute positions of the n_q newest tokens of an n_kv-token context.

    A prefill chunk appends its tokens at the end of the cache [HS2-en], so
    query row t sits at p = n_kv - n_q + t and sees keys 0..p (causal).
    """
    if n_q > n_kv:
        raise ValueError("n_q must not exceed n_kv")
    return np.arange(n_kv - n_q, n_kv, dtype=np.int64)


def window_range(p: int, window: int) -> range:
    """Forced recent window of position p (reading R2): [max(0,p-W+1), p]."""
    return range(max(0, p - window + 1), p + 1)


def candidate_count(p: int, window: int) -> int:
    """|C(p)|: tokens older than the window (reading R3)."""
    return max(0, p - window + 1)


def attention_over_set(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                       keys: np.ndarray, scale: float):
    """Exact softmax attention of the query vectors q [H][d] over key rows `keys`.

    Definition [SSA-3.6]: o = sum_j softmax_j(scale * q.k_j) v_j, evaluated in
    float64 with the row maximum subtracted before exponentiation. Returns
    (o [H][d], lse [H]) with lse = m + ln(sum exp(s - m)). `keys` is an index
    array or a slice (a contiguous range, taken as a view: callers may pass
    float64 caches to avoid per-call conversion of long contexts).
    """
    q = np.asarray(q, dtype=np.float64)
    Ks = np.asarray(K[keys], dtype=np.float64)          # [n][d]
    Vs = np.asarray(V[keys], dtype=np.float64)
    s = scale * (q @ Ks.T)                               # [H][n]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=1, keepdims=True)
    o = (w @ Vs) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def _check_gqa(q_heads: int, kv_heads: int) -> int:
    if kv_heads <= 0 or q_heads % kv_heads:
        raise ValueError("q_heads must be a positive multiple of kv_heads")
    return q_heads // kv_heads


def full_attention_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                        positions, scale: float):
    """Causal GQA attention for the given query rows of one sequence.

    q: [rows][Hq][d]; K, V: [Hkv][n][d]; positions: absolute position of each
    row. Head h attends to keys 0..p of KV head h // G (reading R7). Returns
    (o [rows][Hq][d], lse [rows][Hq]) in float64.
    """
    rows, Hq, d = q.shape
    Hkv = K.shape[0]
    G = _check_gqa(Hq, Hkv)
    o = np.zeros((rows, Hq, d), dtype=np.float64)
    lse = np.zeros((rows, Hq), dtype=np.float64)
    for r in range(rows):
        p = int(positions[r])
        keys = slice(0, p + 1)
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            o[r, hs], lse[r, hs] = attention_over_set(q[r, hs], K[g], V[g], keys, scale)
    return o, lse


def selection_scores(q_group: np.ndarray, Kg: np.ndarray, p: int, window: int,
                     scale: float, lse_group=None) -> np.ndarray:
    """sigma_j for j in C(p), for one query row and one KV group (readings R1, R3).

    q_group: [G][d] (the group's query heads); Kg: [n][d]. Returns float64
    scores of length |C(p)|; position j of the result is token j. With
    lse_group ([G], each head's log-sum-exp over keys 0..p) the score is the
    softmax-normalised one of reading R1': each head's logit minus its
    log-sum-exp, then the maximum over the group.
    """
    c = candidate_count(p, window)
    if c == 0:
        return np.zeros(0, dtype=np.float64)
    s = scale * (np.asarray(q_group, np.float64) @ np.asarray(Kg[:c], np.float64).T)
    if lse_group is not None:
        s = s - np.asarray(lse_group, np.float64)[:, None]
    return s.max(axis=0)


def topk_select(sigma: np.ndarray, k: int):
    """Token-level top-k over the candidate scores of one (row, group).

    Order: score descending, token index ascending on ties (R5), decided on the
    float32 rounding of the scores (R8). Returns (idx, tau) where idx has
    length k, holds the chosen token indices ascending (R6) and is padded with
    -1 (R4), and tau is the float64 score of the k-th ranked candidate (or
    -inf when every candidate is taken).
    """
    n = sigma.shape[0]
    out = np.full(k, -1, dtype=np.int64)
    if k == 0:
        return out, -math.inf
    if n <= k:
        out[:n] = np.arange(n)
        return out, -math.inf
    s32 = sigma.astype(np.float32).astype(np.float64)
    s32 = np.where(s32 == 0.0, 0.0, s32)                # -0.0 ranks as +0.0
    order = np.lexsort((np.arange(n), -s32))            # primary: -score, then j
    chosen = order[:k]
    out[:] = np.sort(chosen)
    return out, float(sigma[chosen[-1]])


def block_select(sigma: np.ndarray, k: int, block: int = 64):
    """Block-level selection (reading R11) over the candidate scores of one
    (row, group): blocks [block*b, block*b + block) of C(p), block score =
    the largest member score, the top k // block blocks by (score desc, block
    index asc) decided on float32 scores (R8), expanded to their tokens.
    Returns (idx of length k, ascending, -1 padded; tau = the float64 score of
    the last block taken, or -inf when every block is taken)."""
    n = sigma.shape[0]
    out = np.full(k, -1, dtype=np.int64)
    nb = k // block
    if nb == 0 or n == 0:
        return out, -math.inf
    nblk = (n + block - 1) // block
    bs = np.array([sigma[b * block:(b + 1) * block].max() for b in range(nblk)])
    if nblk <= nb:
        chosen, tau = np.arange(nblk), -math.inf
    else:
        b32 = bs.astype(np.float32).astype(np.float64)
        b32 = np.where(b32 == 0.0, 0.0, b32)
        order = np.lexsort((np.arange(nblk), -b32))
        chosen = np.sort(order[:nb])
        tau = float(bs[order[nb - 1]])
    toks = np.concatenate([np.arange(b * block, min((b + 1) * block, n)) for b in chosen])
    out[:len(toks)] = toks
    return out, tau


def head_union_select(q_group: np.ndarray, Kg: np.ndarray, p: int, window: int, scale: float, k: int):
    """Union of per-head top-k sets for one (row, group) (reading R12,
    [SSA-3.3] "Grouped Unfolding for GQA"): every head's own token-level
    top-k over C(p), then the set union. Returns (idx of length G*k,
    ascending, -1 padded; list of the G heads' (sigma_h, tau_h))."""
    G = q_group.shape[0]
    out = np.full(G * k, -1, dtype=np.int64)
    chosen, heads = set(), []
    for h in range(G):
        s_h = selection_scores(q_group[h:h + 1], Kg, p, window, scale)
        idx_h, tau_h = topk_select(s_h, k)
        chosen.update(int(j) for j in idx_h if j >= 0)
        heads.append((s_h, tau_h))
    u = sorted(chosen)
    out[:len(u)] = u
    return out, heads


def full_attn_select_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                          positions, k: int, window: int, scale: float, score: str = "logit",
                          blocks: bool = False, union: bool = False):
    """The full-attention layer of a hybrid block for the given query rows.

    It computes causal GQA attention and, per (row, KV group), the top-k token
    indices that the following sparse layers reuse [HS2-cs], [DAIR].
    score: "logit" (reading R1) or "prob" (reading R1', which needs this
    layer's lse first); blocks: block-level selection (reading R11) instead of
    token-level. Returns dict with o [rows][Hq][d], lse [rows][Hq],
    idx [rows][Hkv][k] (int64), tau [rows][Hkv], sigma (list of per-(row,
    group) float64 arrays). union: the union of per-head top-k sets
    (reading R12, logit score only); idx is then [rows][Hkv][G*k] and
    "heads" holds, per (row, group), the G heads' (sigma_h, tau_h).
    """
    if score not in ("logit", "prob"):
        raise ValueError("score must be 'logit' or 'prob'")
    rows, Hq, d = q.shape
    Hkv = K.shape[0]
    G = _check_gqa(Hq, Hkv)
    o, lse = full_attention_rows(q, K, V, positions, scale)
    if union:
        if score != "logit" or blocks:
            raise ValueError("the per-head union uses token-level logit scores")
        idx = np.full((rows, Hkv, G * k), -1, dtype=np.int64)
        heads = []
        for r in range(rows):
            row_heads = []
            for g in range(Hkv):
                idx[r, g], hh = head_union_select(q[r, g * G:(g + 1) * G], K[g], int(positions[r]), window,
                                                  scale, k)
                row_heads.append(hh)
            heads.append(row_heads)
        return {"o": o, "lse": lse, "idx": idx, "heads": heads}
    idx = np.full((rows, Hkv, k), -1, dtype=np.int64)
    tau = np.full((rows, Hkv), -math.inf)
    sig = []
    for r in range(rows):
        p = int(positions[r])
        row_sig = []
        for g in range(Hkv):
            lg = lse[r, g * G:(g + 1) * G] if score == "prob" else None
            s = selection_scores(q[r, g * G:(g + 1) * G], K[g], p, window, scale, lg)
            idx[r, g], tau[r, g] = block_select(s, k) if blocks else topk_select(s, k)
            row_sig.append(s)
        sig.append(row_sig)
    return {"o": o, "lse": lse, "idx": idx, "tau": tau, "sigma": sig}


def sparse_attention_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                          idx: np.ndarray, positions, window: int, scale: float):
    """A sparse-reuse layer: attention over (selected tokens) U (forced window).

    q: [rows][Hq][d] is this layer's own query; K, V and idx [rows][Hkv][k]
    are the full layer's cache and selection, reused unchanged [HS2-cs],
    [DAIR]. Entries of idx equal to -1 are padding. Returns (o, lse).
    """
    rows, Hq, d = q.shape
    Hkv = K.shape[0]
    G = _check_gqa(Hq, Hkv)
    o = np.zeros((rows, Hq, d), dtype=np.float64)
    lse = np.zeros((rows, Hq), dtype=np.float64)
    for r in range(rows):
        p = int(positions[r])
        win = np.array(window_range(p, window), dtype=np.int64)
        for g in range(Hkv):
            sel = idx[r, g]
            sel = sel[sel >= 0]
            keys = np.union1d(sel, win)
            hs = slice(g * G, (g + 1) * G)
            o[r, hs], lse[r, hs] = attention_over_set(q[r, hs], K[g], V[g], keys, scale)
    return o, lse


def decode_step(q_full: np.ndarray, q_sparse: list, kv_new: np.ndarray,
                K: np.ndarray, V: np.ndarray, length: int, k: int,
                window: int, scale: float, score: str = "logit", blocks: bool = False, union: bool = False):
    """One decode step of one sequence through a hybrid block.

    The new token's key/value row is written at slot length-1 of the cache
    first [HS2-en]; then the full layer attends over [0, length) and selects
    once; every sparse layer reuses that one selection and the same cache
    [HS2-cs], [DAIR]. q_full: [Hq][d]; q_sparse: list of [Hq][d]; kv_new:
    [Hkv][2][d]; K, V: [Hkv][cap][d] float arrays, modified in place.
    Returns dict(o_full, lse_full, idx [Hkv][k], tau, sigma, o_sparse list);
    with union (reading R12) idx is [Hkv][G*k] and "heads" replaces tau and
    sigma.
    """
    p = length - 1
    K[:, p] = kv_new[:, 0]
    V[:, p] = kv_new[:, 1]
    pos = np.array([p])
    res = full_attn_select_rows(q_full[None], K, V, pos, k, window, scale, score, blocks, union)
    outs = []
    for qs in q_sparse:
        o, _ = sparse_attention_rows(qs[None], K, V, res["idx"], pos, window, scale)
        outs.append(o[0])
    out = {"o_full": res["o"][0], "lse_full": res["lse"][0], "idx": res["idx"][0], "o_sparse": outs}
    if union:
        out["heads"] = res["heads"][0]
    else:
        out["tau"], out["sigma"] = res["tau"][0], res["sigma"][0]
    return out


def lse_combine(parts):
    """Merge attention partials over disjoint key subsets [SSA-3.6].

    parts: list of (o [H][d], lse [H]) each normalised over its own subset.
    The merged output weights each part by exp(lse_i - lse) with
    lse = log(sum_i exp(lse_i)).
    """
    lses = np.stack([np.asarray(l, np.float64) for _, l in parts])      # [P][H]
    m = lses.max(axis=0)
    w = np.exp(lses - m)
    tot = w.sum(axis=0)
    o = sum(w[i][:, None] * np.asarray(parts[i][0], np.float64) for i in range(len(parts)))
    return o / tot[:, None], m + np.log(tot)


# ---------------------------------------------------------------- FP8 cache

E4M3_MAX = 448.0


def fp8_scale_exponent(amax: float) -> int:
    """Smallest e with amax <= 448 * 2^e (e = 0 for an all-zero head): the
    power-of-two scale of one KV head's K (or V) rows in the FP8 cache, so
    that every value divided by 2^e lies within the e4m3 range and the
    dequantised values (e4m3 times 2^e) are exactly representable in bf16."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    e = math.frexp(amax)[1] - 9
    while amax > E4M3_MAX * 2.0 ** e:
        e += 1
    while amax <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return e


def quantize_fp8(x: np.ndarray, e: int):
    """e4m3 codes of x / 2^e, clamped to +-448, rounded to nearest (ties to
    even) by torch's float8_e4m3fn conversion; returns (codes as uint8,
    dequantised float64 values codes * 2^e)."""
    import torch
    y = torch.from_numpy(np.asarray(x, np.float64) * 2.0 ** (-e)).clamp(-E4M3_MAX, E4M3_MAX)
    q = y.to(torch.float32).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy(), q.to(torch.float64).numpy() * 2.0 ** e


# ---------------------------------------------------------------- KV Bridging

def kv_bridge(h: np.ndarray, w_kv: np.ndarray):
    """KV Bridging (reading R13), [HS2-cs] "Proc neni nutne znovu zpracovat
    cely dlouhy vstup" and [DAIR] "Two levels of KV sharing": the
    full-attention layers of the cross-decoder take their keys and values from
    the hidden states of the self-decoder, so prefill can stop after the
    self-decoder ([DAIR] "Prefill exits early").

    h: [n][d_model] hidden states of n tokens; w_kv: [Hkv][2][d][d_model], the
    projection rows (index 0: keys, 1: values) of each KV head, laid out as a
    linear layer's weight (one row per output feature). Returns (K, V), each
    [Hkv][n][d] float64: K[g][t][e] = sum_i h[t][i] * w_kv[g][0][e][i],
    V[g][t][e] = sum_i h[t][i] * w_kv[g][1][e][i]."""
    h = np.asarray(h, np.float64)
    w = np.asarray(w_kv, np.float64)
    Hkv, two, d, d_model = w.shape
    if two != 2 or h.shape[1] != d_model:
        raise ValueError("w_kv must be [Hkv][2][d][d_model] with d_model = h.shape[1]")
    K = np.stack([h @ w[g, 0].T for g in range(Hkv)])
    V = np.stack([h @ w[g, 1].T for g in range(Hkv)])
    return K, V


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even to bfloat16 precision (8 significant bits), as
    float64 values: the precision the cache stores. Finite inputs within the
    normal range of bf16."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                    # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)  # rint: ties to even
