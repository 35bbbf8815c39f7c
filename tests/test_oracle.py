"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test names what pins it: a library routine on a special case
(torch scaled_dot_product_attention in float64), a closed form, brute force on
tiny inputs, or an invariant stated by the pages (order independence of
softmax over keys, exact log-sum-exp merging of split partials, reuse of one
selection by every sparse layer). Together they are chosen so that a dropped
scale, a wrong causal offset, an off-by-one window or candidate boundary, a
reversed tie rule, a min-for-max score or a wrong GQA head map each fail at
least one test.
"""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle as orc


def bf16_exact(shape, rng, scale=1.0):
    """float32 array of bf16-representable N(0, scale^2) values."""
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * scale)
    return x.to(torch.bfloat16).float().numpy()


def sdpa_rows(q, K, V, positions, n_kv, band=None):
    """torch SDPA (float64, enable_gqa) for query rows at `positions`.

    band=None: causal mask j <= p. band=W: banded mask p-W < j <= p.
    q: [rows][Hq][d]; K, V: [Hkv][n][d].
    """
    rows = q.shape[0]
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2))).double()[None]  # [1][Hq][rows][d]
    kt = torch.from_numpy(np.ascontiguousarray(K[:, :n_kv])).double()[None]
    vt = torch.from_numpy(np.ascontiguousarray(V[:, :n_kv])).double()[None]
    j = torch.arange(n_kv)[None, :]
    p = torch.as_tensor(np.asarray(positions))[:, None]
    mask = j <= p
    if band is not None:
        mask &= j > p - band
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, enable_gqa=True)
    return out[0].transpose(0, 1).numpy()


# ---------------------------------------------------------------- full attention

@pytest.mark.parametrize("Hq,Hkv,n_q,n_kv,d", [(4, 1, 40, 40, 128), (8, 2, 17, 53, 128), (6, 3, 9, 9, 16)])
def test_full_attention_matches_sdpa(Hq, Hkv, n_q, n_kv, d):
    """Library routine pin: causal GQA attention, including a chunk whose rows
    sit at the end of a longer cache, against torch SDPA in float64."""
    rng = np.random.default_rng(1 + n_q + Hq)
    q = bf16_exact((n_q, Hq, d), rng)
    K = bf16_exact((Hkv, n_kv, d), rng)
    V = bf16_exact((Hkv, n_kv, d), rng)
    pos = orc.query_positions(n_q, n_kv)
    o, _ = orc.full_attention_rows(q, K, V, pos, orc.default_scale(d))
    ref = sdpa_rows(q, K, V, pos, n_kv)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_query_positions_chunk_offset():
    """A chunk of n_q new tokens occupies the last n_q cache slots."""
    assert list(orc.query_positions(3, 10)) == [7, 8, 9]
    assert list(orc.query_positions(4, 4)) == [0, 1, 2, 3]
    with pytest.raises(ValueError):
        orc.query_positions(5, 4)


def test_softmax_rows_sum_to_one():
    """Invariant: with V = one-hot rows the output is the attention weight
    vector itself; it must be >= 0, zero beyond the causal limit, sum to 1."""
    rng = np.random.default_rng(7)
    d, n = 128, 100
    q = bf16_exact((n, 4, d), rng, 2.0)
    K = bf16_exact((1, n, d), rng)
    V = np.eye(n, d, dtype=np.float32)[None]          # v_j = e_j
    pos = orc.query_positions(n, n)
    o, _ = orc.full_attention_rows(q, K, V, pos, orc.default_scale(d))
    sums = o.sum(axis=2)
    assert np.all(o >= 0)
    np.testing.assert_allclose(sums, 1.0, atol=1e-5)
    for t in range(n):
        assert np.all(o[t, :, t + 1:] == 0)


def test_lse_closed_form():
    """Closed form: with q = a*e_0 and k_0 = c*e_0, k_j = 0 otherwise, the
    logits are (scale*a*c, 0, ..., 0), so lse = log(exp(scale*a*c) + p) and
    o = (exp(x) v_0 + sum_{j>=1} v_j) / (exp(x) + p)."""
    d, n = 128, 11
    a, c = 3.0, 2.0
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = a
    K = np.zeros((1, n, d), np.float32)
    K[0, 0, 0] = c
    rng = np.random.default_rng(3)
    V = bf16_exact((1, n, d), rng)
    p = n - 1
    o, lse = orc.full_attention_rows(q, K, V, [p], orc.default_scale(d))
    x = a * c / math.sqrt(d)
    assert abs(lse[0, 0] - math.log(math.exp(x) + p)) < 1e-12
    V64 = V.astype(np.float64)
    want = (math.exp(x) * V64[0, 0] + V64[0, 1:].sum(0)) / (math.exp(x) + p)
    np.testing.assert_allclose(o[0, 0], want, atol=1e-12)


def test_zero_query_is_mean_of_values():
    """Closed form: q = 0 gives uniform weights, so o = mean of v over the set,
    for full attention and for a sparse set."""
    rng = np.random.default_rng(5)
    d, n = 128, 30
    q = np.zeros((1, 2, d), np.float32)
    K = bf16_exact((1, n, d), rng)
    V = bf16_exact((1, n, d), rng)
    o, lse = orc.full_attention_rows(q, K, V, [n - 1], 0.1)
    np.testing.assert_allclose(o[0, 0], V[0].astype(np.float64).mean(0), atol=1e-12)
    assert abs(lse[0, 0] - math.log(n)) < 1e-12
    idx = np.array([[[2, 5, -1, -1]]])
    o2, _ = orc.sparse_attention_rows(q, K, V, idx, [n - 1], 3, 0.1)
    want = V[0, [2, 5, 27, 28, 29]].astype(np.float64).mean(0)
    np.testing.assert_allclose(o2[0, 1], want, atol=1e-12)


# ------------------------------------------------------------------ selection

def _beats(sa, a, sb, b):
    return sa > sb or (sa == sb and a < b)


@pytest.mark.parametrize("seed", range(6))
def test_topk_defining_property_and_brute_force(seed):
    """Brute force: on tiny inputs, enumerate every k-subset; exactly one has
    every member beating every non-member under (score desc, index asc), and
    topk_select must return it. Scores are drawn from a small grid so that
    exact ties occur."""
    rng = np.random.default_rng(seed)
    n = 9
    sig = rng.integers(-3, 4, size=n).astype(np.float64) / 4
    for k in range(0, n + 2):
        idx, _ = orc.topk_select(sig, k)
        got = set(int(i) for i in idx if i >= 0)
        if k >= n:
            assert got == set(range(n))
            continue
        winners = []
        for sub in itertools.combinations(range(n), k):
            s = set(sub)
            if all(_beats(sig[i], i, sig[o], o) for i in s for o in range(n) if o not in s):
                winners.append(s)
        assert len(winners) == 1
        assert got == winners[0]
        assert list(idx) == sorted(idx)


def test_topk_negative_zero_ties_by_index():
    """-0.0 and +0.0 are the same score, so the lower index wins the tie."""
    sig = np.array([-1.0, -0.0, 0.0, -0.0, 0.0, -2.0])
    idx, _ = orc.topk_select(sig, 2)
    assert list(idx) == [1, 2]
    idx, _ = orc.topk_select(sig, 3)
    assert list(idx) == [1, 2, 3]


def test_topk_padding_and_count():
    """Fewer candidates than k: every candidate is taken, the rest is -1."""
    idx, tau = orc.topk_select(np.array([0.5, 0.1, 0.9]), 5)
    assert list(idx) == [0, 1, 2, -1, -1] and tau == -math.inf
    idx, _ = orc.topk_select(np.zeros(0), 4)
    assert list(idx) == [-1] * 4


def test_selection_is_group_max_not_mean():
    """Constructed case where the max over the group's heads and the mean
    disagree: head A scores (x=5, y=4), head B (x=-5, y=3). The group max
    ranks x first (5 > 4); a mean would rank y first (3.5 > 0)."""
    d = 128
    scale = 1.0
    K = np.zeros((1, 10, d), np.float32)
    K[0, 0, 0] = 1.0     # key x at position 0
    K[0, 1, 1] = 1.0     # key y at position 1
    q = np.zeros((2, d), np.float32)
    q[0, 0], q[0, 1] = 5.0, 4.0
    q[1, 0], q[1, 1] = -5.0, 3.0
    sig = orc.selection_scores(q, K[0], p=9, window=2, scale=scale)
    assert sig.shape == (8,)
    assert sig[0] == 5.0 and sig[1] == 4.0
    idx, _ = orc.topk_select(sig, 1)
    assert list(idx) == [0]


def test_candidates_exclude_window():
    """Reading R3: candidates are j <= p-W, i.e. exactly p-W+1 of them."""
    rng = np.random.default_rng(11)
    d = 128
    K = bf16_exact((1, 50, d), rng)
    q = bf16_exact((4, d), rng)
    for p, W in [(49, 8), (7, 8), (8, 8), (20, 1)]:
        s = orc.selection_scores(q, K[0], p, W, 0.1)
        assert s.shape[0] == max(0, p - W + 1) == orc.candidate_count(p, W)


def test_head_permutation_invariance():
    """Permuting heads inside a group leaves sigma (a max) unchanged."""
    rng = np.random.default_rng(12)
    d = 128
    K = bf16_exact((1, 40, d), rng)
    q = bf16_exact((8, d), rng)
    s1 = orc.selection_scores(q, K[0], 39, 4, 0.1)
    s2 = orc.selection_scores(q[rng.permutation(8)], K[0], 39, 4, 0.1)
    assert np.array_equal(s1, s2)


def test_nested_selection():
    """Superset property of growing budgets: I_k is contained in I_{k+1}."""
    rng = np.random.default_rng(13)
    d = 128
    K = bf16_exact((1, 64, d), rng)
    q = bf16_exact((4, d), rng)
    s = orc.selection_scores(q, K[0], 63, 4, orc.default_scale(d))
    prev = set()
    for k in range(0, 62):
        cur = set(int(i) for i in orc.topk_select(s, k)[0] if i >= 0)
        assert prev <= cur and len(cur) == min(k, s.shape[0])
        prev = cur


def test_duplicate_keys_pick_lower_index():
    """Exact ties from identical key rows resolve to the lower index."""
    rng = np.random.default_rng(14)
    d = 128
    K = bf16_exact((1, 40, d), rng)
    q = bf16_exact((4, d), rng)
    hot = (q.sum(0) / np.linalg.norm(q.sum(0)) * 16).astype(np.float32)
    hot = torch.from_numpy(hot).to(torch.bfloat16).float().numpy()
    K[0, 9] = hot
    K[0, 3] = hot
    K[0, 20] = hot
    s = orc.selection_scores(q, K[0], 39, 4, orc.default_scale(d))
    assert s[3] == s[9] == s[20] == s.max()
    assert list(orc.topk_select(s, 1)[0]) == [3]
    assert list(orc.topk_select(s, 2)[0]) == [3, 9]


# --------------------------------------------------------------- sparse layers

@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (8, 2)])
def test_sparse_equals_full_when_budget_covers_context(Hq, Hkv):
    """Pin: with k + W >= p + 1 every earlier token is kept, so the sparse
    layer equals causal full attention (itself pinned to SDPA). The budget is
    chosen so that k + W = n exactly, which makes an off-by-one in the
    candidate or window boundary drop a token on the last row."""
    rng = np.random.default_rng(21)
    d, n, W = 128, 48, 5
    k = n - W
    q0 = bf16_exact((n, Hq, d), rng)
    q1 = bf16_exact((n, Hq, d), rng)
    K = bf16_exact((Hkv, n, d), rng)
    V = bf16_exact((Hkv, n, d), rng)
    pos = orc.query_positions(n, n)
    sel = orc.full_attn_select_rows(q0, K, V, pos, k, W, orc.default_scale(d))
    o, _ = orc.sparse_attention_rows(q1, K, V, sel["idx"], pos, W, orc.default_scale(d))
    ref = sdpa_rows(q1, K, V, pos, n)
    np.testing.assert_allclose(o, ref, atol=1e-12)


@pytest.mark.parametrize("W", [1, 4, 16])
def test_k0_equals_sliding_window(W):
    """Pin: with k = 0 the sparse layer is sliding-window attention, i.e.
    SDPA with the band mask p-W < j <= p."""
    rng = np.random.default_rng(22 + W)
    d, n, Hq, Hkv = 128, 40, 4, 2
    q = bf16_exact((n, Hq, d), rng)
    K = bf16_exact((Hkv, n, d), rng)
    V = bf16_exact((Hkv, n, d), rng)
    pos = orc.query_positions(n, n)
    idx = np.full((n, Hkv, 0), -1)
    o, _ = orc.sparse_attention_rows(q, K, V, idx, pos, W, orc.default_scale(d))
    ref = sdpa_rows(q, K, V, pos, n, band=W)
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_sparse_is_key_order_independent():
    """Order independence of softmax over keys: permuting an index row (and
    its padding) leaves the sparse output unchanged."""
    rng = np.random.default_rng(23)
    d, n = 128, 60
    q0 = bf16_exact((n, 4, d), rng)
    q1 = bf16_exact((n, 4, d), rng)
    K = bf16_exact((1, n, d), rng)
    V = bf16_exact((1, n, d), rng)
    pos = orc.query_positions(n, n)
    sel = orc.full_attn_select_rows(q0, K, V, pos, 7, 6, orc.default_scale(d))
    idx = sel["idx"].copy()
    for t in range(n):
        idx[t, 0] = idx[t, 0][rng.permutation(7)]
    o1, _ = orc.sparse_attention_rows(q1, K, V, sel["idx"], pos, 6, orc.default_scale(d))
    o2, _ = orc.sparse_attention_rows(q1, K, V, idx, pos, 6, orc.default_scale(d))
    np.testing.assert_allclose(o1, o2, atol=1e-13)


def test_selected_count_rule():
    """Count of valid indices per row is min(k, max(0, p-W+1))."""
    rng = np.random.default_rng(24)
    d, n, k, W = 128, 70, 9, 13
    q = bf16_exact((n, 4, d), rng)
    K = bf16_exact((1, n, d), rng)
    V = bf16_exact((1, n, d), rng)
    pos = orc.query_positions(n, n)
    sel = orc.full_attn_select_rows(q, K, V, pos, k, W, orc.default_scale(d))
    for t in range(n):
        row = sel["idx"][t, 0]
        cnt = int((row >= 0).sum())
        assert cnt == min(k, max(0, t - W + 1))
        assert np.all(row[:cnt] <= t - W)
        assert np.all(np.diff(row[:cnt]) > 0)
        assert np.all(row[cnt:] == -1)


# ---------------------------------------------------------- chunk and decode

def test_chunk_rows_equal_full_prefill_rows():
    """Consistency: the rows of a chunk at the end of a cache equal the same
    rows of a prefill over the whole sequence (outputs and selections)."""
    rng = np.random.default_rng(31)
    d, n, nq, k, W = 128, 64, 16, 6, 5
    q = bf16_exact((n, 8, d), rng)
    K = bf16_exact((2, n, d), rng)
    V = bf16_exact((2, n, d), rng)
    s = orc.default_scale(d)
    full = orc.full_attn_select_rows(q, K, V, orc.query_positions(n, n), k, W, s)
    chunk = orc.full_attn_select_rows(q[n - nq:], K, V, orc.query_positions(nq, n), k, W, s)
    np.testing.assert_allclose(chunk["o"], full["o"][n - nq:], atol=0)
    assert np.array_equal(chunk["idx"], full["idx"][n - nq:])


def test_decode_step_equals_prefill_row():
    """Consistency: a decode step at position p (after writing kv_new into slot
    p) equals prefill row p, for the full layer and for each sparse layer,
    and every sparse layer uses the one selection of the full layer."""
    rng = np.random.default_rng(32)
    d, n, k, W, Hq, Hkv = 128, 40, 5, 4, 8, 2
    s = orc.default_scale(d)
    q = bf16_exact((n, Hq, d), rng)
    qs = [bf16_exact((n, Hq, d), rng) for _ in range(3)]
    K = bf16_exact((Hkv, n, d), rng)
    V = bf16_exact((Hkv, n, d), rng)
    pos = orc.query_positions(n, n)
    full = orc.full_attn_select_rows(q, K, V, pos, k, W, s)
    sparse = [orc.sparse_attention_rows(x, K, V, full["idx"], pos, W, s)[0] for x in qs]
    Kc = np.zeros((Hkv, n + 3, d), np.float32)
    Vc = np.zeros((Hkv, n + 3, d), np.float32)
    Kc[:, :n - 1] = K[:, :n - 1]
    Vc[:, :n - 1] = V[:, :n - 1]
    kv_new = np.stack([K[:, n - 1], V[:, n - 1]], axis=1)
    dec = orc.decode_step(q[n - 1], [x[n - 1] for x in qs], kv_new, Kc, Vc, n, k, W, s)
    np.testing.assert_allclose(dec["o_full"], full["o"][n - 1], atol=0)
    assert np.array_equal(dec["idx"], full["idx"][n - 1])
    for a, b in zip(dec["o_sparse"], sparse):
        np.testing.assert_allclose(a, b[n - 1], atol=0)
    assert np.array_equal(Kc[:, n - 1], K[:, n - 1])


def test_lse_combine_of_split_partials():
    """Split partials over disjoint key subsets merged with the log-sum-exp
    correction equal attention over the union (split-K decode)."""
    rng = np.random.default_rng(33)
    d, n = 128, 90
    q = bf16_exact((4, d), rng, 2.0)
    K = bf16_exact((n, d), rng)
    V = bf16_exact((n, d), rng)
    keys = np.arange(n)
    whole = orc.attention_over_set(q, K, V, keys, 0.2)
    parts = [orc.attention_over_set(q, K, V, keys[a:b], 0.2) for a, b in [(0, 13), (13, 60), (60, 90)]]
    o, lse = orc.lse_combine(parts)
    np.testing.assert_allclose(o, whole[0], atol=1e-13)
    np.testing.assert_allclose(lse, whole[1], atol=1e-13)


# ---------------------------------------------------------------- normalised score (reading R1')

def test_prob_score_is_log_of_largest_attention_probability():
    """Pinned on torch.softmax (float64): exp(sigma'_j) equals the largest
    attention probability that the group's heads give key j, computed by
    softmax over the causal row independently of the oracle's lse."""
    rng = np.random.default_rng(41)
    G, n, d, W = 4, 90, 128, 8
    q = bf16_exact((1, G, d), rng)
    K = bf16_exact((1, n, d), rng)
    V = bf16_exact((1, n, d), rng)
    scale = orc.default_scale(d)
    p = n - 1
    res = orc.full_attn_select_rows(q, K, V, [p], 10, W, scale, score="prob")
    s = torch.from_numpy(q[0].astype(np.float64)) @ torch.from_numpy(K[0].astype(np.float64)).T * scale
    prob = torch.softmax(s, dim=1)                      # [G][n], causal row covers 0..p = all keys
    want = torch.log(prob.max(dim=0).values[:p - W + 1]).numpy()
    np.testing.assert_allclose(res["sigma"][0][0], want, rtol=0, atol=1e-12)


def test_prob_score_with_one_head_ranks_like_the_logit():
    """G = 1: the normalised score is the logit minus a per-row constant, so
    the selection equals the logit selection."""
    rng = np.random.default_rng(42)
    n, d, W, k = 300, 128, 16, 40
    q = bf16_exact((3, 2, d), rng)
    K = bf16_exact((2, n, d), rng)
    V = bf16_exact((2, n, d), rng)
    pos = [150, 220, 299]
    a = orc.full_attn_select_rows(q, K, V, pos, k, W, orc.default_scale(d), score="logit")
    b = orc.full_attn_select_rows(q, K, V, pos, k, W, orc.default_scale(d), score="prob")
    assert np.array_equal(a["idx"], b["idx"])
    for r in range(3):
        for g in range(2):
            np.testing.assert_allclose(a["sigma"][r][g] - b["sigma"][r][g], b["lse"][r, g], rtol=0, atol=1e-12)


def test_prob_score_prefers_the_sharper_head():
    """Constructed G = 2 case where the two scores disagree: head A is flat
    (many equal logits, large lse), head B is peaked. Key x: A gives 3, B
    gives 0; key y: A gives 0, B gives 2.5. The logit score ranks x first;
    the normalised score ranks y first because head B concentrates its
    probability on y (brute force below)."""
    d, n, W = 128, 40, 1
    K = np.zeros((1, n, d), np.float32)
    K[0, :, 2] = 1.0                    # background keys: logit 3 for head A (flat), 0 for B
    K[0, 0, 2], K[0, 0, 0] = 1.0, 0.0   # key x: A 3, B 0
    K[0, 1, 2], K[0, 1, 1] = 0.0, 1.0   # key y: A 0, B 2.5
    q = np.zeros((1, 2, d), np.float32)
    q[0, 0, 2] = 3.0                    # head A
    q[0, 1, 1] = 2.5                    # head B
    V = np.zeros((1, n, d), np.float32)
    p = n - 1
    lg = orc.full_attn_select_rows(q, K, V, [p], 1, W, 1.0, score="logit")
    pr = orc.full_attn_select_rows(q, K, V, [p], 1, W, 1.0, score="prob")
    # brute force of R1': per head logits over keys 0..p, log-softmax, max over heads
    Kd = K.astype(np.float64)
    logits = np.array([[3.0 * Kd[0, j, 2] for j in range(n)], [2.5 * Kd[0, j, 1] for j in range(n)]])
    lsm = logits - np.log(np.exp(logits).sum(axis=1, keepdims=True))
    best = lsm[:, :p - W + 1].max(axis=0)
    assert int(np.argmax(best)) == 1
    assert lg["idx"][0, 0, 0] != 1 and pr["idx"][0, 0, 0] == 1
    np.testing.assert_allclose(pr["sigma"][0][0], best, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- FP8 cache quantiser

def _e4m3_values():
    """All finite e4m3 values with their codes, from the format's definition
    (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
    subnormal; code 0x7f / 0xff is NaN, so 448 is the largest value)."""
    vals = {}
    for code in range(256):
        s, ex, m = code >> 7, (code >> 3) & 15, code & 7
        if ex == 15 and m == 7:
            continue
        mag = (m / 8.0) * 2.0 ** -6 if ex == 0 else (1 + m / 8.0) * 2.0 ** (ex - 7)
        vals[code] = -mag if s else mag
    return vals


def test_fp8_conversion_is_round_to_nearest_even_by_brute_force():
    """Pins the quantiser's rounding on the e4m3 definition: every in-range
    input maps to the nearest e4m3 value, ties to the even code."""
    vals = _e4m3_values()
    pos = sorted((v, c) for c, v in vals.items() if v >= 0 and not (v == 0 and c == 0x80))
    rng = np.random.default_rng(51)
    xs = list(rng.uniform(-448, 448, 3000)) + list(rng.standard_normal(2000) * 2.0 ** rng.uniform(-10, 8, 2000))
    mids = [(a[0] + b[0]) / 2 for a, b in zip(pos[:-1], pos[1:])]
    xs += mids + [-m for m in mids]
    xs = np.array(xs, np.float32).astype(np.float64)  # float32-exact inputs
    codes, deq = orc.quantize_fp8(xs, 0)
    for x, c, d in zip(xs, codes, deq):
        mag = abs(x)
        best = min(pos, key=lambda vc: (abs(vc[0] - mag), vc[1] & 1))  # nearest, then even code
        assert abs(d) == best[0], (x, d, best)
        if d != 0:
            assert (d < 0) == (x < 0)


def test_fp8_scale_exponent_bounds():
    for amax in [1e-30, 0.013, 1.0, 3.7, 447.99, 448.0, 448.01, 896.0, 1e6]:
        e = orc.fp8_scale_exponent(amax)
        assert amax <= 448.0 * 2.0 ** e
        assert amax > 448.0 * 2.0 ** (e - 1)
    assert orc.fp8_scale_exponent(0.0) == 0


def test_fp8_quantiser_error_bound_and_exact_values():
    """Dequantised values: within 2^-4 relative of the input in the normal
    range (3 mantissa bits, round to nearest); values that are e4m3 numbers
    times 2^e round-trip exactly; the head maximum lands at or below 448."""
    rng = np.random.default_rng(52)
    x = rng.standard_normal((64, 128)) * 3.0
    e = orc.fp8_scale_exponent(np.abs(x).max())
    codes, deq = orc.quantize_fp8(x, e)
    normal = np.abs(x) >= 2.0 ** (e - 6)
    rel = np.abs(deq - x)[normal] / np.abs(x)[normal]
    assert rel.max() <= 2.0 ** -4
    assert np.abs(deq).max() <= 448.0 * 2.0 ** e
    exact = np.array([v for v in _e4m3_values().values()]) * 2.0 ** e
    _, back = orc.quantize_fp8(exact, e)
    assert np.array_equal(back, exact)
    # values past the range saturate instead of becoming NaN
    _, sat = orc.quantize_fp8(np.array([1e9, -1e9]), 0)
    assert list(sat) == [448.0, -448.0]


# ---------------------------------------------------------------- block-level selection (reading R11)

def test_block_select_with_unit_blocks_is_token_select():
    rng = np.random.default_rng(61)
    for n, k in [(500, 40), (70, 64), (3, 8), (129, 128)]:
        sig = rng.standard_normal(n)
        a, ta = orc.topk_select(sig, k)
        b, tb = orc.block_select(sig, k, block=1)
        assert np.array_equal(a, b) and ta == tb


def test_block_select_brute_force():
    """Brute force with plain Python on small rows: every block's maximum,
    ranked by (score desc, index asc), the first k/B blocks expanded."""
    rng = np.random.default_rng(62)
    for n, k, B in [(300, 64, 16), (257, 128, 64), (64, 64, 64), (1000, 192, 64)]:
        sig = np.round(rng.standard_normal(n), 2)  # rounding creates ties
        got, _ = orc.block_select(sig, k, block=B)
        blocks = [(max(sig[i:i + B]), i // B) for i in range(0, n, B)]
        ranked = sorted(blocks, key=lambda t: (-float(np.float32(t[0])), t[1]))[:k // B]
        want = sorted(j for _, b in ranked for j in range(b * B, min(b * B + B, n)))
        assert list(got[:len(want)]) == want and np.all(got[len(want):] == -1)


def test_block_selection_rows_keep_whole_blocks():
    rng = np.random.default_rng(63)
    q = bf16_exact((2, 4, 128), rng)
    K = bf16_exact((1, 900, 128), rng)
    V = bf16_exact((1, 900, 128), rng)
    res = orc.full_attn_select_rows(q, K, V, [600, 899], 128, 32, orc.default_scale(128), blocks=True)
    for r, p in enumerate([600, 899]):
        sel = res["idx"][r, 0]
        sel = sel[sel >= 0]
        c = p - 32 + 1
        for b in set(sel // 64):
            assert set(sel[sel // 64 == b]) == set(range(64 * b, min(64 * b + 64, c)))
        assert len(set(sel // 64)) == 2


# ---------------------------------------------------------------- union of per-head top-k (reading R12)

def test_head_union_with_one_head_is_token_select():
    rng = np.random.default_rng(71)
    q = bf16_exact((1, 128), rng)
    K = bf16_exact((700, 128), rng)
    for p, k in [(699, 64), (100, 128), (40, 8)]:
        got, heads = orc.head_union_select(q, K, p, 16, orc.default_scale(128), k)
        want, tau = orc.topk_select(orc.selection_scores(q, K, p, 16, orc.default_scale(128)), k)
        assert np.array_equal(got, want) and heads[0][1] == tau


def test_head_union_brute_force():
    """Plain Python on small rows: each head's candidates ranked by its own
    float32 logit (desc, index asc), the first k kept, the sets united."""
    rng = np.random.default_rng(72)
    G, n, W, k = 4, 90, 8, 12
    q = np.round(rng.standard_normal((G, 128)), 1)
    K = np.round(rng.standard_normal((n, 128)), 1)  # coarse values: ties
    sc = 0.125
    for p in (n - 1, 50, 15, 7):
        got, _ = orc.head_union_select(q, K, p, W, sc, k)
        c = max(0, p - W + 1)
        union = set()
        for h in range(G):
            logit = [sum(sc * q[h, i] * K[j, i] for i in range(128)) for j in range(c)]
            ranked = sorted(range(c), key=lambda j: (-float(np.float32(logit[j])), j))[:k]
            union.update(ranked)
        want = sorted(union)
        assert list(got[:len(want)]) == want and np.all(got[len(want):] == -1), p


def test_head_union_size_bounds_and_identical_heads():
    rng = np.random.default_rng(73)
    K = bf16_exact((600, 128), rng)
    q = bf16_exact((8, 128), rng)
    got, _ = orc.head_union_select(q, K, 599, 32, orc.default_scale(128), 40)
    size = int((got >= 0).sum())
    assert 40 <= size <= 8 * 40
    # heads that are copies of one head select one set: the union is that set
    q1 = np.repeat(q[:1], 8, axis=0)
    same, _ = orc.head_union_select(q1, K, 599, 32, orc.default_scale(128), 40)
    one, _ = orc.topk_select(orc.selection_scores(q[:1], K, 599, 32, orc.default_scale(128)), 40)
    assert np.array_equal(same[:40], one) and np.all(same[40:] == -1)


def test_head_union_contains_group_max_top_token():
    """The group-max top-1 token is some head's top-1, so it is in the union."""
    rng = np.random.default_rng(74)
    K = bf16_exact((1, 500, 128), rng)
    V = bf16_exact((1, 500, 128), rng)
    q = bf16_exact((3, 4, 128), rng)
    pos = [499, 300, 200]
    u = orc.full_attn_select_rows(q, K, V, pos, 1, 16, orc.default_scale(128), union=True)
    t = orc.full_attn_select_rows(q, K, V, pos, 1, 16, orc.default_scale(128))
    for r in range(3):
        assert t["idx"][r, 0, 0] in set(u["idx"][r, 0].tolist())
        assert u["idx"].shape == (3, 1, 4)


# ---------------------------------------------------------------- KV Bridging (R13)

def test_kv_bridge_one_hot_hidden_states_pick_weight_columns():
    """Pin of the layout: a hidden state that is the unit vector e_i gives, for
    every KV head g, key row = column i of that head's key projection rows and
    value row = column i of its value projection rows. A transposed weight, a
    head or K/V mix-up, or a dropped row fails this."""
    rng = np.random.default_rng(7)
    Hkv, d, d_model = 3, 128, 40
    w = bf16_exact((Hkv, 2, d, d_model), rng)
    cols = [0, 5, 39, 17]
    h = np.zeros((len(cols), d_model), np.float32)
    for t, i in enumerate(cols):
        h[t, i] = 1.0
    K, V = orc.kv_bridge(h, w)
    assert K.shape == (Hkv, len(cols), d) and V.shape == (Hkv, len(cols), d)
    for g in range(Hkv):
        for t, i in enumerate(cols):
            assert np.array_equal(K[g, t], w[g, 0, :, i])
            assert np.array_equal(V[g, t], w[g, 1, :, i])


def test_kv_bridge_matches_torch_linear_in_float64():
    """Pin against a library routine: torch.nn.functional.linear (float64)
    with the heads' K rows and V rows stacked as one weight."""
    rng = np.random.default_rng(8)
    Hkv, d, d_model, n = 2, 128, 96, 33
    h = bf16_exact((n, d_model), rng)
    w = bf16_exact((Hkv, 2, d, d_model), rng, 1 / math.sqrt(d_model))
    K, V = orc.kv_bridge(h, w)
    y = torch.nn.functional.linear(torch.from_numpy(h).double(), torch.from_numpy(w).double().reshape(-1, d_model))
    y = y.reshape(n, Hkv, 2, d).numpy()
    assert np.allclose(K, y[:, :, 0].transpose(1, 0, 2), rtol=0, atol=1e-12)
    assert np.allclose(V, y[:, :, 1].transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_kv_bridge_rows_independent():
    """Each token's K/V depend on its own hidden state only: bridging a chunk
    equals the matching rows of bridging the whole sequence (a chunked
    prefill writes the same cache rows)."""
    rng = np.random.default_rng(9)
    h = bf16_exact((50, 64), rng)
    w = bf16_exact((2, 2, 128, 64), rng, 0.125)
    K, V = orc.kv_bridge(h, w)
    K2, V2 = orc.kv_bridge(h[20:35], w)
    assert np.array_equal(K[:, 20:35], K2) and np.array_equal(V[:, 20:35], V2)


def test_bf16_round_matches_torch_and_ties_to_even():
    """Pin of the cache rounding against torch's float32 -> bfloat16
    conversion (round to nearest even) on random values and on exact halfway
    cases, where the even neighbour must win."""
    rng = np.random.default_rng(10)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(orc.bf16_round(x.astype(np.float64)), want)
    half = 2.0 ** -8  # half a bf16 ulp of [1, 2)
    ties = np.array([1 + half, 1 + 3 * half, -(1 + half), 2 + 2 * half, 1 + 5 * half])
    assert np.array_equal(orc.bf16_round(ties), [1.0, 1 + 4 * half, -1.0, 2.0, 1 + 4 * half])
