"""Acceptance rules for GPU results against the CPU oracle (shared test helpers).

Index rows: every GPU row must be ascending, duplicate-free, hold exactly
min(k, |C(p)|) valid entries followed by -1 padding, and lie in C(p); the
GPU set may differ from the oracle's only by tokens whose oracle score lies
within 1e-3 of the oracle's k-th score (near-ties straddling the cut).
Outputs: bf16 GPU outputs widened to fp32 against the oracle's float64 with
max-abs <= 2e-2 and mean-abs <= 2e-3 over all checked elements; sparse layers
are recomputed by the oracle with the GPU's own selection, so a legitimate
near-tie swap is not counted as an output error.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as orc

TIE_BAND = 1e-3
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


class OutStats:
    def __init__(self):
        self.max_abs = 0.0
        self.sum_abs = 0.0
        self.n = 0

    def add(self, got, want):
        d = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
        self.max_abs = max(self.max_abs, float(d.max()) if d.size else 0.0)
        self.sum_abs += float(d.sum())
        self.n += d.size

    @property
    def mean_abs(self):
        return self.sum_abs / max(1, self.n)

    def check(self, what=""):
        assert self.n > 0
        assert self.max_abs <= MAX_ABS, f"{what}: max-abs {self.max_abs:.3e} > {MAX_ABS}"
        assert self.mean_abs <= MEAN_ABS, f"{what}: mean-abs {self.mean_abs:.3e} > {MEAN_ABS}"


def check_idx_row(got: np.ndarray, ref: np.ndarray, sigma: np.ndarray, tau: float, p: int, window: int, k: int,
                  where=""):
    """Returns the number of near-tie swaps; asserts the rules above."""
    ncand = max(0, p - window + 1)
    cnt = min(k, ncand)
    got = np.asarray(got, np.int64)
    assert got.shape == (k,), where
    assert np.all(got[:cnt] >= 0) and np.all(got[cnt:] == -1), f"{where}: padding/count wrong: {got[:8]}..."
    v = got[:cnt]
    if cnt:
        assert np.all(np.diff(v) > 0), f"{where}: not ascending / duplicates"
        assert v[0] >= 0 and v[-1] <= p - window, f"{where}: index outside C(p)"
    A = set(v.tolist())
    R = set(int(x) for x in ref if x >= 0)
    diff = A ^ R
    for j in diff:
        assert abs(sigma[j] - tau) <= TIE_BAND, \
            f"{where}: token {j} differs (sigma {sigma[j]:.6f}, tau {tau:.6f}, in_gpu={j in A})"
    return len(diff)


def check_block_row(got: np.ndarray, ref: np.ndarray, sigma: np.ndarray, tau: float, p: int, window: int, k: int,
                    where="", block=64):
    """Block-level selection row: whole aligned blocks of C(p), ascending, the
    min(k / block, blocks of C(p)) of them expanded to their tokens, then -1
    padding; the GPU block set may differ from the oracle's only by blocks
    whose block score lies within 1e-3 of the oracle's last block score."""
    ncand = max(0, p - window + 1)
    nblk = -(-ncand // block)
    nsel = min(k // block, nblk)
    got = np.asarray(got, np.int64)
    assert got.shape == (k,), where
    v = got[got >= 0]
    gb = sorted(set((v // block).tolist()))
    assert len(gb) == nsel, f"{where}: {len(gb)} blocks, want {nsel}"
    want = np.concatenate([np.arange(b * block, min((b + 1) * block, ncand)) for b in gb]) if gb else \
        np.zeros(0, np.int64)
    assert np.array_equal(got[:len(want)], want) and np.all(got[len(want):] == -1), \
        f"{where}: not whole ascending blocks then padding: {got[:8]}..."
    R = set(int(x) // block for x in ref if x >= 0)
    diff = set(gb) ^ R
    for b in diff:
        bs = float(sigma[b * block:(b + 1) * block].max())
        assert abs(bs - tau) <= TIE_BAND, f"{where}: block {b} differs (score {bs:.6f}, tau {tau:.6f})"
    return len(diff)


def check_union_row(got: np.ndarray, ref: np.ndarray, heads, p: int, window: int, k: int, where=""):
    """Union of per-head top-k row (G*k entries): ascending, duplicate-free,
    inside C(p), -1 padded. A token only the GPU took must be a near-tie of
    some head (score within 1e-3 of that head's k-th score or above it); a
    token only the oracle took must not be a clear pick (above k-th + 1e-3)
    of any head."""
    G = len(heads)
    ncand = max(0, p - window + 1)
    got = np.asarray(got, np.int64)
    assert got.shape == (G * k,), where
    v = got[got >= 0]
    n = len(v)
    assert np.all(got[:n] >= 0) and np.all(got[n:] == -1), f"{where}: padding not at the end"
    assert min(k, ncand) <= n <= min(G * k, ncand), f"{where}: {n} entries"
    if n:
        assert np.all(np.diff(v) > 0) and v[-1] <= p - window, f"{where}: not ascending or outside C(p)"
    A, R = set(v.tolist()), set(int(x) for x in ref if x >= 0)
    for j in A - R:
        assert any(s[j] >= t - TIE_BAND for s, t in heads), f"{where}: token {j} is no head's pick"
    for j in R - A:
        assert not any(s[j] > t + TIE_BAND for s, t in heads), f"{where}: token {j} missing"
    return len(A ^ R)


def cache_np(kv: torch.Tensor, b: int, n: int):
    """K, V of sequence b as float64 numpy [Hkv][n][d] (exact widening of bf16;
    float64 so that the oracle takes contiguous ranges as views)."""
    K = kv[b, :, :n, 0].cpu().double().numpy()
    V = kv[b, :, :n, 1].cpu().double().numpy()
    return K, V


def sample_rows(n_q: int, n_kv: int, top_k: int, window: int, spans=(), evenly=8):
    """Deterministic query-row sample: first and last rows, the rows at the
    window and top-k boundaries (p = W-1, W, W+k-1, W+k when inside the
    chunk), the first row of some needle spans, and evenly spaced rows."""
    off = n_kv - n_q
    rows = {0, n_q - 1}
    for p in (window - 1, window, window + top_k - 1, window + top_k):
        if off <= p < n_kv:
            rows.add(p - off)
    for t0 in list(spans)[:4]:
        rows.add(int(t0))
    for i in range(evenly):
        rows.add(int(i * (n_q - 1) / max(1, evenly - 1)))
    return sorted(r for r in rows if 0 <= r < n_q)


def check_idx_structure(idx, positions, window, k, chunk=4096):
    """Oracle-free check of EVERY index row, on the device: row r (positions[r]
    = p) must hold min(k, |C(p)|) valid entries, strictly ascending (so no
    duplicates), all in C(p) = [0, p - W], followed by -1 padding.
    idx: int32 tensor [R][Hkv][k] (or [R][k]); positions: int64 tensor [R] on
    the same device. Returns the number of rows checked."""
    if idx.dim() == 2:
        idx = idx[:, None, :]
    R = idx.shape[0]
    assert positions.shape == (R,)
    ar = torch.arange(k, device=idx.device)
    for r0 in range(0, R, chunk):
        blk = idx[r0:r0 + chunk].long()
        p = positions[r0:r0 + chunk].long()
        cnt = (p - window + 1).clamp(min=0, max=k)
        want = ar[None, None, :] < cnt[:, None, None]
        bad = ~torch.where(want, blk >= 0, blk == -1)
        assert not bool(bad.any()), f"rows {r0}..: padding or count wrong at {bad.nonzero()[:4].tolist()}"
        lim = (p - window)[:, None, None]
        assert not bool((want & ((blk > lim) | (blk < 0))).any()), f"rows {r0}..: entry outside C(p)"
        if k > 1:
            up = blk[..., 1:] > blk[..., :-1]
            assert not bool((want[..., 1:] & ~up).any()), f"rows {r0}..: not strictly ascending"
    return R


def check_prefill(q_full, kv, n_kv, top_k, window, o, lse, idx, rows=None, q_sparse=(), o_sparse=(), scale=None,
                  score="logit", blocks=False, union=False, progress=0):
    """Checks one prefill call (and its sparse layers) on the given query rows;
    score names the oracle's selection score ("logit" or "prob"), blocks asks
    for block-level selection."""
    B, n_q, Hq, d = q_full.shape
    scale = orc.default_scale(d) if scale is None else scale
    rows = list(range(n_q)) if rows is None else list(rows)
    pos = orc.query_positions(n_q, n_kv)[rows]
    full_stats, lse_stats, sp_stats = OutStats(), OutStats(), OutStats()
    swaps = 0
    o_np, idx_np = f32(o), idx.cpu().numpy()
    lse_np = None if lse is None else lse.cpu().numpy()
    qs_np = [f32(x) for x in q_sparse]
    os_np = [f32(x) for x in o_sparse]
    for b in range(B):
        K, V = cache_np(kv, b, n_kv)
        qb = f32(q_full[b])[rows]
        if progress:  # long contexts: the oracle in row batches, with a line per batch
            parts = []
            for r0 in range(0, len(rows), progress):
                parts.append(orc.full_attn_select_rows(qb[r0:r0 + progress], K, V, pos[r0:r0 + progress], top_k,
                                                       window, scale, score, blocks=blocks, union=union))
                print(f"[case] oracle rows {r0 + len(parts[-1]['o'])}/{len(rows)}", flush=True)
            res = {"o": np.concatenate([x["o"] for x in parts]), "lse": np.concatenate([x["lse"] for x in parts]),
                   "idx": np.concatenate([x["idx"] for x in parts])}
            if union:
                res["heads"] = sum((x["heads"] for x in parts), [])
            else:
                res["tau"] = np.concatenate([x["tau"] for x in parts])
                res["sigma"] = sum((x["sigma"] for x in parts), [])
        else:
            res = orc.full_attn_select_rows(qb, K, V, pos, top_k, window, scale, score, blocks=blocks, union=union)
        check_row = check_block_row if blocks else check_idx_row
        full_stats.add(o_np[b, rows], res["o"])
        if lse_np is not None:
            lse_stats.add(lse_np[b][:, rows].T, res["lse"])
        for r, t in enumerate(rows):
            for g in range(K.shape[0]):
                if union:
                    swaps += check_union_row(idx_np[b, t, g], res["idx"][r, g], res["heads"][r][g], int(pos[r]),
                                             window, top_k, where=f"b{b} t{t} g{g}")
                    continue
                swaps += check_row(idx_np[b, t, g], res["idx"][r, g], res["sigma"][r][g], res["tau"][r, g],
                                       int(pos[r]), window, top_k, where=f"b{b} t{t} g{g}")
        gidx = idx_np[b][rows]
        for qs, osp in zip(qs_np, os_np):
            ref, _ = orc.sparse_attention_rows(qs[b][rows], K, V, gidx, pos, window, scale)
            sp_stats.add(osp[b, rows], ref)
    full_stats.check("full-layer o")
    if lse_np is not None:
        assert lse_stats.max_abs <= 1e-3, f"lse max-abs {lse_stats.max_abs}"
    if qs_np:
        sp_stats.check("sparse-layer o")
    return {"swaps": swaps, "full": full_stats, "sparse": sp_stats}
