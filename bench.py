#!/usr/bin/env python3
"""Benchmark of the hybrid sparse attention hot path on one MI355X.

One step = one pass of the whole hot path over the 1M-token workload (B=1,
1,048,576 cached tokens + a 16384-token chunk, 32 query / 4 KV heads, d=128,
top-k 4096, window 1024, 256 needles): the chunk's full-attention layer with
token selection and the three sparse layers that reuse its cache and
indices (prefill), then 16 decode steps, each appending a token, running the
full layer with selection once and the three sparse layers on that
selection. Inputs are resident in HBM before timing starts. `value` is the
step's tokens (16384 prefill + 16 decode) per second; the prefill tokens/s
and decode microseconds per step are reported beside it.

Also measured in the same run (not part of `value`): the 32K prefill block
(with the option paths), the 8K chunk over a 128K cache, the batched decode
(64 sequences of 64K-256K tokens, 32 steps), the decode step replayed as one
HIP graph, KV Bridging (the cross-decoder cache built from hidden states)
against the full prefill of the same chunk, a plain copy and the gather
probe (rates the decode and gather rooflines are also given against), and
the CPU oracle timed on a bounded sample of the 1M-token workload.

Per-kernel durations come from the library's HIP-event timing on the stream
the kernels run on; `roofline` describes the kernel that takes the most time
in the step. Prints ONE JSON line on stdout; details go to stderr.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "traffic_counters.md")
METRIC = "prefill tokens/s + decode us/step (sparse attn); % MFMA / HBM roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- work counts

def prefill_counts(w):
    """Algorithmic work of one prefill block: full layer FLOPs = 4 d Hq per
    causal (query, key) pair; sparse layer FLOPs = 4 d Hq per (query, kept
    key) and gathered bytes = 512 per kept key and KV head, plus q, o, idx."""
    d = 128
    off = w.n_kv - w.n_q
    pairs = s_sum = 0
    for t in range(w.n_q):
        p = off + t
        pairs += p + 1
        c = max(0, p - w.window + 1)
        s_sum += min(w.top_k, c) + min(w.window, p + 1)
    qo_bytes = 2 * w.B * w.n_q * w.Hq * d * 2.0
    idx_bytes = 4.0 * w.B * w.n_q * w.Hkv * w.top_k
    return {"full_flops": 4.0 * d * w.Hq * pairs * w.B,
            "sparse_flops_per_layer": 4.0 * d * w.Hq * s_sum * w.B,
            "sparse_gather_bytes_per_layer": 512.0 * w.Hkv * s_sum * w.B,
            "sparse_bytes_per_layer": 512.0 * w.Hkv * s_sum * w.B + qo_bytes + idx_bytes}


def decode_counts(w, lengths, steps):
    """Mean algorithmic bytes per decode step: full layer = every cached row
    (512 B per token and KV head); sparse layer = (k + W) rows per (sequence,
    KV head) + idx + q/o."""
    B = len(lengths)
    full = sum(512.0 * w.Hkv * (L + s + 1) for L in lengths for s in range(steps)) / steps
    rows = sum(min(w.top_k, max(0, L + s + 1 - w.window)) + min(w.window, L + s + 1)
               for L in lengths for s in range(steps)) / steps
    sparse = 512.0 * w.Hkv * rows + 4.0 * B * w.Hkv * w.top_k + 2 * 2.0 * B * w.Hq * 128
    return full, sparse


def hbm_roof(bytes_, us, ceil=None):
    gbs = bytes_ / (us * 1e-6) / 1e9
    r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
         "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": bytes_, "avg_us": round(us, 2)}
    if ceil:
        r["frac_of_copy_ceiling"] = round(gbs / ceil, 4)
    return r


def mfma_roof(flops, us, kernel):
    tf = flops / (us * 1e-6) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / PEAK_BF16_TFLOPS, 4), "kernel": kernel, "flops_per_launch": flops,
            "avg_us": round(us, 1)}


# ---------------------------------------------------------------- traffic

def device_source_hash():
    """sha256 over the kernel sources (the HIP files and the headers they
    include), comments and blank lines removed: a comment edit leaves the
    code, and so the counters taken on it, unchanged."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "token_level_sparse_hs_amd", "csrc")
    for p in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.hpp"))):
        text = open(p).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(os.path.basename(p).encode())
        h.update(code.encode())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per launch from the committed counter summary, used only if it
    was taken on the current kernel sources (else {})."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return {}, "no counter summary"
    m = re.search(r"kernel-sources-sha256: ([0-9a-f]{64})", text)
    if not m or m.group(1) != device_source_hash():
        return {}, "counter summary taken on other kernel sources"
    out = {}
    for kern, wl, val in re.findall(r"^traffic (\S+) (\S+) ([0-9.eE+]+)$", text, flags=re.M):
        out[(kern, wl)] = float(val)
    return out, "counters of the current kernel sources"


# ---------------------------------------------------------------- helpers

def kernel_table(kt, steps):
    return {k: {"launches_per_step": n / steps, "avg_us": round(tot / n * 1e3, 1)} for k, (n, tot) in kt.items()}


def avg_us(kt, name):
    n, tot = kt.get(name, (0, 0.0))
    return tot / n * 1e3 if n else None


class Ctx:
    def __init__(self):
        import torch
        import token_level_sparse_hs_amd as hs
        from token_level_sparse_hs_amd import _lib, synth
        _lib.load()
        self.torch, self.hs, self._lib, self.synth = torch, hs, _lib, synth
        self.dev = "cuda:0"


def decode_inputs(c, w, steps, B=1):
    synth, dev = c.synth, c.dev
    return [{
        "q_full": synth.randn_bf16((B, w.Hq, 128), synth.seed_for(w.cid, synth.T_QDEC, s), dev),
        "q_sparse": [synth.randn_bf16((B, w.Hq, 128), synth.seed_for(w.cid, synth.T_QDEC + 1 + i, s), dev)
                     for i in range(w.sparse_layers)],
        "kv_new": synth.randn_bf16((B, w.Hkv, 2, 128), synth.seed_for(w.cid, synth.T_KVNEW, s), dev),
    } for s in range(steps)]


class PrefillBlock:
    """Full layer with selection + the sparse layers over one prefill workload,
    with its workspaces allocated once."""

    def __init__(self, c, w, kv_capacity=None):
        self.c, self.w = c, w
        hs, _lib = c.hs, c._lib
        log(f"[bench] generating {w.name} inputs")
        self.case = c.synth.make_prefill_case(w, c.dev, kv_capacity=kv_capacity)
        self.q, self.kv, self.qs = self.case["q_full"], self.case["kv"], self.case["q_sparse"]
        shape = hs.make_shape(batch=w.B, n_q=w.n_q, n_kv=w.n_kv, kv_capacity=self.kv.shape[2], q_heads=w.Hq,
                              kv_heads=w.Hkv, top_k=w.top_k, window=w.window)
        self.ws = _lib.alloc_workspace(_lib.workspace_size(_lib.HS_OP_FULL_ATTN_SELECT, shape), c.dev)

    def __call__(self):
        hs, w = self.c.hs, self.w
        o, lse, idx = hs.full_attn_select(self.q, self.kv, w.n_kv, top_k=w.top_k, window=w.window,
                                          workspace=self.ws)
        outs = [hs.sparse_attn_reuse(x, self.kv, idx, top_k=w.top_k, window=w.window, n_kv=w.n_kv)
                for x in self.qs]
        return o, idx, outs


class DecodeSteps:
    """`steps` decode steps of a batch (append + full layer + selection once +
    the sparse layers), workspaces allocated once."""

    def __init__(self, c, w, kv, lengths, steps_data):
        self.c, self.w, self.kv, self.lengths, self.data = c, w, kv, lengths, steps_data
        hs, _lib, torch = c.hs, c._lib, c.torch
        steps = len(steps_data)
        self.bound = max(lengths) + steps
        shape = hs.make_shape(batch=len(lengths), n_q=1, n_kv=0, kv_capacity=kv.shape[2], q_heads=w.Hq,
                              kv_heads=w.Hkv, top_k=w.top_k, window=w.window)
        self.ws_full = _lib.alloc_workspace(_lib.workspace_size(_lib.HS_OP_DECODE_STEP, shape, self.bound), c.dev)
        self.ws_sp = _lib.alloc_workspace(_lib.workspace_size(_lib.HS_OP_SPARSE_ATTN_REUSE, shape, 1), c.dev)
        self.seqs = [torch.tensor([L + s + 1 for L in lengths], dtype=torch.int32, device=c.dev)
                     for s in range(steps)]

    def step(self, s):
        hs, w, st = self.c.hs, self.w, self.data[s]
        o, lse, idx = hs.decode_step(st["q_full"], st["kv_new"], self.kv, self.seqs[s], max(self.lengths) + s + 1,
                                     top_k=w.top_k, window=w.window, workspace=self.ws_full)
        for x in st["q_sparse"]:
            hs.sparse_attn_reuse(x, self.kv, idx, top_k=w.top_k, window=w.window, seq_lens=self.seqs[s],
                                 workspace=self.ws_sp)

    def __call__(self):
        for s in range(len(self.data)):
            self.step(s)


def timed_steps(c, fn, steps, warmup, label):
    """Warm-up, then `steps` timed calls with the library's per-kernel timing
    on; returns (ms per step from the host clock around synchronisations,
    per-kernel {name: (launches, total ms)})."""
    torch, _lib = c.torch, c._lib
    for i in range(warmup):
        fn()
    torch.cuda.synchronize()
    _lib.timing_read()
    _lib.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    _lib.timing_enable(False)
    kt = _lib.timing_read()
    ms = (t1 - t0) * 1e3 / steps
    log(f"[bench] {label}: {ms:.3f} ms/step over {steps} steps")
    for k, (n, tot) in sorted(kt.items(), key=lambda x: -x[1][1]):
        log(f"[bench]   {k:16s} launches={n:6d} avg={tot / n * 1e3:10.1f} us  share/step={tot / steps:9.3f} ms")
    return ms, kt


PREFILL_KERNELS = ("prefill_attn", "sample_scores", "threshold", "select_prefill", "sparse_prefill", "score_pass",
                   "select_blocks", "head_slice", "head_union", "lse_scatter", "kv_bridge")


# ---------------------------------------------------------------- headline

def run_headline(c, args, traffic):
    """The 1M-token step: the chunk's prefill block + its decode steps."""
    torch, w = c.torch, c.synth.WORKLOADS["ctx1m"]
    pre = PrefillBlock(c, w, kv_capacity=w.n_kv + w.decode_steps)
    dec = DecodeSteps(c, w, pre.kv, [w.n_kv], decode_inputs(c, w, w.decode_steps))

    def step():
        pre()
        dec()

    ms, kt = timed_steps(c, step, args.steps, args.warmup, "ctx1m step (prefill block + 16 decode steps)")
    pre_ms = sum(tot for k, (n, tot) in kt.items() if k in PREFILL_KERNELS) / args.steps
    dec_ms = sum(tot for k, (n, tot) in kt.items() if k not in PREFILL_KERNELS) / args.steps
    counts = prefill_counts(w)
    tokens = w.B * (w.n_q + w.decode_steps)
    dom = max(kt.items(), key=lambda x: x[1][1])[0]
    if dom == "sparse_prefill":  # a dense contraction over gathered rows, priced the same way
        roof = mfma_roof(counts["sparse_flops_per_layer"], avg_us(kt, dom), dom)
    else:
        roof = mfma_roof(counts["full_flops"], avg_us(kt, "prefill_attn"), "prefill_attn")
        if dom != "prefill_attn":
            log(f"[bench] note: the kernel with the largest share is {dom}, not prefill_attn")
    t = traffic[0].get((roof["kernel"], "ctx1m"))
    roof["traffic"] = t
    roof["traffic_note"] = traffic[1]
    full_layer_ms = sum(tot for k, (n, tot) in kt.items()
                        if k in ("prefill_attn", "sample_scores", "threshold", "select_prefill")) / args.steps
    fl_tf = counts["full_flops"] / (full_layer_ms * 1e-3) / 1e12
    dfull, dsp = decode_counts(w, [w.n_kv], w.decode_steps)
    out = {
        "value": round(tokens / (ms * 1e-3), 1), "ms_per_step": round(ms, 3),
        "prefill_tokens_per_s": round(w.n_q / (pre_ms * 1e-3), 1), "prefill_block_ms": round(pre_ms, 3),
        "decode_us_per_step": round(dec_ms * 1e3 / w.decode_steps, 2),
        "roofline": roof,
        "full_layer_with_selection": {"ms": round(full_layer_ms, 3), "tflops": round(fl_tf, 1),
                                      "frac_of_peak": round(fl_tf / PEAK_BF16_TFLOPS, 4)},
        "sparse_prefill_layer": {"avg_us": round(avg_us(kt, "sparse_prefill"), 1),
                                 "gather_GBs": round(counts["sparse_gather_bytes_per_layer"] /
                                                     (avg_us(kt, "sparse_prefill") * 1e-6) / 1e9, 1),
                                 "tflops": round(counts["sparse_flops_per_layer"] /
                                                 (avg_us(kt, "sparse_prefill") * 1e-6) / 1e12, 1)},
        "decode_full_roofline": hbm_roof(dfull, avg_us(kt, "decode_full")),
        "decode_sparse_roofline": hbm_roof(dsp, avg_us(kt, "sparse_decode")),
        "kernels": kernel_table(kt, args.steps),
    }
    return out, pre, dec


def memory_side(sp, traffic, workload):
    """Adds the sparse layer's memory-side bytes per launch (FETCH_SIZE +
    WRITE_SIZE from the committed counter summary of the current kernel
    sources) and their rate against the HBM peak; nothing if there is none.
    The algorithmic gather rate beside it counts every gathered row, L2 hits
    included."""
    t = traffic[0].get(("sparse_prefill", workload))
    if t is None:
        sp["memory_side_bytes"] = None
        return
    gbs = t / (sp["avg_us"] * 1e-6) / 1e9
    sp["memory_side_bytes"] = t
    sp["memory_side_GBs"] = round(gbs, 1)
    sp["frac_of_hbm_peak"] = round(gbs / PEAK_HBM_GBS, 4)


def host_case(pre):
    return {"kv": pre.kv.cpu(), "q_full": pre.q.cpu(), "q_sparse": [x.cpu() for x in pre.qs]}


def cpu_baseline(c, args, w, case, dec_data):
    """The oracle on a bounded sample of the headline step: evenly spaced rows
    of the chunk (full layer, selection, three sparse layers) and one decode
    step (append, full layer, selection, three sparse layers), on the very
    inputs the GPU step used, copied to the host."""
    import numpy as np
    import oracle as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    n = w.n_kv
    K = case["kv"][0, :, :n + w.decode_steps, 0].double().numpy()
    V = case["kv"][0, :, :n + w.decode_steps, 1].double().numpy()
    qf = case["q_full"][0].float().numpy()
    qs = [x[0].float().numpy() for x in case["q_sparse"]]
    scale = orc.default_scale(128)
    pos_all = orc.query_positions(w.n_q, n)

    def rows_time(rows):
        t0 = time.perf_counter()
        pos = pos_all[rows]
        res = orc.full_attn_select_rows(qf[rows], K[:, :n], V[:, :n], pos, w.top_k, w.window, scale)
        for x in qs:
            orc.sparse_attention_rows(x[rows], K[:, :n], V[:, :n], res["idx"], pos, w.window, scale)
        return time.perf_counter() - t0

    t_row = rows_time([w.n_q - 1])
    R = int(max(2, min(256, args.cpu_seconds / max(t_row, 1e-4))))
    rows = sorted(set(int(x) for x in np.linspace(0, w.n_q - 1, R)))
    t_rows = rows_time(rows)
    st = dec_data[0]
    t0 = time.perf_counter()
    orc.decode_step(st["q_full"][0].float().cpu().numpy(), [x[0].float().cpu().numpy() for x in st["q_sparse"]],
                    st["kv_new"][0].float().cpu().numpy(), K, V, n + 1, w.top_k, w.window, scale)
    t_dec = time.perf_counter() - t0
    t = t_rows + t_dec
    # the whole step at the sample's per-row and per-decode-step cost (the
    # chunk's rows all attend over about a million keys, so they cost alike)
    full = t_rows / len(rows) * w.n_q + t_dec * w.decode_steps
    return {"value": round((len(rows) + 1) / t, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "cpu": cpu_model(), "host_cpus": os.cpu_count(),
            "step_s_extrapolated": round(full, 1),
            "sample": f"{len(rows)} query rows evenly spaced over the {w.n_q}-row chunk of the 1M-token workload "
                      f"(full layer + selection + {len(qs)} sparse layers each) and 1 decode step "
                      f"(full layer + selection + {len(qs)} sparse layers), {t:.1f} s of CPU time"}


# ---------------------------------------------------------------- extras

def run_prefill_extra(c, args, name, options):
    w = c.synth.WORKLOADS[name]
    pre = PrefillBlock(c, w)
    ms, kt = timed_steps(c, pre, args.extra_steps, 1, f"{name} block")
    counts = prefill_counts(w)
    full_ms = sum(tot for k, (n, tot) in kt.items()
                  if k in ("prefill_attn", "sample_scores", "threshold", "select_prefill")) / args.extra_steps
    fl_tf = counts["full_flops"] / (full_ms * 1e-3) / 1e12
    sp_us = avg_us(kt, "sparse_prefill")
    out = {"workload": name, "ms_per_block": round(ms, 3), "tokens_per_s": round(w.B * w.n_q / (ms * 1e-3), 1),
           "prefill_attn": mfma_roof(counts["full_flops"], avg_us(kt, "prefill_attn"), "prefill_attn"),
           "full_layer_with_selection": {"ms": round(full_ms, 3), "tflops": round(fl_tf, 1),
                                         "frac_of_peak": round(fl_tf / PEAK_BF16_TFLOPS, 4)},
           "sparse_prefill_layer": {"avg_us": round(sp_us, 1),
                                    "gather_bytes": counts["sparse_gather_bytes_per_layer"],
                                    "gather_GBs": round(counts["sparse_gather_bytes_per_layer"] /
                                                        (sp_us * 1e-6) / 1e9, 1),
                                    "tflops": round(counts["sparse_flops_per_layer"] / (sp_us * 1e-6) / 1e12, 1)},
           "kernels": kernel_table(kt, args.extra_steps)}
    if options:
        out["options"] = prefill_options(c, w, pre)
    del pre
    c.torch.cuda.empty_cache()
    return out


def prefill_options(c, w, pre):
    """Options beside the default path, timed on the same inputs: the
    probability selection score, block-level selection and the per-head union
    (full layer), the union's wider sparse layer, and the sparse layer
    gathering from the FP8 copy of the cache."""
    hs, _lib, torch = c.hs, c._lib, c.torch
    q, kv, qs = pre.q, pre.kv, pre.qs
    _, _, idx = hs.full_attn_select(q, kv, w.n_kv, top_k=w.top_k, window=w.window, workspace=pre.ws)
    copy = hs.kv_to_fp8(kv, n_kv=w.n_kv)
    wss = {}
    for f in (hs.HS_FLAG_PROB_SCORE, hs.HS_FLAG_BLOCK_SELECT, hs.HS_FLAG_HEAD_UNION):
        shape = hs.make_shape(batch=w.B, n_q=w.n_q, n_kv=w.n_kv, kv_capacity=kv.shape[2], q_heads=w.Hq,
                              kv_heads=w.Hkv, top_k=w.top_k, window=w.window, flags=f)
        wss[f] = _lib.alloc_workspace(_lib.workspace_size(_lib.HS_OP_FULL_ATTN_SELECT, shape), c.dev)
    _, _, idx_u = hs.full_attn_select(q, kv, w.n_kv, top_k=w.top_k, window=w.window, flags=hs.HS_FLAG_HEAD_UNION,
                                      workspace=wss[hs.HS_FLAG_HEAD_UNION])
    full = lambda f: (lambda: hs.full_attn_select(q, kv, w.n_kv, top_k=w.top_k, window=w.window, flags=f,
                                                  workspace=wss[f]))
    runs = {
        "prob_score_full_layer": full(hs.HS_FLAG_PROB_SCORE),
        "block_select_full_layer": full(hs.HS_FLAG_BLOCK_SELECT),
        "head_union_full_layer": full(hs.HS_FLAG_HEAD_UNION),
        "head_union_sparse_layer": lambda: hs.sparse_attn_reuse(qs[0], kv, idx_u, top_k=w.top_k, window=w.window,
                                                               n_kv=w.n_kv, flags=hs.HS_FLAG_HEAD_UNION),
        "fp8_cache_conversion": lambda: hs.kv_to_fp8(kv, n_kv=w.n_kv, out=copy),
        "fp8_sparse_layer": lambda: hs.sparse_attn_reuse(qs[0], kv, idx, top_k=w.top_k, window=w.window,
                                                         n_kv=w.n_kv, kv_fp8=copy),
    }
    out = {}
    for name, fn in runs.items():
        ms, kt = timed_steps(c, fn, 3, 1, f"{w.name} option {name}")
        out[name] = {"ms": round(ms, 3), "kernels_us": {k: round(t / n * 1e3, 1) for k, (n, t) in kt.items()}}
    del copy, wss, idx_u
    return out


def run_decode_extra(c, args, name, lengths, steps, options):
    """Decode steps of one workload with eager calls; then the step replayed as
    one HIP graph; the FP8 and selection options beside it."""
    torch, hs, _lib, synth = c.torch, c.hs, c._lib, c.synth
    w = synth.WORKLOADS[name]
    log(f"[bench] generating {name} decode cache (sum of lengths {sum(lengths)})")
    case = synth.make_decode_case(w, c.dev, lengths, steps)
    kv = case["kv"]
    dec = DecodeSteps(c, w, kv, lengths, case["steps"])
    ms, kt = timed_steps(c, dec, 1, 1, f"{name}: {steps} decode steps")
    us_step = ms * 1e3 / steps
    g = hs.DecodeStepGraph(kv, batch=len(lengths), q_heads=w.Hq, sparse_layers=w.sparse_layers, top_k=w.top_k,
                           window=w.window)
    st = case["steps"][0]
    g.q.copy_(st["q_full"])
    g.kv_new.copy_(st["kv_new"])
    for d, x in zip(g.q_sparse, st["q_sparse"]):
        d.copy_(x)
    g.seq_lens.copy_(dec.seqs[0])
    g.step(max(lengths) + 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.step(max(lengths) + 1)
    torch.cuda.synchronize()
    us_graph = (time.perf_counter() - t0) * 1e6 / steps
    log(f"[bench] {name}: {us_step:.1f} us/step eager, {us_graph:.1f} us/step as one graph launch")
    dfull, dsp = decode_counts(w, lengths, steps)
    out = {"workload": name, "batch": len(lengths), "context": [min(lengths), max(lengths)], "steps": steps,
           "us_per_step": round(us_step, 2), "us_per_step_graph": round(us_graph, 2),
           "decode_full_roofline": hbm_roof(dfull, avg_us(kt, "decode_full")),
           "decode_sparse_roofline": hbm_roof(dsp, avg_us(kt, "sparse_decode")),
           "select_decode_us": round(avg_us(kt, "select_decode") or 0.0, 1),
           "kernels": kernel_table(kt, steps)}
    if options:
        out["options"] = decode_options(c, w, kv, lengths, dec, case["steps"][0])
    del case, kv, g, dec
    torch.cuda.empty_cache()
    return out


def decode_options(c, w, kv, lengths, dec, st):
    hs, _lib, torch = c.hs, c._lib, c.torch
    out = {}
    seq0, bound = dec.seqs[0], max(lengths) + 1
    copy = hs.kv_to_fp8(kv, n_kv=kv.shape[2])
    _, _, idx0 = hs.decode_step(st["q_full"], st["kv_new"], kv, seq0, bound, top_k=w.top_k, window=w.window,
                                workspace=dec.ws_full)

    def fp8_sparse():
        hs.kv_to_fp8(kv, seq_lens=seq0, out=copy)
        for x in st["q_sparse"]:
            hs.sparse_attn_reuse(x, kv, idx0, top_k=w.top_k, window=w.window, seq_lens=seq0,
                                 workspace=dec.ws_sp, kv_fp8=copy)
    _, kt = timed_steps(c, fp8_sparse, 2, 1, f"{w.name} option fp8 sparse layers")
    out["fp8_sparse_layer_us"] = round(avg_us(kt, "sparse_decode"), 2)
    out["fp8_append_conversion_us"] = round(avg_us(kt, "kv_fp8_convert"), 2)

    # the full layer reading the FP8 copy too (appending the token to it)
    def fp8_full():
        hs.decode_step(st["q_full"], st["kv_new"], kv, seq0, bound, top_k=w.top_k, window=w.window,
                       workspace=dec.ws_full, kv_fp8=copy)
    _, kt = timed_steps(c, fp8_full, 2, 1, f"{w.name} option fp8 full layer")
    fp8_bytes = sum(256.0 * w.Hkv * (L + 1) for L in lengths)
    out["fp8_full_layer_us"] = round(avg_us(kt, "decode_full"), 2)
    out["fp8_full_layer_roofline"] = hbm_roof(fp8_bytes, avg_us(kt, "decode_full"))
    out["fp8_full_layer_step_kernels_us"] = round(sum(t / n * 1e3 for n, t in kt.values()), 2)
    for flag, key, kernels in ((hs.HS_FLAG_BLOCK_SELECT, "block_select_us", ("block_max", "select_blocks")),
                               (hs.HS_FLAG_HEAD_UNION, "head_union_select_us",
                                ("decode_score", "select_decode", "head_union"))):
        shape = hs.make_shape(batch=len(lengths), n_q=1, n_kv=0, kv_capacity=kv.shape[2], q_heads=w.Hq,
                              kv_heads=w.Hkv, top_k=w.top_k, window=w.window, flags=flag)
        ws = _lib.alloc_workspace(_lib.workspace_size(_lib.HS_OP_DECODE_STEP, shape, bound), c.dev)
        call = lambda: hs.decode_step(st["q_full"], st["kv_new"], kv, seq0, bound, top_k=w.top_k, window=w.window,
                                      flags=flag, workspace=ws)
        _, kt = timed_steps(c, call, 1, 1, f"{w.name} option {key}")
        out[key] = round(sum(avg_us(kt, k) or 0.0 for k in kernels), 2)
        del ws
    del copy
    return out


def graph_ctx1m(c, pre, dec):
    """The 1M-context decode step replayed as one HIP graph (the headline runs
    it as eager calls)."""
    hs, torch, w = c.hs, c.torch, dec.w
    g = hs.DecodeStepGraph(pre.kv, batch=1, q_heads=w.Hq, sparse_layers=w.sparse_layers, top_k=w.top_k,
                           window=w.window)
    st = dec.data[0]
    g.q.copy_(st["q_full"])
    g.kv_new.copy_(st["kv_new"])
    for d, x in zip(g.q_sparse, st["q_sparse"]):
        d.copy_(x)
    g.seq_lens.copy_(dec.seqs[0])
    g.step(w.n_kv + 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(w.decode_steps):
        g.step(w.n_kv + 1)
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / w.decode_steps
    log(f"[bench] ctx1m decode step as one graph launch: {us:.1f} us")
    return round(us, 2)


BRIDGE_D_MODEL = 2048  # hidden width of the bridged self-decoder states (the pages give no width)


def kv_bridge_leg(c, head):
    """KV Bridging and the early-exit prefill on the 1M-token workload's
    chunk: with early exit the cross-decoder's prefill work for the chunk is
    only the bridge (its full-attention K/V rows from the self-decoder's
    hidden states); without it, the chunk also runs the full layer with
    selection and the sparse layers (the headline's prefill block). Reports
    both FLOP counts and times; the bridge is a bf16 GEMM priced against the
    matrix peak."""
    torch, hs, synth = c.torch, c.hs, c.synth
    w = synth.WORKLOADS["ctx1m"]
    d_model = BRIDGE_D_MODEL
    h = synth.randn_bf16((1, w.n_q, d_model), synth.seed_for(w.cid, 10), c.dev)
    wt = (synth.randn_bf16((w.Hkv, 2, 128, d_model), synth.seed_for(w.cid, 11), c.dev).float()
          / d_model ** 0.5).to(torch.bfloat16)
    kv = torch.empty((1, w.Hkv, w.n_q, 2, 128), dtype=torch.bfloat16, device=c.dev)
    ms, kt = timed_steps(c, lambda: hs.kv_bridge(h, wt, kv, w.n_q), 10, 2, "kv bridge over the ctx1m chunk")
    us = avg_us(kt, "kv_bridge")
    bridge_flops = 2.0 * w.n_q * d_model * w.Hkv * 2 * 128
    counts = prefill_counts(w)
    full_flops = counts["full_flops"] + w.sparse_layers * counts["sparse_flops_per_layer"] + bridge_flops
    out = {"d_model": d_model, "tokens": w.n_q, "bridge_us": round(us, 1),
           "bridge_roofline": mfma_roof(bridge_flops, us, "kv_bridge"),
           "prefill_flops_with_early_exit": bridge_flops, "prefill_flops_without_early_exit": full_flops,
           "flop_ratio": round(full_flops / bridge_flops, 1),
           "prefill_ms_with_early_exit": round(us * 1e-3, 3),
           "prefill_ms_without_early_exit": round(head["prefill_block_ms"] + us * 1e-3, 3)}
    del h, wt, kv
    torch.cuda.empty_cache()
    return out


def copy_ceiling(c):
    """Bytes moved per second (read + written) by a plain elementwise copy of
    2 GiB (torch's y = x * 1, one streaming kernel): the measured ceiling the
    decode rooflines are also given against."""
    torch = c.torch
    x = torch.ones(1 << 29, dtype=torch.float32, device=c.dev)
    y = torch.empty_like(x)
    torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = 0.0
    for _ in range(5):
        e0.record()
        torch.mul(x, 1.0, out=y)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, 2 * x.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del x, y
    torch.cuda.empty_cache()
    return round(best, 1)


def gather_ceilings(c):
    """Rates of the gather probe (the sparse layers' access pattern without
    their arithmetic) over random 512-byte token rows of buffers that stay in
    L2 (2 MiB), in the last-level cache (64 MiB, the size class of the 32K
    cache) and in HBM (2 GiB, the 1M-token cache). Bytes = 512 per gathered
    row; best of 5 launches of 2^22 rows."""
    import ctypes
    torch, _lib = c.torch, c._lib
    lib = _lib.load()
    out = {}
    n = 1 << 22
    per_wave = 640
    for label, nbytes in (("l2_2MiB", 2 << 20), ("llc_64MiB", 64 << 20), ("hbm_2GiB", 2 << 30)):
        rows = nbytes // 512
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=c.dev)
        g = torch.Generator(device=c.dev)
        g.manual_seed(0x4853)
        idx = torch.randint(0, rows, (n,), generator=g, device=c.dev, dtype=torch.int32)
        waves = -(-n // per_wave)
        res = torch.empty(((waves + 3) // 4) * 256, dtype=torch.int32, device=c.dev)
        call = lambda: _lib.check(lib.hs_gather_probe(_lib.ptr(src), rows, _lib.ptr(idx), n, per_wave, _lib.ptr(res),
                                                      _lib.stream_handle(c.dev)))
        call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = 0.0
        for _ in range(5):
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            best = max(best, n * 512 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        out[label] = round(best, 1)
        log(f"[bench] gather probe {label}: {best:.0f} GB/s")
        del src, idx, res
        torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------- counter runs

def traffic_probe(c, args):
    """For counter runs (rocprofv3 --pmc ... --kernel-include-regex "hs::|MulFunctor"):
    one launch of each kernel of
    the 1M-token step (full layer with selection, one sparse layer, one
    decode step with one sparse layer), the 32K full and sparse layers and one
    batched decode step, then a plain elementwise copy of known size (reads
    and writes 1 GiB) whose counter reading calibrates bytes per counter
    unit. Markers on stderr name each phase."""
    import dataclasses
    torch, hs, synth = c.torch, c.hs, c.synth
    # no needles: planting them launches ~1000 tiny kernels, which the counter
    # mode of the profiler has failed on, and they do not change the traffic
    w = dataclasses.replace(synth.WORKLOADS["ctx1m"], needles=0)
    case = synth.make_prefill_case(w, c.dev, kv_capacity=w.n_kv + 1, sparse_layers=1)
    q, kv, qs = case["q_full"], case["kv"], case["q_sparse"][0]
    o, lse, idx = hs.full_attn_select(q, kv, w.n_kv, top_k=w.top_k, window=w.window)
    hs.sparse_attn_reuse(qs, kv, idx, top_k=w.top_k, window=w.window, n_kv=w.n_kv)
    st = decode_inputs(c, w, 1)[0]
    seq = torch.tensor([w.n_kv + 1], dtype=torch.int32, device=c.dev)
    o2, _, idx2 = hs.decode_step(st["q_full"], st["kv_new"], kv, seq, w.n_kv + 1, top_k=w.top_k, window=w.window)
    hs.sparse_attn_reuse(st["q_sparse"][0], kv, idx2, top_k=w.top_k, window=w.window, seq_lens=seq)
    torch.cuda.synchronize()
    log("[bench] traffic probe: ctx1m layers done")
    del case, q, kv, qs, o, lse, idx, o2, idx2
    torch.cuda.empty_cache()
    w = dataclasses.replace(synth.WORKLOADS["prefill32k"], needles=0)
    case = synth.make_prefill_case(w, c.dev, sparse_layers=1)
    q, kv, qs = case["q_full"], case["kv"], case["q_sparse"][0]
    o, lse, idx = hs.full_attn_select(q, kv, w.n_kv, top_k=w.top_k, window=w.window)
    hs.sparse_attn_reuse(qs, kv, idx, top_k=w.top_k, window=w.window, n_kv=w.n_kv)
    torch.cuda.synchronize()
    log("[bench] traffic probe: prefill32k layers done")
    del case, q, kv, qs, o, lse, idx
    wd = synth.WORKLOADS["decode64"]
    lengths = synth.decode_lengths(wd)
    dcase = synth.make_decode_case(wd, c.dev, lengths, 1, sparse_layers=1)
    st = dcase["steps"][0]
    seq = torch.tensor([L + 1 for L in lengths], dtype=torch.int32, device=c.dev)
    o, lse, idx = hs.decode_step(st["q_full"], st["kv_new"], dcase["kv"], seq, max(lengths) + 1,
                                 top_k=wd.top_k, window=wd.window)
    hs.sparse_attn_reuse(st["q_sparse"][0], dcase["kv"], idx, top_k=wd.top_k, window=wd.window, seq_lens=seq)
    torch.cuda.synchronize()
    log("[bench] traffic probe: decode64 step done")
    del dcase, st, o, lse, idx
    torch.cuda.empty_cache()
    x = torch.ones(1 << 28, dtype=torch.float32, device=c.dev)
    torch.cuda.synchronize()
    y = x * 1.0  # one elementwise kernel: 1 GiB read, 1 GiB written
    torch.cuda.synchronize()
    log(f"[bench] traffic probe done: copy {x.numel() * 4} bytes read and written")
    del y


# Dispatch order of the traffic probe: (kernel-name pattern, workload label,
# library kernel name) for the dispatches whose bytes the summary records.
PROBE_DISPATCHES = [
    ("prefill_attn_kernel", "ctx1m", "prefill_attn"), ("flash_gather_kernel<8, true", "ctx1m", "sparse_prefill"),
    ("flash_gather_kernel<8, false, true", "ctx1m", "decode_full"),
    ("flash_gather_kernel<8, true", "ctx1m", "sparse_decode"),
    ("prefill_attn_kernel", "prefill32k", "prefill_attn"),
    ("flash_gather_kernel<8, true", "prefill32k", "sparse_prefill"),
    ("flash_gather_kernel<8, false, true", "decode64", "decode_full"),
    ("flash_gather_kernel<8, true", "decode64", "sparse_decode"),
]


def summarize_counters(fetch_csv, write_csv):
    """Turns the FETCH_SIZE and WRITE_SIZE counter CSVs of two traffic-probe
    runs into the lines the summary file records: bytes per dispatch, each
    counter scaled by what it reads for the probe's 1 GiB copy (last dispatch)."""
    import csv

    def rows(path):
        r = list(csv.DictReader(open(path)))
        r.sort(key=lambda x: int(x.get("Dispatch_Id", x.get("Dispatch_ID", 0))))
        return [(x["Kernel_Name"], float(x["Counter_Value"])) for x in r]
    fr, wr = rows(fetch_csv), rows(write_csv)
    fscale = (1 << 30) / (fr[-1][1] * 1024)
    wscale = (1 << 30) / (wr[-1][1] * 1024)
    print(f"calibration: FETCH_SIZE x {fscale:.3f}, WRITE_SIZE x {wscale:.3f} (1 GiB copy reads {fr[-1][1]:.0f} KiB, "
          f"writes {wr[-1][1]:.0f} KiB)")
    print(f"kernel-sources-sha256: {device_source_hash()}")
    pos = 0
    for pat, wl, kern in PROBE_DISPATCHES:
        while pos < len(fr) and pat not in fr[pos][0]:
            pos += 1
        if pos >= len(fr):
            break
        f = fr[pos][1] * 1024 * fscale
        wb = wr[pos][1] * 1024 * wscale
        print(f"| {kern} | {wl} | {fr[pos][1]:.0f} | {wr[pos][1]:.0f} | {f:.4g} | {wb:.4g} |")
        print(f"traffic {kern} {wl} {f + wb:.4e}")
        pos += 1


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--extra-steps", type=int, default=5, help="timed blocks of each extra prefill workload")
    ap.add_argument("--decode-steps", type=int, default=32, help="steps of the batched decode workload")
    ap.add_argument("--no-extras", action="store_true", help="the headline step only")
    ap.add_argument("--no-options", action="store_true", help="no option-path runs beside the default path")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--traffic-probe", action="store_true",
                    help="one launch of each counted kernel and a 1 GiB calibration copy, for counter runs")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the traffic lines of two --traffic-probe counter runs (no GPU needed)")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the hot path is single-GPU by design); --gpus {args.gpus} "
              f"is not supported", file=sys.stderr)
        sys.exit(2)

    c = Ctx()
    if args.traffic_probe:
        traffic_probe(c, args)
        return
    traffic = stored_traffic()
    log(f"[bench] traffic figures: {traffic[1]}")
    head, pre, dec = run_headline(c, args, traffic)
    w = c.synth.WORKLOADS["ctx1m"]
    extras = {}
    if not args.no_extras:
        extras["decode_ctx1m_graph_us_per_step"] = graph_ctx1m(c, pre, dec)
    case_host = None if args.no_cpu_baseline else host_case(pre)
    dec_data = dec.data
    del pre, dec
    c.torch.cuda.empty_cache()
    if not args.no_extras:
        extras["prefill32k"] = run_prefill_extra(c, args, "prefill32k", not args.no_options)
        extras["chunk128k"] = run_prefill_extra(c, args, "chunk128k", False)
        wd = c.synth.WORKLOADS["decode64"]
        extras["decode64"] = run_decode_extra(c, args, "decode64", c.synth.decode_lengths(wd), args.decode_steps,
                                              not args.no_options)
        extras["kv_bridge_early_exit"] = kv_bridge_leg(c, head)
        extras["copy_ceiling_GBs"] = copy_ceiling(c)
        extras["gather_ceiling_GBs"] = gather_ceilings(c)
        for key in ("decode_full_roofline", "decode_sparse_roofline"):
            r = extras["decode64"][key]
            r["frac_of_copy_ceiling"] = round(r["achieved"] / extras["copy_ceiling_GBs"], 4)
            head[key]["frac_of_copy_ceiling"] = round(head[key]["achieved"] / extras["copy_ceiling_GBs"], 4)
        memory_side(extras["prefill32k"]["sparse_prefill_layer"], traffic, "prefill32k")
    memory_side(head["sparse_prefill_layer"], traffic, "ctx1m")
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample of the 1M-token step")
        cpu = cpu_baseline(c, args, w, case_host, dec_data)
        log(f"[bench] oracle: {cpu}")

    line = {
        "metric": METRIC,
        "value": head.pop("value"),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "none (one GPU)",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "ctx1m", "batch": w.B, "cached_tokens": w.n_kv - w.n_q, "chunk_tokens": w.n_q,
                   "decode_steps": w.decode_steps, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": 128,
                   "top_k": w.top_k, "window": w.window, "sparse_layers": w.sparse_layers, "needles": w.needles,
                   "parallelism": "single-gpu"},
        "roofline": head.pop("roofline"),
        **head,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
