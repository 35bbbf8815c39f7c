/*
 * hysparse.h - C ABI of libhysparse: token-level hybrid sparse attention with
 * KV Reuse on AMD Instinct MI355X (gfx950).
 *
 * The operations follow these web pages (cited by title and section):
 *
 *  [HS2-cs]  "HySparse2 od Xiaomi zkracuje zpracovani dlouheho kontextu",
 *            section "Proc neni nutne znovu zpracovat cely dlouhy vstup"
 *            (KV Reuse paragraph): the sparse layers of a hybrid block take
 *            over the KV cache and the token selection of the full-attention
 *            layer before them; selection is per token; recent tokens are
 *            always included and share the cache with the selected ones.
 *  [DAIR]    "DAIR.AI weekly: HySparse2 ..." bullets "Two levels of KV
 *            sharing" and "Prefill exits early": same facts; a forced window
 *            of recent tokens replaces the sliding-window branch.
 *  [HS2-en]  "HySparse2 Cuts the Prefill Path for Tool-Using Agents", section
 *            "Tool Responses Turn Prefill Into the Bottleneck": prefill writes
 *            the KV cache that decoding reuses.
 *  [SSA-3.3] "Simplified Sparse Attention via Gist Tokens", section 3.3
 *            "Selective Unfolding and Hybrid Attention", paragraph "Grouped
 *            Unfolding for GQA": per-head top-k, united within a KV group.
 *  [SSA-3.6] "Simplified Sparse Attention via Gist Tokens", section 3.6
 *            "Kernel Design": sparse kernels compute exact attention over the
 *            kept keys; split partials merge by the log-sum-exp correction.
 *
 * Definitions used by every call (d = head_dim = 128, G = q_heads/kv_heads,
 * query head h reads KV head g = h / G):
 *   p          absolute position of a query row. Prefill/chunk: row t of n_q
 *              new rows sits at p = n_kv - n_q + t. Decode: p = seq_lens[b]-1.
 *   s_h(j)     scale * <q_h, k_g(j)>, scale = 1/sqrt(d) unless given.
 *   Win(p)     [max(0, p-W+1), p]: forced recent window, the query included.
 *   C(p)       {j : 0 <= j <= p-W}: top-k candidates (tokens older than the
 *              window).
 *   sigma(j)   max over the G heads of group g of s_h(j): selection score.
 *   I(p, g)    top_k members of C(p) by (sigma desc, j asc); all of C(p) when
 *              |C(p)| <= top_k.
 * The pages do not print the score, the window extent or the candidate set;
 * the definitions above are the readings this library implements.
 *
 * Conventions (all calls):
 *  - Element types: q, o, kv, kv_new are bf16 (raw uint16 storage);
 *    lse is fp32; idx and seq_lens are int32. All are device pointers.
 *  - Layouts (row-major, innermost last):
 *      q, o (prefill)   [batch][n_q][q_heads][d]
 *      q, o (decode)    [batch][q_heads][d]            (n_q == 1)
 *      lse              [batch][q_heads][n_q]           (may be NULL)
 *      idx              [batch][n_q][kv_heads][top_k]   ascending, -1 padded
 *      kv_new           [batch][kv_heads][2][d]         (K row, then V row)
 *      kv (cache)       element (b, g, t, K|V, e) at
 *                         b*kv_stride_b + g*kv_stride_h + t*kv_stride_t
 *                         + (V ? kv_v_offset : 0) + e
 *                       Strides of 0 select the default interleaved layout
 *                       [batch][kv_heads][kv_capacity][2][d]. Every K and V
 *                       row must start on a 16-byte boundary.
 *  - Ownership: the caller owns every buffer, including the workspace sized
 *    by hs_workspace_size. The library allocates no device memory and keeps
 *    no pointer after a call returns.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *    stream). All work is enqueued asynchronously on it; buffers must stay
 *    valid until the stream reaches them. No call synchronises the host.
 *  - Graph capture: with timing off, a call enqueues kernel launches only
 *    (no allocation, copy, memset, event or host wait), so calls may be
 *    captured into a HIP graph and replayed ([SSA-3.6] "End-to-end decode
 *    overhead": per-step launches dominate once kernels take microseconds).
 *    Host arguments (shape, max_seq_len, workspace) are fixed at capture;
 *    device data (q, kv, seq_lens, ...) is read at replay, so a captured
 *    decode step serves any lengths up to the max_seq_len it was captured
 *    with.
 *  - Errors: arguments are validated on the host before anything is
 *    enqueued, so a non-OK status means no work was queued (except
 *    HS_ERR_HIP, reported when a launch fails). A detail message for the
 *    calling thread's last failure is returned by hs_last_error(). No C++
 *    exception crosses this boundary. Faults inside kernels surface at the
 *    caller's next synchronisation, as for any HIP kernel.
 *  - Device: the current HIP device must be gfx950, else HS_ERR_UNSUPPORTED.
 *  - Inputs must be finite; NaN or Inf inputs give unspecified results.
 *  - Calls are reentrant; concurrent calls need separate workspaces.
 */
#ifndef HYSPARSE_H
#define HYSPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HS_VERSION 10000 /* major*10000 + minor*100 + patch */

typedef enum {
  HS_OK = 0,
  HS_ERR_INVALID_ARG = 1, /* bad shape, pointer, alignment or size         */
  HS_ERR_UNSUPPORTED = 2, /* device is not gfx950, or an unsupported shape  */
  HS_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required    */
  HS_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed    */
  HS_ERR_INTERNAL = 5
} hs_status;

typedef enum {
  HS_OP_FULL_ATTN_SELECT = 0,
  HS_OP_SPARSE_ATTN_REUSE = 1,
  HS_OP_DECODE_STEP = 2
} hs_op;

/* hs_shape.flags */
#define HS_FLAG_EXACT_RESCAN 1u /* every selection row takes the exact
                                   rescan path instead of the sampled
                                   threshold filter (testing hook; same
                                   results, slower) */
#define HS_FLAG_PROB_SCORE 2u   /* selection score sigma'(j) = max over the
                                   group's heads h of s_h(j) - lse_h, lse_h
                                   the natural-log softmax denominator of
                                   head h over keys 0..p: the log of the
                                   largest attention probability the group
                                   gives token j (the pages leave the score
                                   open; this is the softmax-normalised
                                   alternative to the logit default). Needs
                                   the layer's lse first, so the selection
                                   runs as its own pass after attention
                                   (prefill: a QK-only pass; decode: a
                                   second read of the K rows). Affects
                                   hs_full_attn_select and hs_decode_step;
                                   lse may still be NULL (kept in the
                                   workspace). */
/* Block-level selection, the choice that token-level selection replaces
   ([HS2-cs] section "Proc neni nutne znovu zpracovat cely dlouhy vstup";
   [DAIR] bullet "Prefill exits early"), kept as an ablation: C(p) is cut into aligned
   blocks of 64 tokens, a block scores the largest sigma of its candidates,
   the top top_k/64 blocks (ties: lower block first) are taken whole and
   written as their tokens, ascending, -1 padded (the last block of C(p) may
   be partial). Needs top_k % 64 == 0 (else HS_ERR_INVALID_ARG); not
   combined with HS_FLAG_PROB_SCORE (HS_ERR_UNSUPPORTED). Read by
   hs_full_attn_select and hs_decode_step. */
#define HS_FLAG_BLOCK_SELECT 8u
/* Union of per-head top-k sets, the grouped-unfolding rule for GQA
   ([SSA-3.3] "Grouped Unfolding for GQA"): each query head of a group ranks
   C(p) by its own scaled logit and keeps its top top_k; the group's row is
   the union of the G sets, ascending, in a row of G * top_k entries padded
   with -1. With this flag, idx of hs_full_attn_select and hs_decode_step is
   [..][Hkv][G * top_k], and hs_sparse_attn_reuse, given the same flag and
   top_k, reads rows of that length. Prefill runs the layer as G passes of
   one head per group (outputs and lse unchanged up to rounding order);
   decode adds one pass over the K rows for the heads' scores. Not combined
   with HS_FLAG_PROB_SCORE or HS_FLAG_BLOCK_SELECT (HS_ERR_UNSUPPORTED). */
#define HS_FLAG_HEAD_UNION 16u
#define HS_FLAG_FP8_KV 4u       /* hs_sparse_attn_reuse and hs_decode_step
                                   read keys and values from the FP8 copy
                                   of the cache made by hs_kv_fp8_convert
                                   (kv then points to that copy; strides
                                   must be 0). The pages leave the cache
                                   precision open ([DAIR] "Cheaper at 1M
                                   tokens" gives the cache size only): this
                                   halves the bytes read. hs_decode_step
                                   then writes kv_new into the copy,
                                   quantised with the stored scales of its
                                   KV head (values beyond the range
                                   saturate), and leaves any bf16 cache
                                   alone; it takes the logit score (token
                                   or block level), not HS_FLAG_PROB_SCORE
                                   or HS_FLAG_HEAD_UNION (HS_ERR_UNSUPPORTED).
                                   Rejected by hs_full_attn_select. */

typedef struct {
  int32_t batch;       /* B >= 1                                            */
  int32_t n_q;         /* query rows per sequence; 1 for decode calls       */
  int32_t n_kv;        /* prefill: keys visible to the last query row       */
  int32_t kv_capacity; /* token slots per (b, kv head) in the cache         */
  int32_t q_heads;     /* Hq; Hq % Hkv == 0 and Hq / Hkv in {1,2,4,8}       */
  int32_t kv_heads;    /* Hkv >= 1                                          */
  int32_t head_dim;    /* must be 128                                       */
  int32_t top_k;       /* k >= 0                                            */
  int32_t window;      /* W >= 1 (the window contains the query itself)     */
  float scale;         /* 0 selects 1/sqrt(head_dim)                        */
  int64_t kv_stride_b; /* elements; 0 with the three below = default layout */
  int64_t kv_stride_h;
  int64_t kv_stride_t;
  int64_t kv_v_offset;
  uint32_t flags;      /* HS_FLAG_*                                         */
  uint32_t reserved;   /* must be 0                                         */
} hs_shape;

/* Workspace bytes that `op` needs for shape `s`. For HS_OP_DECODE_STEP and
 * for decode calls of HS_OP_SPARSE_ATTN_REUSE, max_seq_len bounds every
 * seq_lens[b] of the calls the workspace will serve; it is ignored for
 * prefill. Writes the size to *bytes (0 is a valid answer). */
hs_status hs_workspace_size(hs_op op, const hs_shape* s, int32_t max_seq_len,
                            size_t* bytes);

/* Full-attention layer of a hybrid block, prefill or chunked prefill
 * ([HS2-cs], [DAIR], [HS2-en]). For every batch b, query row t and query
 * head h: o = softmax_j(s_h(j)) v_g(j) over 0 <= j <= p (causal GQA
 * attention) and lse = log sum_j exp(s_h(j)). For every (b, t, g): idx row =
 * I(p, g) in ascending order, -1 padded to top_k.
 *   q    bf16 [B][n_q][Hq][d]; kv: the cache, rows [0, n_kv) valid (the
 *        chunk's own K/V rows already written at [n_kv-n_q, n_kv)).
 *   o    bf16 [B][n_q][Hq][d]; lse fp32 [B][Hq][n_q] or NULL;
 *   idx  int32 [B][n_q][Hkv][top_k] (may be NULL only when top_k == 0).
 * Requires 1 <= n_q <= n_kv <= kv_capacity. */
hs_status hs_full_attn_select(const hs_shape* s, const void* q, const void* kv,
                              void* o, float* lse, int32_t* idx, void* ws,
                              size_t ws_bytes, void* stream);

/* Diagnostics of the token-level selection of hs_full_attn_select (not
 * needed to use the library). After a call with workspace ws (and once the
 * stream has reached it), the workspace holds, at these byte offsets from ws:
 *   defer_count_off   uint32: rows the one-wave selection queued for the
 *                     block-wide path (candidate count outside [k, buffer],
 *                     more candidates than one wave holds, or a forced rescan);
 *   defer_rows_off    int32[that count]: those rows, as (b*n_q + t)*Hkv + g,
 *                     in no particular order;
 *   rescan_count_off  uint32: queued rows whose scores were recomputed
 *                     exactly because the candidate buffer could not be
 *                     trusted (too few or too many entries).
 * Returns HS_ERR_UNSUPPORTED when the shape's selection keeps no such record
 * (top_k == 0, HS_FLAG_BLOCK_SELECT, HS_FLAG_HEAD_UNION). Runs on the host
 * only; reads nothing. */
hs_status hs_select_diagnostics(const hs_shape* s, size_t* defer_rows_off,
                                size_t* defer_count_off,
                                size_t* rescan_count_off);

/* One sparse layer of a hybrid block ([HS2-cs], [DAIR]): reuses the full
 * layer's KV cache and selection. For every row and head h (group g):
 * o = softmax over j in S of s_h(j), weighted sum of v_g(j), where
 * S = {valid entries of the idx row} U Win(p). Writes nothing to the cache.
 *   Prefill: seq_lens == NULL; q, o [B][n_q][Hq][d]; idx [B][n_q][Hkv][k];
 *            p = n_kv - n_q + t.
 *   Decode:  seq_lens != NULL (device int32 [B], context length including
 *            the newest token), n_q == 1; q, o [B][Hq][d]; idx [B][Hkv][k];
 *            p = seq_lens[b] - 1.
 * Every valid idx entry must lie in C(p) and rows must hold no duplicates
 * (as produced by hs_full_attn_select / hs_decode_step); entries < 0 are
 * padding. */
hs_status hs_sparse_attn_reuse(const hs_shape* s, const void* q,
                               const void* kv, const int32_t* idx,
                               const int32_t* seq_lens, void* o, void* ws,
                               size_t ws_bytes, void* stream);

/* Full-attention layer for one decode step over a batch ([HS2-en],
 * [HS2-cs]): writes kv_new[b] into cache slot seq_lens[b]-1, attends over
 * [0, seq_lens[b]) for each query head, and selects once: idx[b][g] =
 * I(seq_lens[b]-1, g), which the following sparse layers pass unchanged to
 * hs_sparse_attn_reuse (decode form).
 *   q       bf16 [B][Hq][d];  kv_new bf16 [B][Hkv][2][d];  kv: the cache.
 *   seq_lens device int32 [B], 1 <= seq_lens[b] <= max_seq_len
 *           <= kv_capacity (host-side bound used for launch sizing).
 *   o       bf16 [B][Hq][d]; lse fp32 [B][Hq] or NULL;
 *   idx     int32 [B][Hkv][top_k]. */
hs_status hs_decode_step(const hs_shape* s, const void* q, const void* kv_new,
                         void* kv, const int32_t* seq_lens,
                         int32_t max_seq_len, void* o, float* lse,
                         int32_t* idx, void* ws, size_t ws_bytes,
                         void* stream);

/* KV Bridging ([HS2-cs] section "Proc neni nutne znovu zpracovat cely dlouhy
 * vstup": the cross-decoder's full-attention layers build their keys and
 * values from the self-decoder's hidden states; [DAIR] bullets "Two levels
 * of KV sharing" and "Prefill exits early": since every cross-decoder cache
 * comes from the self-decoder, prefill can stop once the self-decoder is
 * done). Writes, for every batch entry b, chunk row t < n_q and KV head g,
 * cache row p = n_kv - n_q + t:
 *   K_g(p) = h[b][t] W[g][0]^T,   V_g(p) = h[b][t] W[g][1]^T
 * (a linear projection with no bias, norm or position rotation: the pages
 * name only its input and output), fp32 accumulation, stored as bf16 rounded
 * to nearest even.
 *   hidden  bf16 [B][n_q][d_model], the self-decoder's hidden states of the
 *           chunk's tokens;
 *   w_kv    bf16 [Hkv][2][128][d_model], the projection rows (index 0: keys,
 *           1: values) of each KV head, laid out as a linear layer's weight;
 *   kv      the cache, in the layout of s (strides allowed); only the rows
 *           above are written.
 * Uses s->batch, n_q, n_kv, kv_capacity, kv_heads, the strides (q_heads,
 * top_k and window are validated as for the other calls but not used).
 * Needs 1 <= n_q <= n_kv <= kv_capacity and d_model a multiple of 64 in
 * [64, 65536] (else HS_ERR_UNSUPPORTED). A decode step bridges its token by
 * treating kv_new [B][Hkv][2][128] as a cache of capacity 1 (n_q = n_kv = 1).
 * Runs on `stream`; errors as for the other calls. */
hs_status hs_kv_bridge(const hs_shape* s, const void* hidden, int32_t d_model,
                       const void* w_kv, void* kv, void* stream);

/* hs_decode_step without a caller workspace, for callers that cannot
 * allocate device memory or manage a workspace (code under HIP graph
 * capture, tight serving loops, hosts that forbid allocation): identical
 * arguments and results except ws, which is the library's own scratch, a
 * static device array of 64 MiB per GPU (held from the library's first use
 * on that GPU until the process ends). Calls whose step needs more scratch
 * than that (hs_workspace_size(HS_OP_DECODE_STEP, s, max_seq_len) > 64 MiB;
 * e.g. a single sequence of up to about a million tokens fits, 64
 * sequences of 256K tokens do not) fail with HS_ERR_WORKSPACE before
 * anything is enqueued. The call allocates nothing; its first call on a
 * device looks up the scratch address there. Every call on one GPU shares
 * that GPU's scratch, which keeps the last call's contents (the step needs
 * none of it cleared): calls that may overlap on one GPU (other streams, or
 * other threads) race and must be serialised by the caller. */
hs_status hs_decode_step_noalloc(const hs_shape* s, const void* q,
                                 const void* kv_new, void* kv,
                                 const int32_t* seq_lens, int32_t max_seq_len,
                                 void* o, float* lse, int32_t* idx,
                                 void* stream);

/* Diagnostics: per-kernel timing. While enabled (on != 0), every kernel the
 * library launches is bracketed by a pair of HIP events recorded on the
 * call's stream, so durations are those of the kernels themselves on the
 * stream they run on. Accumulates per kernel name until read. Process-wide;
 * enabling costs two event records per launch. */
typedef struct {
  char name[48];     /* kernel name, e.g. "prefill_attn"                     */
  int64_t launches;  /* launches timed since the last read                   */
  double total_ms;   /* summed durations                                     */
} hs_kernel_time;

hs_status hs_timing_enable(int32_t on);

/* Waits for every recorded event, writes up to `max` entries to `out`,
 * sets *count to the number of distinct kernels, and clears the totals. */
hs_status hs_timing_read(hs_kernel_time* out, int32_t max, int32_t* count);

/* FP8 (e4m3) copy of a bf16 cache for the sparse layers (HS_FLAG_FP8_KV).
 *
 * Layout of the copy (caller-owned device buffer of hs_kv_fp8_size bytes,
 * 16-byte aligned): codes [batch][kv_heads][kv_capacity][2][128] bytes (K row
 * then V row of each token), then [batch][kv_heads][2] uint32 (scratch of
 * the conversion), then [batch][kv_heads][2] float scales 2^e_K, 2^e_V.
 * A stored value x of KV head (b, g) is e4m3(clamp(x / 2^e, -448, 448)),
 * rounded to nearest even, and reads back as code * 2^e: every such value is
 * a bf16 value, so the sparse kernels compute on it exactly.
 *
 * hs_kv_fp8_size: bytes of the copy for s->batch, kv_heads, kv_capacity.
 * hs_kv_fp8_convert:
 *   seq_lens == NULL (prefill form): per (b, g), e_K and e_V are the smallest
 *     exponents with max |x| <= 448 * 2^e over rows [0, n_kv) (0 for an
 *     all-zero head), stored, and rows [0, n_kv) are converted; needs
 *     1 <= n_kv <= kv_capacity.
 *   seq_lens != NULL (decode form, device int32 [batch]): row seq_lens[b]-1
 *     of every (b, g) is converted with the stored scales (values beyond the
 *     range saturate at +-448 * 2^e); call it after hs_decode_step appended
 *     the row.
 *   kv: the bf16 cache in the layout of hs_shape (strides allowed). Runs on
 *   `stream`; errors as for the other calls. */
hs_status hs_kv_fp8_size(const hs_shape* s, size_t* bytes);
hs_status hs_kv_fp8_convert(const hs_shape* s, const void* kv, void* kv8, const int32_t* seq_lens, void* stream);

/* Diagnostics: gather-rate probe (not needed to use the library). Reads
 * the 512-byte rows src[idx[i]] (i < n; K half then V half, the layout of one
 * token of one KV head in the default cache) with the memory access pattern
 * of the sparse layers' gathers and none of their arithmetic, per_wave keys
 * per wave (1..2048, staged in LDS like the sparse layers' key lists), and writes one folded word per lane to out (uint32 [64 * ceil(n /
 * per_wave)], rounded up to whole 4-wave blocks). Every idx[i] must lie in
 * [0, src_rows); rows beyond src_rows * 512 bytes read as zero. Measures the
 * rate at which the chip can gather rows from a buffer of a given size (L2,
 * last-level cache or HBM resident). Runs on `stream`. */
hs_status hs_gather_probe(const void* src, int64_t src_rows, const int32_t* idx, int64_t n, int32_t per_wave,
                          uint32_t* out, void* stream);

/* Static English name of a status code. */
const char* hs_status_string(hs_status st);

/* Detail message of the calling thread's most recent failed call ("" if
 * none). Valid until the thread's next library call. */
const char* hs_last_error(void);

/* HS_VERSION of the built library. */
int32_t hs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HYSPARSE_H */
