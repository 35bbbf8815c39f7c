// C ABI of libhysparse: argument validation, workspace planning and launch
// orchestration. Every argument is checked on the host before anything is
// enqueued; the library allocates no device memory and never synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/hysparse.h"
#include "hs_kernels.hpp"

namespace {

thread_local std::string g_last_error;

hs_status fail(hs_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
hs_status fail(hs_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

hs_status ok() {
  g_last_error.clear();
  return HS_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// ------------------------------------------------------------ device check

std::mutex g_arch_mu;
std::vector<int> g_arch_state;  // per device: 0 unknown, 1 ok, 2 unsupported

hs_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(HS_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_arch_mu);
  if ((int)g_arch_state.size() <= dev) g_arch_state.resize(dev + 1, 0);
  if (g_arch_state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(HS_ERR_HIP, "hipGetDeviceProperties failed");
    g_arch_state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (g_arch_state[dev] == 2) return fail(HS_ERR_UNSUPPORTED, "device %d is %s, libhysparse needs gfx950", dev, prop.gcnArchName);
  }
  if (g_arch_state[dev] == 2) return fail(HS_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return HS_OK;
}

// ------------------------------------------------------------ shape checks

struct Layout {
  int64_t sb, sh, st, voff;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hs_status validate_common(const hs_shape* s, Layout* lay) {
  if (!s) return fail(HS_ERR_INVALID_ARG, "shape is NULL");
  if (s->reserved != 0) return fail(HS_ERR_INVALID_ARG, "reserved must be 0");
  if (s->batch < 1) return fail(HS_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", s->batch);
  if (s->head_dim != 128) return fail(HS_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", s->head_dim);
  if (s->kv_heads < 1 || s->q_heads < 1 || s->q_heads % s->kv_heads != 0)
    return fail(HS_ERR_INVALID_ARG, "q_heads (%d) must be a positive multiple of kv_heads (%d)", s->q_heads, s->kv_heads);
  const int G = s->q_heads / s->kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(HS_ERR_UNSUPPORTED, "q_heads/kv_heads must be 1, 2, 4 or 8 (got %d)", G);
  if (s->top_k < 0 || s->top_k > hs::kMaxTopK)
    return fail(HS_ERR_INVALID_ARG, "top_k must be in [0, %d] (got %d)", hs::kMaxTopK, s->top_k);
  if (s->window < 1) return fail(HS_ERR_INVALID_ARG, "window must be >= 1 (got %d)", s->window);
  if (s->kv_capacity < 1) return fail(HS_ERR_INVALID_ARG, "kv_capacity must be >= 1");
  if (!(s->scale >= 0.f) || std::isinf(s->scale)) return fail(HS_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if ((s->flags & ~(HS_FLAG_EXACT_RESCAN | HS_FLAG_PROB_SCORE | HS_FLAG_FP8_KV | HS_FLAG_BLOCK_SELECT |
                    HS_FLAG_HEAD_UNION)) != 0)
    return fail(HS_ERR_INVALID_ARG, "unknown flags 0x%x", s->flags);
  if ((s->flags & HS_FLAG_HEAD_UNION) && (s->flags & (HS_FLAG_PROB_SCORE | HS_FLAG_BLOCK_SELECT)))
    return fail(HS_ERR_UNSUPPORTED, "the per-head union uses token-level logit scores");
  if ((s->flags & HS_FLAG_BLOCK_SELECT) && s->top_k % 64 != 0)
    return fail(HS_ERR_INVALID_ARG, "block-level selection needs top_k %% 64 == 0 (got %d)", s->top_k);
  if ((s->flags & HS_FLAG_BLOCK_SELECT) && (s->flags & HS_FLAG_PROB_SCORE))
    return fail(HS_ERR_UNSUPPORTED, "block-level selection uses the logit score");
  if ((s->flags & HS_FLAG_FP8_KV) && (s->kv_stride_b || s->kv_stride_h || s->kv_stride_t || s->kv_v_offset))
    return fail(HS_ERR_INVALID_ARG, "the FP8 cache copy has a fixed layout: strides must be 0");
  Layout l;
  if (s->kv_stride_b == 0 && s->kv_stride_h == 0 && s->kv_stride_t == 0 && s->kv_v_offset == 0) {
    l.st = 2 * 128;
    l.voff = 128;
    l.sh = (int64_t)s->kv_capacity * l.st;
    l.sb = (int64_t)s->kv_heads * l.sh;
  } else {
    l.sb = s->kv_stride_b;
    l.sh = s->kv_stride_h;
    l.st = s->kv_stride_t;
    l.voff = s->kv_v_offset;
    if (l.sb < 0 || l.sh < 0 || l.st <= 0 || l.voff < 0)
      return fail(HS_ERR_INVALID_ARG, "cache strides must be non-negative (t-stride positive)");
    if (l.sb % 8 || l.sh % 8 || l.st % 8 || l.voff % 8)
      return fail(HS_ERR_INVALID_ARG, "cache strides and V offset must be multiples of 8 elements (16-byte rows)");
  }
  // Rows of one (b, g) slab are addressed with 32-bit element offsets.
  if ((double)l.st * (double)s->kv_capacity + (double)l.voff + 128.0 > 2147483647.0)
    return fail(HS_ERR_UNSUPPORTED, "one (batch, kv head) cache slab must span < 2^31 elements");
  *lay = l;
  return HS_OK;
}

float eff_scale(const hs_shape* s) { return s->scale == 0.f ? 1.0f / std::sqrt((float)s->head_dim) : s->scale; }

bool head_union(const hs_shape* s) { return (s->flags & HS_FLAG_HEAD_UNION) && s->top_k > 0; }

// The sparse layers see an index row of G * top_k entries under the per-head
// union: their shape is the caller's with that row length.
hs_shape sparse_shape(const hs_shape* s) {
  hs_shape t = *s;
  if (head_union(s)) t.top_k = s->top_k * (s->q_heads / s->kv_heads);
  t.flags &= ~HS_FLAG_HEAD_UNION;
  return t;
}

// Prefill under the per-head union: the layer runs as G passes of a one-head-
// per-group layer (query heads g*G + r for pass r), whose shape this is.
hs_shape union_pass_shape(const hs_shape* s) {
  hs_shape t = *s;
  t.q_heads = s->kv_heads;
  t.flags &= ~HS_FLAG_HEAD_UNION;
  return t;
}

hs::KvView kv_view(const void* kv, const Layout& l) {
  return hs::KvView{static_cast<const uint16_t*>(kv), l.sb, l.sh, (int32_t)l.st, (int32_t)l.voff};
}

// ------------------------------------------------------------ plans

struct PrefillPlan {
  int64_t rows = 0;
  int cap = 0;
  int stride = 1;
  int max_samples = 0;
  bool sample = false;
  size_t off_theta = 0, off_counts = 0, off_bs = 0, off_bj = 0, off_samples = 0, off_stat = 0, off_defer = 0,
         off_lse = 0, off_blk = 0, total = 0;
  bool prob = false;  // probability score: selection pass after attention, lse kept here
  bool block = false; // block-level selection: block scores at off_blk
  int blk_stride = 0;
};

struct UnionPlan {
  size_t inner = 0, off_q = 0, off_o = 0, off_lse = 0, off_lists = 0, total = 0;
};
PrefillPlan plan_prefill(const hs_shape* s);
UnionPlan plan_union_prefill(const hs_shape* s) {
  UnionPlan u;
  const hs_shape si = union_pass_shape(s);
  const int G = s->q_heads / s->kv_heads;
  const int64_t rows = (int64_t)s->batch * s->n_q * s->kv_heads;
  size_t o = align_up(plan_prefill(&si).total);
  u.inner = o;
  u.off_q = o;
  o = align_up(o + (size_t)rows * 128 * 2);
  u.off_o = o;
  o = align_up(o + (size_t)rows * 128 * 2);
  u.off_lse = o;
  o = align_up(o + (size_t)rows * 4);
  u.off_lists = o;
  o = align_up(o + (size_t)G * rows * s->top_k * 4);
  u.total = o;
  return u;
}

PrefillPlan plan_prefill(const hs_shape* s) {
  PrefillPlan p;
  p.rows = (int64_t)s->batch * s->n_q * s->kv_heads;
  if (s->top_k == 0) return p;
  const int64_t max_cand = std::max<int64_t>(0, (int64_t)s->n_kv - s->window + 1);
  if (s->flags & HS_FLAG_BLOCK_SELECT) {  // block scores only
    p.block = true;
    p.blk_stride = (int)std::max<int64_t>(1, (max_cand + 63) / 64);
    p.off_blk = 0;
    p.total = align_up((size_t)p.rows * p.blk_stride * 4);
    return p;
  }
  p.cap = (int)std::min<int64_t>(round_up(3 * (int64_t)s->top_k + 256, 64), std::max<int64_t>(max_cand, 1));
  p.sample = max_cand > p.cap;
  // about 64 expected samples among a row's top k (stride k/64), but no more
  // than 16384 samples per row: the threshold block holds that many in registers
  p.stride = (int)std::max<int64_t>({1, s->top_k / 64, (max_cand + 16383) / 16384});
  p.max_samples = p.sample ? (int)round_up((max_cand + p.stride - 1) / p.stride, 64) : 0;
  size_t o = 0;
  p.off_theta = o;
  o = align_up(o + (size_t)p.rows * 4);
  p.off_counts = o;
  o = align_up(o + (size_t)p.rows * 4);
  p.off_bs = o;
  o = align_up(o + (size_t)p.rows * p.cap * 4);
  p.off_bj = o;
  o = align_up(o + (size_t)p.rows * p.cap * 4);
  p.off_samples = o;
  o = align_up(o + (size_t)p.rows * p.max_samples * 4);
  p.off_stat = o;
  o = align_up(o + 4);
  p.off_defer = o;  // queued rows of the selection, then their count and the rescan count
  o = align_up(o + (size_t)p.rows * 4 + 8);
  p.prob = (s->flags & HS_FLAG_PROB_SCORE) != 0;
  if (p.prob) {
    p.off_lse = o;
    o = align_up(o + (size_t)s->batch * s->q_heads * s->n_q * 4);
  }
  p.total = o;
  return p;
}

struct DecodePlan {
  int splits = 1, split_len = 32;
  bool in_block = false;  // sparse decode: splits merged inside the block
  int64_t sigma_stride = 0;
  int sel_slices = 0;     // sliced selection (0: one block per row)
  bool prob = false;      // probability score: score pass after the full layer
  bool block = false;     // block-level selection from the score rows
  bool head_union = false; // per-head score rows and lists, then their union
  int blk_stride = 0;
  size_t off_sigma = 0, off_part = 0, off_theta = 0, off_samp = 0, off_segcnt = 0, off_segkey = 0, off_segidx = 0,
         off_lse = 0, off_blk = 0, off_hidx = 0, total = 0;
};

// Splits a per-(b, g) key stream of up to `nkeys` keys so that the grid holds
// roughly `waves` waves, in multiples of 32 keys. Many short splits keep the
// last round of resident waves small relative to the whole.
void plan_splits(int64_t bg, int64_t nkeys, int* splits, int* split_len, int64_t waves = 8192) {
  const int64_t target = std::max<int64_t>(1, (waves + bg - 1) / bg);
  int64_t len = round_up(std::max<int64_t>(1, (nkeys + target - 1) / target), 32);
  len = std::max<int64_t>(len, 32);
  *split_len = (int)len;
  *splits = (int)std::max<int64_t>(1, (nkeys + len - 1) / len);
}

// SIMDs of the chip (256 CUs x 4): decode grids are sized in these.
constexpr int64_t kChipSimds = 1024;

DecodePlan plan_decode_full(const hs_shape* s, int max_seq_len) {
  DecodePlan p;
  const int G = s->q_heads / s->kv_heads;
  const int64_t bg = (int64_t)s->batch * s->kv_heads;
  // Splits of about kFullSplitKeys keys (measured best both for 64 sequences
  // of 64K-256K tokens and for one sequence of 1M), but at least two waves
  // per SIMD over the batch, and no more splits than the merge takes.
  constexpr int64_t kFullSplitKeys = 2048, kMinWaves = 2 * kChipSimds, kMaxSplits = 4096;
  int64_t splits = std::max((max_seq_len + kFullSplitKeys - 1) / kFullSplitKeys, (kMinWaves + bg - 1) / bg);
  splits = std::min(splits, kMaxSplits);
  int64_t len = std::max<int64_t>(32, round_up((max_seq_len + splits - 1) / splits, 32));
  // an odd multiple of 32 keys: split starts a power-of-two stride apart
  // (1 MiB at 2048 keys) cost ~12% of the single-sequence 1M-context stream
  if ((len / 32) % 2 == 0) len += 32;
  p.split_len = (int)len;
  p.splits = (int)((max_seq_len + len - 1) / len);
  p.sigma_stride = round_up(max_seq_len, 64);
  // score rows: one per (b, g), or one per query head under the per-head union
  p.head_union = head_union(s);
  const int64_t sel_rows = p.head_union ? (int64_t)s->batch * s->q_heads : bg;
  size_t o = 0;
  p.off_sigma = o;
  o = align_up(o + (s->top_k > 0 ? (size_t)sel_rows * p.sigma_stride * 4 : 0));
  p.off_part = o;
  o = align_up(o + (size_t)bg * p.splits * G * (128 + 2) * 4);
  // Rows longer than one block's registers hold are selected in slices spread
  // over the chip (a threshold block per row, a filter block per slice of a
  // row, a final block per row); survivors get room for a whole slice each
  // (no overflow). With one block per row instead, even 256 rows of 64K-256K
  // candidates left the chip mostly idle (215 us for 0.22 GB of score rows).
  const int64_t max_cand = (int64_t)max_seq_len - s->window;
  if (s->top_k > 0 && !(s->flags & HS_FLAG_BLOCK_SELECT) && max_cand > hs::kSelRegKeys) {
    const int64_t ns = (max_cand + hs::kDecSlice - 1) / hs::kDecSlice;
    if (ns <= hs::kMaxDecSlices) p.sel_slices = (int)ns;
  }
  if (p.sel_slices > 0) {
    const size_t seg = (size_t)sel_rows * p.sel_slices;
    p.off_theta = o;
    o = align_up(o + (size_t)sel_rows * 4);
    p.off_samp = o;
    o = align_up(o + (size_t)sel_rows * hs::kDecSamples * 4);
    p.off_segcnt = o;
    o = align_up(o + seg * 4);
    p.off_segkey = o;
    o = align_up(o + seg * hs::kDecSlice * 4);
    p.off_segidx = o;
    o = align_up(o + seg * hs::kDecSlice * 4);
  }
  p.prob = s->top_k > 0 && (s->flags & HS_FLAG_PROB_SCORE) != 0;
  if (p.prob) {
    p.off_lse = o;
    o = align_up(o + (size_t)s->batch * s->q_heads * 4);
  }
  if (p.head_union) {  // the heads' own top-k lists
    p.off_hidx = o;
    o = align_up(o + (size_t)sel_rows * s->top_k * 4);
  }
  p.block = s->top_k > 0 && (s->flags & HS_FLAG_BLOCK_SELECT) != 0;
  if (p.block) {
    p.blk_stride = (int)std::max<int64_t>(1, (max_cand + 64) / 64);
    p.off_blk = o;
    o = align_up(o + (size_t)bg * p.blk_stride * 4);
  }
  p.total = o;
  return p;
}


// Sparse decode: each (b, g) row gathers top_k + W keys. When the batch has
// at least a quarter as many rows as the chip has SIMDs, every row is split
// four ways over the waves of one block, which merge their partials in LDS
// (no workspace, no merge kernel); the split-per-wave grid then holds at
// least one long-running wave per SIMD, which measured faster than more,
// shorter waves (the per-wave start-up is paid once per 640 keys at
// decode64). Smaller batches split finer for about one wave per SIMD and
// merge in a separate kernel.
DecodePlan plan_decode_sparse(const hs_shape* s) {
  DecodePlan p;
  const int G = s->q_heads / s->kv_heads;
  const int64_t bg = (int64_t)s->batch * s->kv_heads;
  const int64_t ns = (int64_t)s->top_k + s->window;
  if (bg * 4 >= kChipSimds) {
    p.in_block = true;
    p.splits = 4;
    p.split_len = (int)round_up((ns + 3) / 4, 32);
    p.total = 0;
    return p;
  }
  plan_splits(bg, ns, &p.splits, &p.split_len, kChipSimds);
  p.off_part = 0;
  p.total = p.splits > 1 ? align_up((size_t)bg * p.splits * G * (128 + 2) * 4) : 0;
  return p;
}

// ------------------------------------------------------------ timing

struct TimingState {
  std::mutex mu;
  bool on = false;
  struct Rec {
    const char* name;
    hipEvent_t a, b;
  };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;
  std::map<std::string, std::pair<int64_t, double>> acc;
};
TimingState g_timing;

hipEvent_t take_event() {
  if (!g_timing.pool.empty()) {
    hipEvent_t e = g_timing.pool.back();
    g_timing.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` (which enqueues one kernel on stream s); with timing on, the
// kernel is bracketed by two events on the same stream.
template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
  bool on;
  {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    on = g_timing.on;
  }
  if (!on) return launch();
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    a = take_event();
    b = take_event();
  }
  if (!a || !b) return launch();
  // Event failures only cost this launch its timing record.
  (void)hipEventRecord(a, s);
  hipError_t e = launch();
  (void)hipEventRecord(b, s);
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.pending.push_back({name, a, b});
  return e;
}

#define HIP_TRY(expr)                                                                     \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess) return fail(HS_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

}  // namespace

extern "C" {

const char* hs_status_string(hs_status st) {
  switch (st) {
    case HS_OK: return "ok";
    case HS_ERR_INVALID_ARG: return "invalid argument";
    case HS_ERR_UNSUPPORTED: return "unsupported";
    case HS_ERR_WORKSPACE: return "workspace too small";
    case HS_ERR_HIP: return "HIP error";
    case HS_ERR_INTERNAL: return "internal error";
  }
  return "unknown status";
}

const char* hs_last_error(void) { return g_last_error.c_str(); }

hs_status hs_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.on = on != 0;
  return ok();
}

hs_status hs_timing_read(hs_kernel_time* out, int32_t max, int32_t* count) {
  if (!count || (max > 0 && !out)) return fail(HS_ERR_INVALID_ARG, "out/count is NULL");
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (auto& r : g_timing.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      return fail(HS_ERR_HIP, "timing event failed for %s", r.name);
    auto& a = g_timing.acc[r.name];
    a.first += 1;
    a.second += ms;
    g_timing.pool.push_back(r.a);
    g_timing.pool.push_back(r.b);
  }
  g_timing.pending.clear();
  int32_t n = 0;
  for (auto& kv : g_timing.acc) {
    if (n < max) {
      std::snprintf(out[n].name, sizeof out[n].name, "%s", kv.first.c_str());
      out[n].launches = kv.second.first;
      out[n].total_ms = kv.second.second;
    }
    ++n;
  }
  *count = n;
  g_timing.acc.clear();
  return ok();
}

int32_t hs_version(void) { return HS_VERSION; }

hs_status hs_workspace_size(hs_op op, const hs_shape* s, int32_t max_seq_len, size_t* bytes) {
  Layout lay;
  if (!bytes) return fail(HS_ERR_INVALID_ARG, "bytes is NULL");
  hs_status st = validate_common(s, &lay);
  if (st != HS_OK) return st;
  switch (op) {
    case HS_OP_FULL_ATTN_SELECT:
      if (s->n_q < 1 || s->n_kv < s->n_q) return fail(HS_ERR_INVALID_ARG, "need 1 <= n_q <= n_kv");
      *bytes = head_union(s) ? plan_union_prefill(s).total : plan_prefill(s).total;
      return ok();
    case HS_OP_SPARSE_ATTN_REUSE: {
      const hs_shape su = sparse_shape(s);
      *bytes = max_seq_len > 0 ? plan_decode_sparse(&su).total : 0;
      return ok();
    }
    case HS_OP_DECODE_STEP:
      if (max_seq_len < 1) return fail(HS_ERR_INVALID_ARG, "max_seq_len must be >= 1");
      *bytes = plan_decode_full(s, max_seq_len).total;
      return ok();
  }
  return fail(HS_ERR_INVALID_ARG, "unknown op %d", (int)op);
}

hs_status hs_full_attn_select(const hs_shape* s, const void* q, const void* kv, void* o, float* lse, int32_t* idx,
                              void* ws, size_t ws_bytes, void* stream) {
  Layout lay;
  hs_status st = validate_common(s, &lay);
  if (st != HS_OK) return st;
  if (s->n_q < 1 || s->n_kv < s->n_q || s->n_kv > s->kv_capacity)
    return fail(HS_ERR_INVALID_ARG, "need 1 <= n_q (%d) <= n_kv (%d) <= kv_capacity (%d)", s->n_q, s->n_kv, s->kv_capacity);
  if (s->flags & HS_FLAG_FP8_KV) return fail(HS_ERR_UNSUPPORTED, "the FP8 cache copy serves hs_sparse_attn_reuse only");
  if (!q || !kv || !o) return fail(HS_ERR_INVALID_ARG, "q, kv and o must be non-NULL");
  if (s->top_k > 0 && !idx) return fail(HS_ERR_INVALID_ARG, "idx must be non-NULL when top_k > 0");
  if (!aligned16(q) || !aligned16(kv) || !aligned16(o)) return fail(HS_ERR_INVALID_ARG, "q, kv and o must be 16-byte aligned");
  if ((lse && (reinterpret_cast<uintptr_t>(lse) & 3)) || (idx && (reinterpret_cast<uintptr_t>(idx) & 3)))
    return fail(HS_ERR_INVALID_ARG, "lse and idx must be 4-byte aligned");
  if (head_union(s)) {
    // G passes of the one-head-per-group layer (pass r: query heads g*G + r),
    // which give those heads' outputs, lse and own top-k lists; then the
    // union of each group's G lists [SSA-3.3 grouped unfolding].
    const UnionPlan up = plan_union_prefill(s);
    if (!ws || ws_bytes < up.total) return fail(HS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", up.total, ws_bytes);
    if (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) return fail(HS_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    st = check_device();
    if (st != HS_OK) return st;
    hipStream_t hst = static_cast<hipStream_t>(stream);
    char* w = static_cast<char*>(ws);
    const hs_shape si = union_pass_shape(s);
    const int G = s->q_heads / s->kv_heads;
    const int64_t bt = (int64_t)s->batch * s->n_q, rows = bt * s->kv_heads;
    uint16_t* qr = reinterpret_cast<uint16_t*>(w + up.off_q);
    uint16_t* orr = reinterpret_cast<uint16_t*>(w + up.off_o);
    float* lr = lse ? reinterpret_cast<float*>(w + up.off_lse) : nullptr;
    int32_t* lists = reinterpret_cast<int32_t*>(w + up.off_lists);
    for (int r = 0; r < G; ++r) {
      HIP_TRY(timed("head_slice", hst, [&] {
        return hs::launch_head_slice(static_cast<const uint16_t*>(q), qr, bt, s->kv_heads, G, r, true, hst);
      }));
      st = hs_full_attn_select(&si, qr, kv, orr, lr, lists + (size_t)r * rows * s->top_k, w, up.inner, stream);
      if (st != HS_OK) return st;
      HIP_TRY(timed("head_slice", hst, [&] {
        return hs::launch_head_slice(orr, static_cast<uint16_t*>(o), bt, s->kv_heads, G, r, false, hst);
      }));
      if (lse)
        HIP_TRY(timed("lse_scatter", hst, [&] {
          return hs::launch_lse_scatter(lr, lse, s->batch, s->kv_heads, G, r, s->n_q, hst);
        }));
    }
    hs::UnionParams un{};
    un.lists = lists; un.row_stride = s->top_k; un.head_stride = rows * s->top_k; un.G = G; un.k = s->top_k;
    un.B = s->batch; un.n_q = s->n_q; un.n_kv = s->n_kv; un.Hkv = s->kv_heads; un.window = s->window;
    un.seq_lens = nullptr; un.out = idx;
    HIP_TRY(timed("head_union", hst, [&] { return hs::launch_head_union(un, rows, hst); }));
    return ok();
  }
  const PrefillPlan plan = plan_prefill(s);
  if (plan.total > 0 && (!ws || ws_bytes < plan.total))
    return fail(HS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.total, ws_bytes);
  if (plan.total > 0 && (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)))
    return fail(HS_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  st = check_device();
  if (st != HS_OK) return st;

  hipStream_t hst = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  const float scale = eff_scale(s);
  const hs::KvView kvv = kv_view(kv, lay);
  const bool select = s->top_k > 0;
  float* theta = select ? reinterpret_cast<float*>(w + plan.off_theta) : nullptr;
  // probability score: attention first (its lse feeds the score), then the
  // sampled threshold and a QK-only candidate pass
  const bool prob = select && plan.prob;
  float* lse_buf = prob && !lse ? reinterpret_cast<float*>(w + plan.off_lse) : lse;
  if (select && plan.block) {
    hs::PrefillParams pp{};
    pp.q = static_cast<const uint16_t*>(q);
    pp.kv = kvv;
    pp.o = static_cast<uint16_t*>(o);
    pp.lse = lse;
    pp.B = s->batch; pp.n_q = s->n_q; pp.n_kv = s->n_kv; pp.Hq = s->q_heads; pp.Hkv = s->kv_heads; pp.window = s->window;
    pp.scale = scale;
    pp.select = 2;
    pp.blk_score = reinterpret_cast<float*>(w + plan.off_blk);
    pp.blk_stride = plan.blk_stride;
    HIP_TRY(timed("prefill_attn", hst, [&] { return hs::launch_prefill_attn(pp, hst); }));
    hs::BlockSelectParams bp{};
    bp.B = s->batch; bp.n_q = s->n_q; bp.n_kv = s->n_kv; bp.Hkv = s->kv_heads; bp.top_k = s->top_k; bp.window = s->window;
    bp.blk_score = pp.blk_score; bp.blk_stride = plan.blk_stride; bp.idx = idx;
    HIP_TRY(timed("select_blocks", hst, [&] { return hs::launch_select_blocks(bp, plan.rows, hst); }));
    return ok();
  }

  hs::PrefillParams pp{};
  pp.q = static_cast<const uint16_t*>(q);
  pp.kv = kvv;
  pp.o = static_cast<uint16_t*>(o);
  pp.lse = lse_buf;
  pp.B = s->batch; pp.n_q = s->n_q; pp.n_kv = s->n_kv; pp.Hq = s->q_heads; pp.Hkv = s->kv_heads; pp.window = s->window;
  pp.scale = scale;
  pp.select = select && !prob ? 1 : 0;
  pp.theta = theta;
  pp.buf_sigma = select ? reinterpret_cast<float*>(w + plan.off_bs) : nullptr;
  pp.buf_j = select ? reinterpret_cast<int32_t*>(w + plan.off_bj) : nullptr;
  pp.counts = select ? reinterpret_cast<int32_t*>(w + plan.off_counts) : nullptr;
  pp.cap = plan.cap;
  if (prob) HIP_TRY(timed("prefill_attn", hst, [&] { return hs::launch_prefill_attn(pp, hst); }));

  if (select) {
    if (plan.sample) {
      hs::SampleParams sp{};
      sp.q = static_cast<const uint16_t*>(q);
      sp.kv = kvv;
      sp.B = s->batch; sp.n_q = s->n_q; sp.n_kv = s->n_kv; sp.Hq = s->q_heads; sp.Hkv = s->kv_heads;
      sp.window = s->window; sp.scale = scale; sp.stride = plan.stride; sp.max_samples = plan.max_samples;
      sp.samples = reinterpret_cast<float*>(w + plan.off_samples);
      sp.lse = prob ? lse_buf : nullptr;
      HIP_TRY(timed("sample_scores", hst, [&] { return hs::launch_sample_scores(sp, hst); }));
    }
    hs::ThresholdParams tp{};
    tp.B = s->batch; tp.n_q = s->n_q; tp.n_kv = s->n_kv; tp.Hkv = s->kv_heads; tp.top_k = s->top_k;
    tp.window = s->window; tp.cap = plan.cap; tp.stride = plan.stride; tp.max_samples = plan.max_samples;
    tp.samples = reinterpret_cast<const float*>(w + plan.off_samples);
    tp.theta = theta;
    tp.defer_count = reinterpret_cast<uint32_t*>(w + plan.off_defer + (size_t)plan.rows * 4);
    HIP_TRY(timed("threshold", hst, [&] { return hs::launch_threshold(tp, plan.rows, hst); }));
  }

  if (prob) {
    hs::PrefillParams cp = pp;
    cp.select = 1;
    HIP_TRY(timed("score_pass", hst, [&] { return hs::launch_score_pass(cp, hst); }));
  } else {
    HIP_TRY(timed("prefill_attn", hst, [&] { return hs::launch_prefill_attn(pp, hst); }));
  }

  if (select) {
    hs::SelectParams sp{};
    sp.q = static_cast<const uint16_t*>(q);
    sp.kv = kvv;
    sp.B = s->batch; sp.n_q = s->n_q; sp.n_kv = s->n_kv; sp.Hq = s->q_heads; sp.Hkv = s->kv_heads;
    sp.top_k = s->top_k; sp.window = s->window; sp.scale = scale;
    sp.buf_sigma = pp.buf_sigma; sp.buf_j = pp.buf_j; sp.counts = pp.counts; sp.cap = plan.cap;
    sp.force_rescan = (s->flags & HS_FLAG_EXACT_RESCAN) ? 1 : 0;
    sp.idx = idx;
    sp.rescan_count = reinterpret_cast<uint32_t*>(w + plan.off_defer + (size_t)plan.rows * 4 + 4);
    sp.defer_rows = reinterpret_cast<int32_t*>(w + plan.off_defer);
    sp.defer_count = reinterpret_cast<uint32_t*>(w + plan.off_defer + (size_t)plan.rows * 4);
    sp.lse = prob ? lse_buf : nullptr;
    HIP_TRY(timed("select_prefill", hst, [&] { return hs::launch_select_prefill(sp, plan.rows, hst); }));
  }
  return ok();
}

hs_status hs_select_diagnostics(const hs_shape* s, size_t* defer_rows_off, size_t* defer_count_off,
                                size_t* rescan_count_off) {
  Layout lay;
  if (!defer_rows_off || !defer_count_off || !rescan_count_off)
    return fail(HS_ERR_INVALID_ARG, "offset pointers must be non-NULL");
  hs_status st = validate_common(s, &lay);
  if (st != HS_OK) return st;
  if (s->n_q < 1 || s->n_kv < s->n_q) return fail(HS_ERR_INVALID_ARG, "need 1 <= n_q <= n_kv");
  if (s->top_k == 0 || (s->flags & (HS_FLAG_BLOCK_SELECT | HS_FLAG_HEAD_UNION)))
    return fail(HS_ERR_UNSUPPORTED, "only the token-level selection of hs_full_attn_select keeps these records");
  const PrefillPlan plan = plan_prefill(s);
  *defer_rows_off = plan.off_defer;
  *defer_count_off = plan.off_defer + (size_t)plan.rows * 4;
  *rescan_count_off = plan.off_defer + (size_t)plan.rows * 4 + 4;
  return ok();
}

hs_status hs_sparse_attn_reuse(const hs_shape* s_in, const void* q, const void* kv, const int32_t* idx,
                               const int32_t* seq_lens, void* o, void* ws, size_t ws_bytes, void* stream) {
  Layout lay;
  hs_status st = validate_common(s_in, &lay);
  if (st != HS_OK) return st;
  const hs_shape su = sparse_shape(s_in);  // index rows of G * top_k entries under the per-head union
  const hs_shape* s = &su;
  const bool decode = seq_lens != nullptr;
  if (decode) {
    if (s->n_q != 1) return fail(HS_ERR_INVALID_ARG, "decode calls need n_q == 1 (got %d)", s->n_q);
  } else if (s->n_q < 1 || s->n_kv < s->n_q || s->n_kv > s->kv_capacity) {
    return fail(HS_ERR_INVALID_ARG, "need 1 <= n_q (%d) <= n_kv (%d) <= kv_capacity (%d)", s->n_q, s->n_kv, s->kv_capacity);
  }
  if (!q || !kv || !o) return fail(HS_ERR_INVALID_ARG, "q, kv and o must be non-NULL");
  if (s->top_k > 0 && !idx) return fail(HS_ERR_INVALID_ARG, "idx must be non-NULL when top_k > 0");
  if (!aligned16(q) || !aligned16(kv) || !aligned16(o)) return fail(HS_ERR_INVALID_ARG, "q, kv and o must be 16-byte aligned");
  DecodePlan plan;
  if (decode) {
    plan = plan_decode_sparse(s);
    if (plan.total > 0 && (!ws || ws_bytes < plan.total))
      return fail(HS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.total, ws_bytes);
    if (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) return fail(HS_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  }
  st = check_device();
  if (st != HS_OK) return st;
  hipStream_t hst = static_cast<hipStream_t>(stream);

  hs::DecodeParams dp{};
  dp.q = static_cast<const uint16_t*>(q);
  dp.kv = kv_view(kv, lay);
  if (s->flags & HS_FLAG_FP8_KV) {  // kv is the FP8 copy made by hs_kv_fp8_convert
    dp.kv8 = static_cast<const uint8_t*>(kv);
    dp.kv8_scale = reinterpret_cast<const float*>(dp.kv8 + hs::kv8_codes_bytes(s->batch, s->kv_heads, s->kv_capacity) +
                                                  (size_t)s->batch * s->kv_heads * 8);
    dp.kv8_cap = s->kv_capacity;
  }
  dp.B = s->batch; dp.n_q = decode ? 1 : s->n_q; dp.n_kv = decode ? s->kv_capacity : s->n_kv; dp.Hq = s->q_heads; dp.Hkv = s->kv_heads;
  dp.top_k = s->top_k; dp.window = s->window; dp.scale = eff_scale(s);
  dp.seq_lens = seq_lens;
  dp.idx = idx;
  dp.o = static_cast<uint16_t*>(o);
  dp.lse = nullptr;
  if (decode) {
    dp.splits = plan.splits;
    dp.split_len = plan.split_len;
    dp.combine_in_block = plan.in_block ? 1 : 0;
    dp.part = plan.in_block || plan.splits == 1 ? nullptr
                                                : reinterpret_cast<float*>(static_cast<char*>(ws) + plan.off_part);
  } else {
    dp.splits = 1;
    dp.split_len = s->top_k + s->window + 32;
  }
  HIP_TRY(timed(decode ? "sparse_decode" : "sparse_prefill", hst, [&] { return hs::launch_sparse(dp, hst); }));
  if (decode && plan.splits > 1 && !plan.in_block) {
    hs::CombineParams cp{};
    cp.part = dp.part; cp.o = dp.o; cp.lse = nullptr; cp.seq_lens = seq_lens;
    cp.B = s->batch; cp.Hq = s->q_heads; cp.Hkv = s->kv_heads; cp.splits = plan.splits; cp.split_len = plan.split_len;
    cp.sparse_k = s->top_k; cp.window = s->window; cp.max_len = s->kv_capacity;
    HIP_TRY(timed("lse_combine", hst, [&] { return hs::launch_combine(cp, hst); }));
  }
  return ok();
}

hs_status hs_decode_step_noalloc(const hs_shape* s, const void* q, const void* kv_new, void* kv,
                                 const int32_t* seq_lens, int32_t max_seq_len, void* o, float* lse, int32_t* idx,
                                 void* stream) {
  Layout lay;
  hs_status st = validate_common(s, &lay);
  if (st != HS_OK) return st;
  if (max_seq_len < 1 || max_seq_len > s->kv_capacity)
    return fail(HS_ERR_INVALID_ARG, "need 1 <= max_seq_len (%d) <= kv_capacity (%d)", max_seq_len, s->kv_capacity);
  const size_t need = plan_decode_full(s, max_seq_len).total;
  if (need > hs::kStaticScratchBytes)
    return fail(HS_ERR_WORKSPACE, "this step needs %zu bytes of scratch; the library's static scratch holds %zu "
                "(use hs_decode_step with a caller workspace)", need, hs::kStaticScratchBytes);
  st = check_device();
  if (st != HS_OK) return st;
  void* scratch = nullptr;
  HIP_TRY(hs::static_scratch(&scratch));
  return hs_decode_step(s, q, kv_new, kv, seq_lens, max_seq_len, o, lse, idx, scratch, hs::kStaticScratchBytes,
                        stream);
}

hs_status hs_decode_step(const hs_shape* s, const void* q, const void* kv_new, void* kv, const int32_t* seq_lens,
                         int32_t max_seq_len, void* o, float* lse, int32_t* idx, void* ws, size_t ws_bytes,
                         void* stream) {
  Layout lay;
  hs_status st = validate_common(s, &lay);
  if (st != HS_OK) return st;
  if (s->n_q != 1) return fail(HS_ERR_INVALID_ARG, "decode calls need n_q == 1 (got %d)", s->n_q);
  if (max_seq_len < 1 || max_seq_len > s->kv_capacity)
    return fail(HS_ERR_INVALID_ARG, "need 1 <= max_seq_len (%d) <= kv_capacity (%d)", max_seq_len, s->kv_capacity);
  const bool fp8 = (s->flags & HS_FLAG_FP8_KV) != 0;
  if (fp8 && (s->flags & (HS_FLAG_PROB_SCORE | HS_FLAG_HEAD_UNION)))
    return fail(HS_ERR_UNSUPPORTED, "the FP8 decode step takes the logit score (token or block level)");
  if (!q || !kv_new || !kv || !seq_lens || !o) return fail(HS_ERR_INVALID_ARG, "q, kv_new, kv, seq_lens and o must be non-NULL");
  if (s->top_k > 0 && !idx) return fail(HS_ERR_INVALID_ARG, "idx must be non-NULL when top_k > 0");
  if (!aligned16(q) || !aligned16(kv_new) || !aligned16(kv) || !aligned16(o))
    return fail(HS_ERR_INVALID_ARG, "q, kv_new, kv and o must be 16-byte aligned");
  const DecodePlan plan = plan_decode_full(s, max_seq_len);
  if (!ws || ws_bytes < plan.total) return fail(HS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.total, ws_bytes);
  if (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) return fail(HS_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  st = check_device();
  if (st != HS_OK) return st;
  hipStream_t hst = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);

  hs::DecodeParams dp{};
  if (fp8) {
    // kv is the FP8 copy: the new token's rows are quantised with the stored
    // scales of its KV head into slot seq_lens[b] - 1, and the layer reads
    // codes (kv_new seen as a one-row cache: token stride 0)
    hs::Fp8ConvertParams cp{};
    cp.kv = hs::KvView{static_cast<const uint16_t*>(kv_new), (int64_t)s->kv_heads * 256, 256, 0, 128};
    cp.kv8 = static_cast<uint8_t*>(kv);
    cp.B = s->batch; cp.Hkv = s->kv_heads; cp.n_kv = 1; cp.cap = s->kv_capacity;
    cp.seq_lens = seq_lens;
    HIP_TRY(timed("kv_append", hst, [&] { return hs::launch_kv_convert_fp8(cp, hst); }));
    dp.kv8 = static_cast<const uint8_t*>(kv);
    dp.kv8_scale = reinterpret_cast<const float*>(dp.kv8 + hs::kv8_codes_bytes(s->batch, s->kv_heads, s->kv_capacity) +
                                                  (size_t)s->batch * s->kv_heads * 8);
    dp.kv8_cap = s->kv_capacity;
  } else {
    hs::AppendParams ap{};
    ap.kv_new = static_cast<const uint16_t*>(kv_new);
    ap.kv = static_cast<uint16_t*>(kv);
    ap.sb = lay.sb; ap.sh = lay.sh; ap.st = lay.st; ap.voff = lay.voff;
    ap.seq_lens = seq_lens; ap.B = s->batch; ap.Hkv = s->kv_heads; ap.cap = max_seq_len;
    HIP_TRY(timed("kv_append", hst, [&] { return hs::launch_append(ap, hst); }));
  }

  dp.q = static_cast<const uint16_t*>(q);
  dp.kv = kv_view(kv, lay);
  dp.B = s->batch; dp.n_q = 1; dp.n_kv = max_seq_len; dp.Hq = s->q_heads; dp.Hkv = s->kv_heads;
  dp.top_k = s->top_k; dp.window = s->window; dp.scale = eff_scale(s);
  dp.seq_lens = seq_lens;
  dp.splits = plan.splits; dp.split_len = plan.split_len;
  dp.o = static_cast<uint16_t*>(o);
  float* lse_buf = plan.prob && !lse ? reinterpret_cast<float*>(w + plan.off_lse) : lse;
  dp.lse = lse_buf;
  dp.part = reinterpret_cast<float*>(w + plan.off_part);
  float* sigma = s->top_k > 0 ? reinterpret_cast<float*>(w + plan.off_sigma) : nullptr;
  dp.sigma = plan.prob || plan.head_union ? nullptr : sigma;  // those scores are written by their own pass
  dp.sigma_stride = plan.sigma_stride;
  float* samp = plan.sel_slices > 0 ? reinterpret_cast<float*>(w + plan.off_samp) : nullptr;
  dp.samp = samp;
  HIP_TRY(timed("decode_full", hst, [&] { return hs::launch_decode_full(dp, hst); }));
  if (plan.splits > 1) {
    hs::CombineParams cp{};
    cp.part = dp.part; cp.o = dp.o; cp.lse = lse_buf; cp.seq_lens = seq_lens;
    cp.B = s->batch; cp.Hq = s->q_heads; cp.Hkv = s->kv_heads; cp.splits = plan.splits; cp.split_len = plan.split_len;
    cp.sparse_k = -1; cp.window = s->window; cp.max_len = max_seq_len;
    HIP_TRY(timed("lse_combine", hst, [&] { return hs::launch_combine(cp, hst); }));
  }
  if (plan.prob) {
    hs::DecodeScoreParams zp{};
    zp.q = dp.q; zp.kv = dp.kv; zp.seq_lens = seq_lens; zp.lse = lse_buf;
    zp.B = s->batch; zp.Hq = s->q_heads; zp.Hkv = s->kv_heads; zp.window = s->window; zp.scale = dp.scale;
    zp.sigma = sigma; zp.sigma_stride = plan.sigma_stride; zp.max_cand = max_seq_len - s->window; zp.max_len = max_seq_len;
    zp.samp = samp;
    HIP_TRY(timed("decode_score", hst, [&] { return hs::launch_decode_prob_score(zp, hst); }));
  }
  if (plan.head_union) {
    const int G = s->q_heads / s->kv_heads;
    hs::DecodeScoreParams zp{};
    zp.q = dp.q; zp.kv = dp.kv; zp.seq_lens = seq_lens; zp.lse = nullptr;
    zp.B = s->batch; zp.Hq = s->q_heads; zp.Hkv = s->kv_heads; zp.window = s->window; zp.scale = dp.scale;
    zp.sigma = sigma; zp.sigma_stride = plan.sigma_stride; zp.max_cand = max_seq_len - s->window; zp.max_len = max_seq_len;
    zp.samp = samp;
    zp.per_head = 1;
    HIP_TRY(timed("decode_score", hst, [&] { return hs::launch_decode_prob_score(zp, hst); }));
    int32_t* hidx = reinterpret_cast<int32_t*>(w + plan.off_hidx);
    hs::SelectDecodeParams sp{};
    sp.B = s->batch; sp.Hkv = s->q_heads; sp.top_k = s->top_k; sp.window = s->window;
    sp.seq_lens = seq_lens; sp.max_len = max_seq_len; sp.sigma = sigma; sp.sigma_stride = plan.sigma_stride; sp.idx = hidx;
    sp.nslices = plan.sel_slices;
    if (plan.sel_slices > 0) {
      sp.theta_key = reinterpret_cast<uint32_t*>(w + plan.off_theta);
      sp.samp = samp;
      sp.seg_count = reinterpret_cast<uint32_t*>(w + plan.off_segcnt);
      sp.seg_key = reinterpret_cast<uint32_t*>(w + plan.off_segkey);
      sp.seg_idx = reinterpret_cast<int32_t*>(w + plan.off_segidx);
    }
    HIP_TRY(timed("select_decode", hst, [&] { return hs::launch_select_decode(sp, s->batch * s->q_heads, hst); }));
    hs::UnionParams un{};
    un.lists = hidx; un.row_stride = (int64_t)G * s->top_k; un.head_stride = s->top_k; un.G = G; un.k = s->top_k;
    un.B = s->batch; un.n_q = 1; un.Hkv = s->kv_heads; un.window = s->window; un.seq_lens = seq_lens; un.max_len = max_seq_len; un.out = idx;
    HIP_TRY(timed("head_union", hst, [&] { return hs::launch_head_union(un, (int64_t)s->batch * s->kv_heads, hst); }));
    return ok();
  }
  if (plan.block) {
    hs::BlockMaxParams mp{};
    mp.sigma = sigma; mp.sigma_stride = plan.sigma_stride; mp.seq_lens = seq_lens; mp.max_len = max_seq_len;
    mp.B = s->batch; mp.Hkv = s->kv_heads; mp.window = s->window;
    mp.blk_score = reinterpret_cast<float*>(w + plan.off_blk); mp.blk_stride = plan.blk_stride;
    HIP_TRY(timed("block_max", hst, [&] { return hs::launch_block_max(mp, hst); }));
    hs::BlockSelectParams bp{};
    bp.B = s->batch; bp.n_q = 1; bp.Hkv = s->kv_heads; bp.top_k = s->top_k; bp.window = s->window;
    bp.seq_lens = seq_lens; bp.max_len = max_seq_len; bp.blk_score = mp.blk_score; bp.blk_stride = plan.blk_stride; bp.idx = idx;
    HIP_TRY(timed("select_blocks", hst, [&] { return hs::launch_select_blocks(bp, (int64_t)s->batch * s->kv_heads, hst); }));
    return ok();
  }
  if (s->top_k > 0) {
    hs::SelectDecodeParams sp{};
    sp.B = s->batch; sp.Hkv = s->kv_heads; sp.top_k = s->top_k; sp.window = s->window;
    sp.seq_lens = seq_lens; sp.max_len = max_seq_len; sp.sigma = sigma; sp.sigma_stride = plan.sigma_stride; sp.idx = idx;
    sp.nslices = plan.sel_slices;
    if (plan.sel_slices > 0) {
      sp.theta_key = reinterpret_cast<uint32_t*>(w + plan.off_theta);
      sp.samp = samp;
      sp.seg_count = reinterpret_cast<uint32_t*>(w + plan.off_segcnt);
      sp.seg_key = reinterpret_cast<uint32_t*>(w + plan.off_segkey);
      sp.seg_idx = reinterpret_cast<int32_t*>(w + plan.off_segidx);
    }
    HIP_TRY(timed("select_decode", hst, [&] { return hs::launch_select_decode(sp, s->batch * s->kv_heads, hst); }));
  }
  return ok();
}

hs_status hs_kv_bridge(const hs_shape* s, const void* hidden, int32_t d_model, const void* w_kv, void* kv,
                       void* stream) {
  Layout lay;
  hs_status st = validate_common(s, &lay);
  if (st != HS_OK) return st;
  if (s->flags & HS_FLAG_FP8_KV) return fail(HS_ERR_UNSUPPORTED, "the bridge writes the bf16 cache");
  if (s->n_q < 1 || s->n_kv < s->n_q || s->n_kv > s->kv_capacity)
    return fail(HS_ERR_INVALID_ARG, "need 1 <= n_q (%d) <= n_kv (%d) <= kv_capacity (%d)", s->n_q, s->n_kv, s->kv_capacity);
  if (d_model < 64 || d_model % 64 != 0 || d_model > 65536)
    return fail(HS_ERR_UNSUPPORTED, "d_model must be a multiple of 64 in [64, 65536] (got %d)", d_model);
  if (!hidden || !w_kv || !kv) return fail(HS_ERR_INVALID_ARG, "hidden, w_kv and kv must be non-NULL");
  if (!aligned16(hidden) || !aligned16(w_kv) || !aligned16(kv))
    return fail(HS_ERR_INVALID_ARG, "hidden, w_kv and kv must be 16-byte aligned");
  st = check_device();
  if (st != HS_OK) return st;
  hipStream_t hst = static_cast<hipStream_t>(stream);
  hs::BridgeParams p{};
  p.h = static_cast<const uint16_t*>(hidden);
  p.w = static_cast<const uint16_t*>(w_kv);
  p.kv = static_cast<uint16_t*>(kv);
  p.sb = lay.sb; p.sh = lay.sh; p.st = lay.st; p.voff = lay.voff;
  p.B = s->batch; p.n_q = s->n_q; p.n_kv = s->n_kv; p.Hkv = s->kv_heads; p.d_model = d_model;
  HIP_TRY(timed("kv_bridge", hst, [&] { return hs::launch_kv_bridge(p, hst); }));
  return ok();
}

hs_status hs_gather_probe(const void* src, int64_t src_rows, const int32_t* idx, int64_t n, int32_t per_wave,
                          uint32_t* out, void* stream) {
  if (!src || !idx || !out) return fail(HS_ERR_INVALID_ARG, "src, idx and out must be non-NULL");
  if (!aligned16(src)) return fail(HS_ERR_INVALID_ARG, "src must be 16-byte aligned");
  if (src_rows < 1 || src_rows > (int64_t)(0xffffffffu / 512u))
    return fail(HS_ERR_INVALID_ARG, "src_rows must be in [1, 2^32 / 512)");
  if (n < 1 || per_wave < 1 || per_wave > 2048)
    return fail(HS_ERR_INVALID_ARG, "need n >= 1 and 1 <= per_wave <= 2048");
  hs_status st = check_device();
  if (st != HS_OK) return st;
  hipStream_t hst = static_cast<hipStream_t>(stream);
  hs::ProbeParams p{static_cast<const uint8_t*>(src), (uint32_t)(src_rows * 512), idx, n, per_wave, out};
  HIP_TRY(timed("gather_probe", hst, [&] { return hs::launch_gather_probe(p, hst); }));
  return ok();
}

hs_status hs_kv_fp8_size(const hs_shape* s, size_t* bytes) {
  if (!s || !bytes) return fail(HS_ERR_INVALID_ARG, "shape and bytes must be non-NULL");
  if (s->batch < 1 || s->kv_heads < 1 || s->kv_capacity < 1)
    return fail(HS_ERR_INVALID_ARG, "need batch, kv_heads and kv_capacity >= 1");
  *bytes = (size_t)hs::kv8_total_bytes(s->batch, s->kv_heads, s->kv_capacity);
  return ok();
}

hs_status hs_kv_fp8_convert(const hs_shape* s, const void* kv, void* kv8, const int32_t* seq_lens, void* stream) {
  Layout lay;
  hs_status st = validate_common(s, &lay);
  if (st != HS_OK) return st;
  if (!kv || !kv8) return fail(HS_ERR_INVALID_ARG, "kv and kv8 must be non-NULL");
  if (!aligned16(kv) || !aligned16(kv8)) return fail(HS_ERR_INVALID_ARG, "kv and kv8 must be 16-byte aligned");
  if (!seq_lens && (s->n_kv < 1 || s->n_kv > s->kv_capacity))
    return fail(HS_ERR_INVALID_ARG, "need 1 <= n_kv (%d) <= kv_capacity (%d)", s->n_kv, s->kv_capacity);
  st = check_device();
  if (st != HS_OK) return st;
  hipStream_t hst = static_cast<hipStream_t>(stream);
  hs::Fp8ConvertParams cp{};
  cp.kv = kv_view(kv, lay);
  cp.kv8 = static_cast<uint8_t*>(kv8);
  cp.B = s->batch; cp.Hkv = s->kv_heads; cp.n_kv = s->n_kv; cp.cap = s->kv_capacity;
  cp.seq_lens = seq_lens;
  HIP_TRY(timed("kv_fp8_convert", hst, [&] { return hs::launch_kv_convert_fp8(cp, hst); }));
  return ok();
}

}  // extern "C"
