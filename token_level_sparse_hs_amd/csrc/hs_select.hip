// Exact token-level top-k selection on fp32 score bits (gfx950).
//
// What is selected (token-level selection with a forced recent window, as in
// "HySparse2 od Xiaomi zkracuje zpracovani dlouheho kontextu", section "Proc
// neni nutne znovu zpracovat cely dlouhy vstup", and the DAIR.AI weekly's
// "Prefill exits early" bullet): for one (query row, KV group), the top_k
// candidates j in C(p) = [0, p-W] ordered by (score desc, j asc), emitted in
// ascending j order and padded with -1. The pages leave the score open; the
// score here is the group's maximum scaled logit, computed by the attention
// kernels and handed over as fp32.
//
// Method: an MSB-first radix select over the order-preserving 32-bit image of
// each score (8-bit digits, per-wave LDS histograms) finds the exact k-th key
// T and how many elements equal to T are still needed. Every source lists its
// elements in ascending token order, so one ordered pass emits the selection
// already sorted: a block-wide exclusive scan of per-thread (above-T, equal-T)
// counts gives each thread its output offset, and ties at T are taken in token
// order, i.e. lowest index first. One 256-thread block handles one row.
//  * Rows of up to 8192 elements are held in registers (32 per thread, each
//    thread a contiguous run) for all passes.
//  * Longer rows are first filtered: the m-th largest of 2048 strided samples
//    bounds the k-th score from below with overwhelming probability; each wave
//    appends the elements at or above it from its quarter of the row, in order,
//    to LDS, and the register path runs on those. If the filter does not
//    provably contain the top k (too few or too many survivors), the row falls
//    back to a streaming radix select over the whole row.
//
// Element sources:
//   kBuffer  (score, index) pairs appended by the prefill attention kernel for
//            scores at or above a per-row threshold; the count decides whether
//            the buffer provably holds the top_k (count >= min(k,|C|) and no
//            overflow). Otherwise the row is rescanned exactly (kRescan).
//   kDense   a dense score row indexed by token (decode).
//   kRescan  scores recomputed on the fly from q and the cache with fp32 VALU
//            dot products (slow, exact; the fallback and the testing path).
//   threshold mode: the m-th largest of a dense row of sampled scores (the
//            per-row filter threshold used by the prefill attention kernel).
#include "hs_common.hpp"
#include "hs_kernels.hpp"

namespace hs {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / 64;

struct SelShared {
  uint32_t hist[kSelWaves][256];
  uint32_t prefix;       // digits fixed so far
  uint32_t need;         // rank still to find within the current prefix
  uint32_t eq_count;     // elements equal to the full key after the last pass
  uint32_t found_digit;
  uint32_t found_gt;
  uint32_t found_eq;
  uint32_t nsel;
  int32_t flag;
  uint32_t wave_tot[kSelWaves];
  uint32_t cnt[kSelWaves];
};

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// After a histogram pass: wave 0 finds the digit d holding the `need`-th
// element in the requested direction (descending: largest digits first).
__device__ void pick_digit(SelShared& sh, bool descending, uint32_t need) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    uint32_t c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int d = descending ? 255 - 4 * lane - q : 4 * lane + q;
      c[q] = sh.hist[0][d] + sh.hist[1][d] + sh.hist[2][d] + sh.hist[3][d];
    }
    int local = (int)(c[0] + c[1] + c[2] + c[3]);
    int incl = wave_incl_scan(local);
    int excl = incl - local;
    if ((uint32_t)excl < need && need <= (uint32_t)incl) {
      uint32_t acc = (uint32_t)excl;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (acc + c[q] >= need) {
          sh.found_digit = descending ? 255 - 4 * lane - q : 4 * lane + q;
          sh.found_gt = acc;
          sh.found_eq = c[q];
          break;
        }
        acc += c[q];
      }
    }
  }
}

__device__ __forceinline__ void clear_hist(SelShared& sh) {
  for (int i = threadIdx.x; i < kSelWaves * 256; i += kSelThreads) (&sh.hist[0][0])[i] = 0;
}

__device__ __forceinline__ uint32_t block_excl_scan(SelShared& sh, uint32_t v) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t incl = (uint32_t)wave_incl_scan((int)v);
  if (lane == 63) sh.wave_tot[wave] = incl;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += sh.wave_tot[w];
  __syncthreads();
  return base + incl - v;
}

// ---------------------------------------------------------------- sources

struct DenseSrc {
  const float* s;
  __device__ __forceinline__ uint32_t key(int i) const { return score_key(s[i]); }
  __device__ __forceinline__ int32_t index(int i) const { return i; }
};

struct BufSrc {
  const float* s;
  const int32_t* j;
  __device__ __forceinline__ uint32_t key(int i) const { return score_key(s[i]); }
  __device__ __forceinline__ int32_t index(int i) const { return j[i]; }
};

// Scores recomputed from the group's query heads (fp32 copy in LDS) and the
// cache: sigma_j = max_h fl(scale * <q_h, k_j>), dot products in fp32, in
// dimension order.
struct RescanSrc {
  const float* qs;  // LDS [G][128]
  const uint16_t* krow0;
  int64_t kstride;
  int G;
  float scale;
  __device__ uint32_t key(int i) const {
    const uint16_t* kr = krow0 + (int64_t)i * kstride;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int c = 0; c < kHeadDim / 8; ++c) {
      const u32x4 w = ld16(kr + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float kv = (e & 1) ? bf16hi(w[e >> 1]) : bf16lo(w[e >> 1]);
#pragma unroll
        for (int h = 0; h < 8; ++h)
          if (h < G) acc[h] = fmaf(qs[h * kHeadDim + 8 * c + e], kv, acc[h]);
      }
    }
    float best = kNegInf;
#pragma unroll
    for (int h = 0; h < 8; ++h)
      if (h < G) best = fmaxf(best, acc[h] * scale);
    return score_key(best);
  }
  __device__ __forceinline__ int32_t index(int i) const { return i; }
};

// Radix search for the key T of the element of rank `rank` (1-based, largest
// first) among n elements. Leaves in shared: prefix = T, found_gt = number of
// elements with key > T, eq_count = number with key == T.
template <class Src>
__device__ void find_kth_key(SelShared& sh, const Src& src, int n, uint32_t rank) {
  const int wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) { sh.prefix = 0; sh.need = rank; }
  uint32_t gt_total = 0;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t pmask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
    clear_hist(sh);
    __syncthreads();
    const uint32_t prefix = sh.prefix;
    for (int i = threadIdx.x; i < n; i += kSelThreads) {
      uint32_t k = src.key(i);
      if ((k & pmask) == prefix) atomicAdd(&sh.hist[wave][(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    pick_digit(sh, true, sh.need);
    __syncthreads();
    if (threadIdx.x == 0) {
      sh.prefix = prefix | (sh.found_digit << shift);
      sh.need -= sh.found_gt;
      sh.eq_count = sh.found_eq;
    }
    gt_total += 0;
    __syncthreads();
  }
  if (threadIdx.x == 0) sh.found_gt = rank - sh.need;  // elements strictly above T
  __syncthreads();
}

// Streaming top-k of an index-ordered source of any length (the fallback):
// find_kth_key over the whole row, then each thread walks a contiguous run of
// the row twice (count, then write) around one block-wide scan, so the output
// is ascending and ties at T are taken lowest index first.
template <class Src>
__device__ void topk_stream(SelShared& sh, const Src& src, int n, int k, int32_t* out) {
  find_kth_key(sh, src, n, (uint32_t)k);
  const uint32_t T = sh.prefix;
  const uint32_t need = (uint32_t)k - sh.found_gt;  // tied elements to keep
  __syncthreads();
  const int per = (n + kSelThreads - 1) / kSelThreads;
  const int i0 = imin(n, threadIdx.x * per), i1 = imin(n, i0 + per);
  uint32_t ngt = 0, neq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = src.key(i);
    ngt += key > T;
    neq += key == T;
  }
  // counts can exceed 16 bits here: scan them separately
  const uint32_t gt_before = block_excl_scan(sh, ngt);
  const uint32_t eq_before = block_excl_scan(sh, neq);
  uint32_t pos = gt_before + (eq_before < need ? eq_before : need);
  uint32_t eq_rank = eq_before;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = src.key(i);
    bool sel = key > T;
    if (key == T) {
      sel = eq_rank < need;
      ++eq_rank;
    }
    if (sel) out[pos++] = src.index(i);
  }
}

// ---------------------------------------------------------------- register path

constexpr int kE = 32;                    // elements per thread in registers
constexpr int kRegCap = kSelThreads * kE; // 8192
constexpr int kSamples = 2048;

struct RadixResult {
  uint32_t prefix;  // decided high bits of the threshold key
  uint32_t mask;    // which bits are decided
  uint32_t need;    // elements still needed among those equal to prefix
  bool take_all;    // every element equal to prefix (under mask) is selected
};

// Radix search over register-held keys (0 = empty slot) for the element of
// rank `rank` (1-based, largest first). Stops early once a whole bucket is
// needed.
template <int E>
__device__ RadixResult radix_regs(SelShared& sh, const uint32_t (&key)[E], uint32_t rank) {
  const int wave = threadIdx.x >> 6;
  RadixResult r{0u, 0u, rank, false};
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    clear_hist(sh);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e] && (key[e] & r.mask) == r.prefix) atomicAdd(&sh.hist[wave][(key[e] >> shift) & 255u], 1u);
    __syncthreads();
    pick_digit(sh, true, r.need);
    __syncthreads();
    r.prefix |= sh.found_digit << shift;
    r.mask |= 0xffu << shift;
    r.need -= sh.found_gt;
    if (sh.found_eq == r.need) {
      r.take_all = true;
      break;
    }
  }
  __syncthreads();
  return r;
}

// Exact top-k (k < n <= kRegCap) of an index-ordered source; writes the k
// selected indices ascending to out.
template <class Src>
__device__ void topk_regs(SelShared& sh, const Src& src, int n, int k, int32_t* out) {
  const int E = (n + kSelThreads - 1) / kSelThreads;
  const int beg = threadIdx.x * E;
  uint32_t key[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) key[e] = (e < E && beg + e < n) ? src.key(beg + e) : 0u;
  const RadixResult r = radix_regs<kE>(sh, key, (uint32_t)k);
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    if (!key[e]) continue;
    const uint32_t km = key[e] & r.mask;
    ngt += km > r.prefix;
    neq += km == r.prefix;
  }
  const uint32_t excl = block_excl_scan(sh, ngt | (neq << 16));
  const uint32_t eq_before = excl >> 16;
  uint32_t pos = (excl & 0xffffu) + (r.take_all ? eq_before : (eq_before < r.need ? eq_before : r.need));
  uint32_t eq_rank = eq_before;
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    if (!key[e]) continue;
    const uint32_t km = key[e] & r.mask;
    bool sel = km > r.prefix;
    if (km == r.prefix) {
      sel = r.take_all || eq_rank < r.need;
      ++eq_rank;
    }
    if (sel) out[pos++] = src.index(beg + e);
  }
}

struct LdsSrc {
  const uint32_t* k;
  const int32_t* j;
  __device__ __forceinline__ uint32_t key(int i) const { return k[i]; }
  __device__ __forceinline__ int32_t index(int i) const { return j[i]; }
};

// Long rows: sampled threshold, ordered filter into LDS, then topk_regs.
// Returns false (nothing written) when the filter cannot be used.
template <class Src>
__device__ bool topk_filtered(SelShared& sh, uint32_t* lkey, int32_t* lidx, const Src& src, int n, int k,
                              int32_t* out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const double mu = (double)k * kSamples / (double)n;
  const int m = (int)ceil(mu + 6.0 * sqrt(mu)) + 1;
  if (m >= kSamples) return false;
  constexpr int ES = kSamples / kSelThreads;
  uint32_t skey[ES];
#pragma unroll
  for (int e = 0; e < ES; ++e) {
    const int s = threadIdx.x * ES + e;
    skey[e] = src.key((int)(((int64_t)s * n) / kSamples));
  }
  const RadixResult r = radix_regs<ES>(sh, skey, (uint32_t)m);
  const uint32_t theta = r.prefix;  // keys >= theta include the m largest samples
  // Each wave filters a contiguous quarter of the row into its LDS region.
  constexpr int kRegion = kRegCap / kSelWaves;
  const int q0 = (int)(((int64_t)n * wave) / kSelWaves), q1 = (int)(((int64_t)n * (wave + 1)) / kSelWaves);
  uint32_t cnt = 0;
  for (int i0 = q0; i0 < q1; i0 += 64) {
    const int i = i0 + lane;
    uint32_t kk = 0;
    if (i < q1) kk = src.key(i);
    const bool pass = i < q1 && kk >= theta;
    const uint64_t bm = ballot(pass);
    const uint32_t pos = cnt + lane_prefix(bm);
    if (pass && pos < (uint32_t)kRegion) {
      lkey[wave * kRegion + pos] = kk;
      lidx[wave * kRegion + pos] = src.index(i);
    }
    cnt += (uint32_t)__popcll(bm);
  }
  if (lane == 0) sh.cnt[wave] = cnt;
  __syncthreads();
  uint32_t total = 0;
  bool over = false;
  for (int w = 0; w < kSelWaves; ++w) {
    total += sh.cnt[w];
    over |= sh.cnt[w] > (uint32_t)kRegion;
  }
  if (over || total < (uint32_t)k) {
    __syncthreads();
    return false;
  }
  // Compact the regions in wave order (keeps ascending index order).
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += sh.cnt[w];
  // move through registers to avoid overlapping copies: read all, sync, write
  uint32_t tk[kRegion / 64];
  int32_t tj[kRegion / 64];
#pragma unroll
  for (int e = 0; e < kRegion / 64; ++e) {
    const uint32_t i = lane + 64u * e;
    tk[e] = i < cnt ? lkey[wave * kRegion + i] : 0u;
    tj[e] = i < cnt ? lidx[wave * kRegion + i] : 0;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kRegion / 64; ++e) {
    const uint32_t i = lane + 64u * e;
    if (i < cnt) {
      lkey[base + i] = tk[e];
      lidx[base + i] = tj[e];
    }
  }
  __syncthreads();
  if ((int)total == k) {
    for (int i = threadIdx.x; i < k; i += kSelThreads) out[i] = lidx[i];
    return true;
  }
  topk_regs(sh, LdsSrc{lkey, lidx}, (int)total, k, out);
  return true;
}

// ---------------------------------------------------------------- kernels

// Dispatch by row length: registers, LDS filter (BIG kernels only), stream.
template <bool BIG, class Src>
__device__ void topk_any(SelShared& sh, uint32_t* lkey, int32_t* lidx, const Src& src, int n, int k, int32_t* out) {
  if (n <= kRegCap) {
    topk_regs(sh, src, n, k, out);
    return;
  }
  if constexpr (BIG) {
    if (topk_filtered(sh, lkey, lidx, src, n, k, out)) return;
  }
  topk_stream(sh, src, n, k, out);
}

template <bool BIG>
struct SelLds {
  uint32_t key[BIG ? kRegCap : 1];
  int32_t idx[BIG ? kRegCap : 1];
};

// Top-k over the candidate buffer of each (b, t, g) row of a prefill call.
template <bool BIG>
__global__ __launch_bounds__(kSelThreads) void select_prefill_kernel(SelectParams P) {
  __shared__ SelShared sh;
  __shared__ SelLds<BIG> lds;
  __shared__ float qs[8 * kHeadDim];
  const int64_t row = blockIdx.x;
  const int g = (int)(row % P.Hkv);
  const int64_t bt = row / P.Hkv;
  const int t = (int)(bt % P.n_q);
  const int b = (int)(bt / P.n_q);
  const int p = P.n_kv - P.n_q + t;
  const int ncand = imax(0, p - P.window + 1);
  int32_t* out = P.idx + row * P.top_k;
  if (ncand <= P.top_k) {
    // reading: fewer candidates than k -> all of C(p), then -1 padding
    for (int i = threadIdx.x; i < P.top_k; i += kSelThreads) out[i] = i < ncand ? i : -1;
    return;
  }
  const int cnt = P.counts[row];
  const bool ok = !P.force_rescan && cnt >= P.top_k && cnt <= P.cap;
  if (ok) {
    BufSrc src{P.buf_sigma + row * (int64_t)P.cap, P.buf_j + row * (int64_t)P.cap};
    if (cnt == P.top_k) {
      for (int i = threadIdx.x; i < cnt; i += kSelThreads) out[i] = src.index(i);
      return;
    }
    topk_any<BIG>(sh, lds.key, lds.idx, src, cnt, P.top_k, out);
    return;
  }
  // Exact rescan of every candidate.
  const int G = P.Hq / P.Hkv;
  const uint16_t* qrow = P.q + (bt * P.Hq + (int64_t)g * G) * kHeadDim;
  for (int i = threadIdx.x; i < G * kHeadDim; i += kSelThreads) {
    uint16_t v = qrow[i];
    qs[i] = __uint_as_float((uint32_t)v << 16);
  }
  __syncthreads();
  RescanSrc src{qs, P.kv.slab(b, g), P.kv.st, G, P.scale};
  topk_any<BIG>(sh, lds.key, lds.idx, src, ncand, P.top_k, out);
  if (threadIdx.x == 0 && P.rescan_count) atomicAdd(P.rescan_count, 1u);
}

// Per-row filter threshold from sampled scores: theta = the m-th largest valid
// sample, with m chosen so that, for exchangeable scores, the full candidate
// set holds at least top_k scores >= theta except with negligible
// probability (mean + 6 standard deviations of the sampled count above the
// true k-th score, plus one). Rows whose candidates all fit the buffer get
// theta = -inf.
__global__ __launch_bounds__(kSelThreads) void threshold_kernel(ThresholdParams P) {
  __shared__ SelShared sh;
  const int64_t row = blockIdx.x;
  const int64_t bt = row / P.Hkv;
  const int t = (int)(bt % P.n_q);
  const int p = P.n_kv - P.n_q + t;
  const int ncand = imax(0, p - P.window + 1);
  if (ncand <= P.cap) {
    if (threadIdx.x == 0) P.theta[row] = kNegInf;
    return;
  }
  const int nsamp = (ncand + P.stride - 1) / P.stride;  // samples j = s*stride <= p-W
  const double mu = (double)nsamp * (double)P.top_k / (double)ncand;
  int m = (int)ceil(mu + 6.0 * sqrt(mu)) + 1;
  if (m > nsamp) {
    if (threadIdx.x == 0) P.theta[row] = kNegInf;
    return;
  }
  DenseSrc src{P.samples + row * (int64_t)P.max_samples};
  if (nsamp <= kRegCap) {
    const int E = (nsamp + kSelThreads - 1) / kSelThreads;
    const int beg = threadIdx.x * E;
    uint32_t key[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) key[e] = (e < E && beg + e < nsamp) ? src.key(beg + e) : 0u;
    const RadixResult r = radix_regs<kE>(sh, key, (uint32_t)m);
    // take_all leaves the low bits open: prefix is then a lower bound
    if (threadIdx.x == 0) P.theta[row] = key_to_score(r.prefix);
  } else {
    find_kth_key(sh, src, nsamp, (uint32_t)m);
    if (threadIdx.x == 0) P.theta[row] = key_to_score(sh.prefix);
  }
}

// Decode: top-k over the dense score row of each (b, g).
__global__ __launch_bounds__(kSelThreads) void select_decode_kernel(SelectDecodeParams P) {
  __shared__ SelShared sh;
  __shared__ SelLds<true> lds;
  const int row = blockIdx.x;  // b * Hkv + g
  const int b = row / P.Hkv;
  const int p = P.seq_lens[b] - 1;
  const int ncand = imax(0, p - P.window + 1);
  int32_t* out = P.idx + (int64_t)row * P.top_k;
  if (ncand <= P.top_k) {
    for (int i = threadIdx.x; i < P.top_k; i += kSelThreads) out[i] = i < ncand ? i : -1;
    return;
  }
  DenseSrc src{P.sigma + (int64_t)row * P.sigma_stride};
  topk_any<true>(sh, lds.key, lds.idx, src, ncand, P.top_k, out);
}

hipError_t launch_select_prefill(const SelectParams& p, int64_t rows, hipStream_t s) {
  if (p.cap > kRegCap)
    select_prefill_kernel<true><<<dim3((unsigned)rows), dim3(kSelThreads), 0, s>>>(p);
  else
    select_prefill_kernel<false><<<dim3((unsigned)rows), dim3(kSelThreads), 0, s>>>(p);
  return hipGetLastError();
}
hipError_t launch_threshold(const ThresholdParams& p, int64_t rows, hipStream_t s) {
  threshold_kernel<<<dim3((unsigned)rows), dim3(kSelThreads), 0, s>>>(p);
  return hipGetLastError();
}
hipError_t launch_select_decode(const SelectDecodeParams& p, int rows, hipStream_t s) {
  select_decode_kernel<<<dim3((unsigned)rows), dim3(kSelThreads), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace hs
