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
#include <algorithm>

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
// dimension order; with per-head log-sum-exps ls, the probability score
// max_h fl(scale * <q_h, k_j> - ls_h).
struct RescanSrc {
  const float* qs;  // LDS [G][128]
  const uint16_t* krow0;
  int64_t kstride;
  int G;
  float scale;
  const float* ls;  // LDS [G] or null
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
      if (h < G) best = fmaxf(best, ls ? fmaf(acc[h], scale, -ls[h]) : acc[h] * scale);
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
static_assert(kRegCap == kSelRegKeys, "host and device agree on the register path's capacity");
constexpr int kSamples = 2048;

struct RadixResult {
  uint32_t prefix;  // decided high bits of the threshold key
  uint32_t mask;    // which bits are decided
  uint32_t need;    // elements still needed among those equal to prefix
  bool take_all;    // every element equal to prefix (under mask) is selected
};

constexpr int kHistCopies = 8;
constexpr int kHistStride = 256 + 64 / kHistCopies;  // words per copy: bins + dump slots

// Block-wide form of wave_radix over the register keys of all kSelThreads
// threads (slots e < eslots, wave-uniform; 0 = empty): the bits all keys
// share are decided from a block min/max, then 8-bit digits, counted into
// kBlkCopies copies per wave (each lane into copy lane % kBlkCopies of its
// wave's set, so lanes with equal digits mostly hit different words), and
// every wave picks the digit from the summed copies itself. A plain block
// radix sent all of a row's keys to one or two bins in its first passes
// (scores share their sign and leading exponent bits), and the LDS atomics
// of a wave to one word serialise. `hist` holds kBlkHistWords words; the
// min/max exchange uses sh.wave_tot and sh.cnt.
constexpr int kBlkCopies = 4;                      // histogram copies per wave
constexpr int kBlkStride = 256 + 64 / kBlkCopies;  // words per copy: bins + dump slots
constexpr int kBlkHistWords = kSelWaves * kBlkCopies * kBlkStride;

template <int E>
__device__ RadixResult block_radix(SelShared& sh, uint32_t* hist, const uint32_t (&key)[E], int eslots,
                                   uint32_t rank) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t kmax = 0u, kmin = 0xffffffffu;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kmax = key[e] > kmax ? key[e] : kmax;
    kmin = (key[e] && key[e] < kmin) ? key[e] : kmin;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t a = (uint32_t)__shfl_xor((int)kmax, o, 64), c = (uint32_t)__shfl_xor((int)kmin, o, 64);
    kmax = a > kmax ? a : kmax;
    kmin = c < kmin ? c : kmin;
  }
  if (lane == 0) {
    sh.wave_tot[wave] = kmax;
    sh.cnt[wave] = kmin;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    kmax = sh.wave_tot[w] > kmax ? sh.wave_tot[w] : kmax;
    kmin = sh.cnt[w] < kmin ? sh.cnt[w] : kmin;
  }
  RadixResult r{kmax, 0xffffffffu, rank, false};
  const uint32_t diff = kmax ^ kmin;
  if (diff == 0u) {  // every key equal: the first `rank` in index order
    __syncthreads();  // the exchange words are read before anyone reuses them
    return r;
  }
  int hi = 31 - __builtin_clz(diff);
  r.mask = hi == 31 ? 0u : ~((2u << hi) - 1u);
  r.prefix = kmax & r.mask;
  uint32_t* my = hist + (wave * kBlkCopies + lane % kBlkCopies) * kBlkStride;
#pragma unroll 1
  while (hi >= 0) {
    const int shift = imax(hi - 7, 0);
    const uint32_t dmask = (2u << (hi - shift)) - 1u;
    __syncthreads();  // earlier readers of this LDS (the previous pass, or the caller's) are done
    for (int i = threadIdx.x; i < kBlkHistWords / 4; i += kSelThreads)
      reinterpret_cast<u32x4*>(hist)[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    const uint32_t lim = hi == 31 ? 0xffffffffu : (2u << hi) - 1u;
    const uint32_t dump = 256u + (uint32_t)(lane / kBlkCopies);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (e < eslots) {  // wave-uniform
        const uint32_t d = key[e] - r.prefix;
        atomicAdd(&my[(key[e] != 0u && d <= lim) ? d >> shift : dump], 1u);
      }
    }
    __syncthreads();
    // lane l owns digits 255 - 4l - q (descending): bins 252 - 4l .. 255 - 4l
    u32x4 cv = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int cp = 0; cp < kSelWaves * kBlkCopies; ++cp)
      cv += *reinterpret_cast<const u32x4*>(hist + cp * kBlkStride + 252 - 4 * lane);
    const uint32_t c[4] = {cv[3], cv[2], cv[1], cv[0]};
    const int local = (int)(c[0] + c[1] + c[2] + c[3]);
    const int incl = wave_incl_scan(local);
    const uint64_t hit = ballot((uint32_t)incl >= r.need);
    const int L = __builtin_ctzll(hit);  // first lane reaching the rank
    uint32_t acc = (uint32_t)(incl - local), dsel = 0u, gt = 0u, eq = 0u;
    bool found = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (!found && acc + c[q] >= r.need) {
        found = true;
        dsel = 255u - 4u * (uint32_t)lane - (uint32_t)q;
        gt = acc;
        eq = c[q];
      }
      acc += c[q];
    }
    dsel = (uint32_t)__builtin_amdgcn_readlane((int)dsel, L);
    gt = (uint32_t)__builtin_amdgcn_readlane((int)gt, L);
    eq = (uint32_t)__builtin_amdgcn_readlane((int)eq, L);
    r.prefix |= dsel << shift;
    r.mask |= dmask << shift;
    r.need -= gt;
    if (eq == r.need) {
      r.take_all = true;
      break;
    }
    hi = shift - 1;
  }
  __syncthreads();  // every wave has read the histograms: callers may reuse that LDS
  return r;
}

// The four largest of a thread's register keys (descending; 0 = empty), by
// insertion with min/max pairs. A sampled threshold only needs a lower bound
// on the m-th largest sample, and the m-th largest of any subset is one: the
// m-th largest of the union of every thread's top four equals it unless some
// thread holds five of the top m (for m = 113 of 16384 samples, 64 per
// thread, about one row in 40), and is a little lower then. The radix over
// that union (all from the upper tail, so the bits they share are skipped)
// avoids most LDS atomics; over all samples, which span both signs, the
// first digit sends nearly every lane to a few bins.
template <int E>
__device__ __forceinline__ void top4_regs(const uint32_t (&key)[E], uint32_t (&t)[4]) {
  t[0] = t[1] = t[2] = t[3] = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    uint32_t x = key[e];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const uint32_t hi = t[i] > x ? t[i] : x, lo = t[i] > x ? x : t[i];
      t[i] = hi;
      x = lo;
    }
    t[3] = t[3] > x ? t[3] : x;
  }
}

// Exact top-k (k < n <= E * kSelThreads) of an index-ordered source; writes
// the k selected indices ascending to out. Each thread holds a contiguous run
// of the source in E registers.
template <int E, class Src>
__device__ void topk_regs_e(SelShared& sh, uint32_t* hist, const Src& src, int n, int k, int32_t* out) {
  const int run = __builtin_amdgcn_readfirstlane((n + kSelThreads - 1) / kSelThreads);  // block-uniform
  const int beg = threadIdx.x * run;
  // Keys in groups of 8 slots (block-uniform test), each group's reads issued
  // together at clamped in-range positions and masked afterwards: a read
  // under a per-element condition made the compiler wait for each in turn.
  static_assert(E % 8 == 0, "slots in groups of 8");
  uint32_t key[E];
#pragma unroll
  for (int e0 = 0; e0 < E; e0 += 8) {
    if (e0 < run) {
#pragma unroll
      for (int u = 0; u < 8; ++u) key[e0 + u] = src.key(imin(beg + e0 + u, n - 1));
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) key[e0 + u] = 0u;
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] &= 0u - (uint32_t)(e < run && beg + e < n);
  const RadixResult r = block_radix<E>(sh, hist, key, run, (uint32_t)k);
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (!key[e]) continue;
    const uint32_t km = key[e] & r.mask;
    ngt += km > r.prefix;
    neq += km == r.prefix;
  }
  const uint32_t excl = block_excl_scan(sh, ngt | (neq << 16));
  const uint32_t eq_before = excl >> 16;
  uint32_t pos = (excl & 0xffffu) + (r.take_all ? eq_before : (eq_before < r.need ? eq_before : r.need));
  uint32_t eq_rank = eq_before;
  // indices read in groups of 8 as the keys were (a read per selected
  // element, under its condition, waited for each in turn)
#pragma unroll
  for (int e0 = 0; e0 < E; e0 += 8) {
    if (e0 < run) {
      int32_t jv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) jv[u] = src.index(imin(beg + e0 + u, n - 1));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t kk = key[e0 + u];
        if (!kk) continue;
        const uint32_t km = kk & r.mask;
        bool sel = km > r.prefix;
        if (km == r.prefix) {
          sel = r.take_all || eq_rank < r.need;
          ++eq_rank;
        }
        if (sel) out[pos++] = jv[u];
      }
    }
  }
}

template <class Src>
__device__ void topk_regs(SelShared& sh, uint32_t* hist, const Src& src, int n, int k, int32_t* out) {
  topk_regs_e<kE>(sh, hist, src, n, k, out);
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
  uint32_t* const hist = lkey;  // the histograms overlay the filter's LDS while it is not in use
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
  const RadixResult r = block_radix<ES>(sh, hist, skey, ES, (uint32_t)m);
  const uint32_t theta = r.prefix;  // keys >= theta include the m largest samples
  // Each wave filters a contiguous quarter of the row into its LDS region.
  constexpr int kRegion = kRegCap / kSelWaves;
  const int q0 = (int)(((int64_t)n * wave) / kSelWaves), q1 = (int)(((int64_t)n * (wave + 1)) / kSelWaves);
  uint32_t cnt = 0;
  // kFilterBatch loads in flight per lane: a long row is read at memory
  // throughput rather than one latency per 64 elements
  constexpr int kFilterBatch = 16;
  for (int i0 = q0; i0 < q1; i0 += 64 * kFilterBatch) {
    uint32_t kb[kFilterBatch];
#pragma unroll
    for (int u = 0; u < kFilterBatch; ++u) kb[u] = src.key(imin(i0 + 64 * u + lane, q1 - 1));  // clamped
#pragma unroll
    for (int u = 0; u < kFilterBatch; ++u) {
      const int i = i0 + 64 * u + lane;
      const bool pass = i < q1 && kb[u] >= theta;
      const uint64_t bm = ballot(pass);
      const uint32_t pos = cnt + lane_prefix(bm);
      if (pass && pos < (uint32_t)kRegion) {
        lkey[wave * kRegion + pos] = kb[u];
        lidx[wave * kRegion + pos] = src.index(i);
      }
      cnt += (uint32_t)__popcll(bm);
    }
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
  topk_regs(sh, hist, LdsSrc{lkey, lidx}, (int)total, k, out);
  return true;
}

// ---------------------------------------------------------------- kernels

// Dispatch by row length: registers, LDS filter (BIG kernels only), stream.
// `hist` (kBlkHistWords words) may be lkey in BIG kernels.
template <bool BIG, class Src>
__device__ void topk_any(SelShared& sh, uint32_t* hist, uint32_t* lkey, int32_t* lidx, const Src& src, int n, int k,
                         int32_t* out) {
  if (n <= kRegCap) {
    topk_regs(sh, hist, src, n, k, out);
    return;
  }
  if constexpr (BIG) {
    if (topk_filtered(sh, lkey, lidx, src, n, k, out)) return;
  }
  topk_stream(sh, src, n, k, out);
}

template <bool BIG>
struct SelLds {
  __attribute__((aligned(16))) uint32_t key[BIG ? kRegCap : 1];
  int32_t idx[BIG ? kRegCap : 1];
};

// ---------------------------------------------------------------- wave path

// Wave-level radix search over lane-strided register keys (0 = empty) for the
// element of rank `rank` (1-based, largest first). The bits above the highest
// bit in which the keys differ are decided up front (scores in one row share
// sign and leading exponent bits), then 8-bit digits follow from there; the
// search stops early once a whole bucket is needed. Keys sit at slot e of
// lane l for element 64e + l < n. `hist` is this wave's LDS histogram in
// kHistCopies copies (lane l counts into copy l % copies: scores cluster in
// few digits, and LDS atomics from many lanes to one address serialise),
// each with 256 digit bins and one dump slot per lane of the copy for the
// keys outside the current prefix, so every lane adds unconditionally (a
// wave's LDS operations execute in order).

template <int E>
__device__ RadixResult wave_radix(uint32_t* hist, const uint32_t (&key)[E], int n, uint32_t rank) {
  const int lane = threadIdx.x & 63;
  uint32_t kmax = 0u, kmin = 0xffffffffu;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kmax = key[e] > kmax ? key[e] : kmax;
    kmin = (key[e] && key[e] < kmin) ? key[e] : kmin;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t a = (uint32_t)__shfl_xor((int)kmax, o, 64), c = (uint32_t)__shfl_xor((int)kmin, o, 64);
    kmax = a > kmax ? a : kmax;
    kmin = c < kmin ? c : kmin;
  }
  kmax = (uint32_t)uniform((int)kmax);
  kmin = (uint32_t)uniform((int)kmin);
  RadixResult r{kmax, 0xffffffffu, rank, false};
  const uint32_t diff = kmax ^ kmin;
  if (diff == 0u) return r;  // every key equal: the first `rank` in index order
  int hi = 31 - __builtin_clz(diff);
  r.mask = hi == 31 ? 0u : ~((2u << hi) - 1u);
  r.prefix = kmax & r.mask;
  uint32_t* my = hist + (lane % kHistCopies) * kHistStride;
#pragma unroll 1
  while (hi >= 0) {
    const int shift = imax(hi - 7, 0);
    const uint32_t dmask = (2u << (hi - shift)) - 1u;
    for (int i = lane; i < kHistCopies * kHistStride / 4; i += 64)
      reinterpret_cast<u32x4*>(hist)[i] = u32x4{0u, 0u, 0u, 0u};
    // key in the current prefix <=> key - prefix <= lim = 2^(hi+1) - 1; its
    // digit is then (key - prefix) >> shift. Anything else (empty slots
    // included, prefix being nonzero) goes to the dump bin.
    const uint32_t lim = hi == 31 ? 0xffffffffu : (2u << hi) - 1u;
    const uint32_t dump = 256u + (uint32_t)(lane / kHistCopies);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (64 * e < n) {  // wave-uniform: slots past the row are skipped
        const uint32_t d = key[e] - r.prefix;
        atomicAdd(&my[(key[e] != 0u && d <= lim) ? d >> shift : dump], 1u);
      }
    }
    // lane l owns digits 255 - 4l - q (descending): bins 252 - 4l .. 255 - 4l
    u32x4 cv = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int cp = 0; cp < kHistCopies; ++cp) cv += *reinterpret_cast<const u32x4*>(hist + cp * kHistStride + 252 - 4 * lane);
    const uint32_t c[4] = {cv[3], cv[2], cv[1], cv[0]};
    const int local = (int)(c[0] + c[1] + c[2] + c[3]);
    const int incl = wave_incl_scan(local);
    const uint64_t hit = ballot((uint32_t)incl >= r.need);
    const int L = __builtin_ctzll(hit);  // first lane reaching the rank
    uint32_t acc = (uint32_t)(incl - local), dsel = 0u, gt = 0u, eq = 0u;
    bool found = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (!found && acc + c[q] >= r.need) {
        found = true;
        dsel = 255u - 4u * (uint32_t)lane - (uint32_t)q;
        gt = acc;
        eq = c[q];
      }
      acc += c[q];
    }
    dsel = (uint32_t)__builtin_amdgcn_readlane((int)dsel, L);
    gt = (uint32_t)__builtin_amdgcn_readlane((int)gt, L);
    eq = (uint32_t)__builtin_amdgcn_readlane((int)eq, L);
    r.prefix |= dsel << shift;
    r.mask |= dmask << shift;
    r.need -= gt;
    if (eq == r.need) {
      r.take_all = true;
      break;
    }
    hi = shift - 1;
  }
  return r;
}

constexpr int kWaveE = 80;       // candidates per lane of the wave path (rows of up to 5120)
constexpr int kWaveEBig = 128;   // the same for calls whose rows expect more (rows of up to 8192)

// One wave per (b, t, g) row: the candidate buffer is read lane-strided
// (coalesced) into registers, the k-th key is found by wave_radix, and the
// selection is written in ascending token order with one ballot per
// register slot (ties at the k-th key are taken in token order). Rows the
// wave path cannot take (forced rescan, a count outside [k, cap], or more
// candidates than it holds) are queued for the block-wide path.
template <int E>  // register slots per lane: rows of up to 64 * E candidates
__global__ __launch_bounds__(256, E > kWaveE ? 2 : 3) void select_prefill_wave_kernel(SelectParams P, int64_t rows) {
  __shared__ __attribute__((aligned(16))) uint32_t hist_all[4][kHistCopies * kHistStride];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = uniform((int)blockIdx.x * 4 + wave);  // rows < 2^31
  if (row >= rows) return;
  const int64_t bt = row / P.Hkv;
  const int t = (int)(bt % P.n_q);
  const int p = P.n_kv - P.n_q + t;
  const int ncand = imax(0, p - P.window + 1);
  const int k = P.top_k;
  int32_t* out = P.idx + row * k;
  if (ncand <= k) {
    // reading: fewer candidates than k -> all of C(p), then -1 padding
    for (int i = lane; i < k; i += 64) out[i] = i < ncand ? i : -1;
    return;
  }
  const int cnt = uniform(P.counts[row]);
  if (P.force_rescan || cnt < k || cnt > P.cap || cnt > 64 * E) {
    if (lane == 0) P.defer_rows[atomicAdd(P.defer_count, 1u)] = (int32_t)row;
    return;
  }
  // loads past the row's count return 0 (buffer range check), so no clamping
  const __amdgpu_buffer_rsrc_t rs_s = make_rsrc_sized(P.buf_sigma + row * (int64_t)P.cap, 4u * (uint32_t)cnt);
  const __amdgpu_buffer_rsrc_t rs_j = make_rsrc_sized(P.buf_j + row * (int64_t)P.cap, 4u * (uint32_t)cnt);
  // selected indices: stores of unselected lanes aim past the row (dropped)
  const __amdgpu_buffer_rsrc_t rs_o = make_rsrc_sized(out, 4u * (uint32_t)k);
  if (cnt == k) {
    for (int i = lane; i < k; i += 64) out[i] = P.buf_j[row * (int64_t)P.cap + i];
    return;
  }
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {  // slots past the count: no load issued (wave-uniform branch)
    key[e] = 0u;
    if (64 * e < cnt) key[e] = buf_ld4(rs_s, 4u * (uint32_t)lane + 256u * (uint32_t)e);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = 64 * e + lane < cnt ? score_key(__uint_as_float(key[e])) : 0u;
  const RadixResult r = wave_radix<E>(hist_all[wave], key, cnt, (uint32_t)k);
  uint32_t out_run = 0, eq_run = 0;
  constexpr int kGroup = 8;  // index loads in flight per step (bounds register use)
#pragma unroll
  for (int e0 = 0; e0 < E; e0 += kGroup) {
    if (64 * e0 >= cnt) continue;  // (not break: the loop stays fully unrolled)
    uint32_t j[kGroup];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) j[u] = buf_ld4(rs_j, 4u * (uint32_t)lane + 256u * (uint32_t)(e0 + u));
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const uint32_t kk = key[e0 + u];
      const uint32_t km = kk & r.mask;
      const bool gt = kk != 0u && km > r.prefix;
      const bool eq = kk != 0u && km == r.prefix;
      const uint64_t eqm = ballot(eq);
      const uint32_t eq_before = eq_run + lane_prefix(eqm);
      eq_run += (uint32_t)__popcll(eqm);
      const bool sel = gt || (eq && (r.take_all || eq_before < r.need));
      const uint64_t selm = ballot(sel);
      buf_st4(rs_o, sel ? 4u * (out_run + lane_prefix(selm)) : kDropOffset, j[u]);
      out_run += (uint32_t)__popcll(selm);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Block-wide top-k of one (b, t, g) row of a prefill call (the rows the wave
// path queued): buffer path when the candidate count proves the buffer holds
// the top k, exact rescan otherwise.
template <bool BIG>
__device__ void select_prefill_row(const SelectParams& P, int64_t row, SelShared& sh, uint32_t* hist, SelLds<BIG>& lds,
                                   float* qs) {
  const int g = (int)(row % P.Hkv);
  const int64_t bt = row / P.Hkv;
  const int t = (int)(bt % P.n_q);
  const int b = (int)(bt / P.n_q);
  const int p = P.n_kv - P.n_q + t;
  const int ncand = imax(0, p - P.window + 1);
  int32_t* out = P.idx + row * P.top_k;
  if (ncand <= P.top_k) {
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
    topk_any<BIG>(sh, hist, lds.key, lds.idx, src, cnt, P.top_k, out);
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
  float* ls = qs + G * kHeadDim;  // the group's log-sum-exps (probability score)
  if (P.lse && threadIdx.x < G) ls[threadIdx.x] = P.lse[((int64_t)b * P.Hq + g * G + threadIdx.x) * P.n_q + t];
  __syncthreads();
  RescanSrc src{qs, P.kv.slab(b, g), P.kv.st, G, P.scale, P.lse ? ls : nullptr};
  topk_any<BIG>(sh, hist, lds.key, lds.idx, src, ncand, P.top_k, out);
  if (threadIdx.x == 0 && P.rescan_count) atomicAdd(P.rescan_count, 1u);
}

// Persistent blocks over the queued rows.
template <bool BIG>
__global__ __launch_bounds__(kSelThreads) void select_prefill_deferred_kernel(SelectParams P) {
  __shared__ SelShared sh;
  __shared__ SelLds<BIG> lds;
  __shared__ __attribute__((aligned(16))) uint32_t hist_own[BIG ? 4 : kBlkHistWords];
  __shared__ float qs[8 * kHeadDim + 8];
  uint32_t* const hist = BIG ? lds.key : hist_own;  // BIG: the histograms overlay the key array
  const uint32_t n = *reinterpret_cast<volatile const uint32_t*>(P.defer_count);
  for (uint32_t li = blockIdx.x; li < n; li += gridDim.x) {
    select_prefill_row<BIG>(P, P.defer_rows[li], sh, hist, lds, qs);
    __syncthreads();
  }
}

// Per-row filter threshold from sampled scores: theta = the m-th largest valid
// sample, with m chosen so that, for exchangeable scores, the full candidate
// set holds at least top_k scores >= theta except with negligible
// probability (mean + 6 standard deviations of the sampled count above the
// true k-th score, plus one). Rows whose candidates all fit the buffer (and
// the wave selection path, when samples exist) get theta = -inf.
__global__ __launch_bounds__(kSelThreads) void threshold_kernel(ThresholdParams P) {
  __shared__ SelShared sh;
  __shared__ __attribute__((aligned(16))) uint32_t hist[kBlkHistWords];
  const int64_t row = blockIdx.x;
  if (row == 0 && threadIdx.x == 0 && P.defer_count) P.defer_count[0] = P.defer_count[1] = 0u;
  const int64_t bt = row / P.Hkv;
  const int t = (int)(bt % P.n_q);
  const int p = P.n_kv - P.n_q + t;
  const int ncand = imax(0, p - P.window + 1);
  // Whole rows go to the buffer when they fit it and, if samples exist, also
  // fit the wave selection path; longer rows get a sampled threshold.
  if (ncand <= P.cap && (P.max_samples == 0 || ncand <= 64 * kWaveE)) {
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
  constexpr int kThrE = 64;  // samples per thread in registers: rows of up to 16384 samples
  if (nsamp <= kThrE * kSelThreads) {
    // thread t holds samples 4(t + 256e) .. +3: 16-byte loads, coalesced
    const __amdgpu_buffer_rsrc_t rs = make_rsrc_sized(src.s, 4u * (uint32_t)nsamp);
    const int slots = (nsamp + 4 * kSelThreads - 1) / (4 * kSelThreads);  // 16-byte loads holding samples
    // all loads first and unconditionally (past the row: range-checked, read as 0), then the keys
    u32x4 v[kThrE / 4];
#pragma unroll
    for (int e = 0; e < kThrE / 4; ++e) v[e] = buf_ld16(rs, 16u * (uint32_t)((int)threadIdx.x + kSelThreads * e));
    uint32_t key[kThrE];
#pragma unroll
    for (int e = 0; e < kThrE / 4; ++e)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        key[4 * e + q] = score_key_if(__uint_as_float(v[e][q]), 4 * ((int)threadIdx.x + kSelThreads * e) + q < nsamp);
    RadixResult r;
    if (m <= 4 * kSelThreads) {
      uint32_t t4[4];
      top4_regs<kThrE>(key, t4);
      r = block_radix<4>(sh, hist, t4, 4, (uint32_t)m);
    } else {
      r = block_radix<kThrE>(sh, hist, key, 4 * slots, (uint32_t)m);
    }
    // take_all leaves the low bits open: prefix is then a lower bound
    if (threadIdx.x == 0) P.theta[row] = key_to_score(r.prefix);
  } else {
    find_kth_key(sh, src, nsamp, (uint32_t)m);
    if (threadIdx.x == 0) P.theta[row] = key_to_score(sh.prefix);
  }
}

// The same threshold with one wave per row, for calls whose rows hold at
// most 64 * kWaveE samples (lane-strided register keys, wave_radix).
template <int E>  // register slots per lane: rows of up to 64 * E samples
__global__ __launch_bounds__(256, 2) void threshold_wave_kernel(ThresholdParams P, int64_t rows) {
  __shared__ __attribute__((aligned(16))) uint32_t hist_all[4][kHistCopies * kHistStride];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = uniform((int)blockIdx.x * 4 + wave);  // rows < 2^31
  if (row >= rows) return;
  if (row == 0 && lane == 0 && P.defer_count) P.defer_count[0] = P.defer_count[1] = 0u;
  const int64_t bt = row / P.Hkv;
  const int t = (int)(bt % P.n_q);
  const int p = P.n_kv - P.n_q + t;
  const int ncand = imax(0, p - P.window + 1);
  if (ncand <= P.cap && (P.max_samples == 0 || ncand <= 64 * kWaveE)) {
    if (lane == 0) P.theta[row] = kNegInf;
    return;
  }
  const int nsamp = (ncand + P.stride - 1) / P.stride;
  const double mu = (double)nsamp * (double)P.top_k / (double)ncand;
  const int m = (int)ceil(mu + 6.0 * sqrt(mu)) + 1;
  if (m > nsamp) {
    if (lane == 0) P.theta[row] = kNegInf;
    return;
  }
  const __amdgpu_buffer_rsrc_t rs = make_rsrc_sized(P.samples + row * (int64_t)P.max_samples, 4u * (uint32_t)nsamp);
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = buf_ld4(rs, 4u * (uint32_t)lane + 256u * (uint32_t)e);
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = 64 * e + lane < nsamp ? score_key(__uint_as_float(key[e])) : 0u;
  const RadixResult r = wave_radix<E>(hist_all[wave], key, nsamp, (uint32_t)m);
  // take_all leaves the low bits open: prefix is then a lower bound
  if (lane == 0) P.theta[row] = key_to_score(r.prefix);
}

// Decode: top-k over the dense score row of each (b, g).
__global__ __launch_bounds__(kSelThreads) void select_decode_kernel(SelectDecodeParams P) {
  __shared__ SelShared sh;
  __shared__ SelLds<true> lds;
  const int row = blockIdx.x;  // b * Hkv + g
  const int b = row / P.Hkv;
  const int p = dec_len(P.seq_lens, b, P.max_len) - 1;
  const int ncand = imax(0, p - P.window + 1);
  int32_t* out = P.idx + (int64_t)row * P.top_k;
  if (ncand <= P.top_k) {
    for (int i = threadIdx.x; i < P.top_k; i += kSelThreads) out[i] = i < ncand ? i : -1;
    return;
  }
  DenseSrc src{P.sigma + (int64_t)row * P.sigma_stride};
  topk_any<true>(sh, lds.key, lds.key, lds.idx, src, ncand, P.top_k, out);
}

// ---------------------------------------------------------------- decode, long rows
//
// A decode score row of a long sequence (a million keys at the 1M-token
// context) is too long for one block to scan at memory speed, and a batch of
// one sequence has only Hkv such rows. Three launches spread it over the chip:
//  1. threshold: one block per row reads the row's S samples (every 2^s-th
//     key, at most kDecSamples, written beside the score row by the kernel
//     that produced it, so this reads 64 KB instead of the row) and takes
//     their m-th largest, m = mu + 6 sqrt(mu) + 1 with mu = k S / n the
//     expected number of samples among the row's top k, so that the k-th
//     largest key of the row lies at or above it with overwhelming
//     probability;
//  2. filter: one wave per (slice of kDecSlice keys, row) keeps the keys at
//     or above the threshold, in index order, with their indices;
//  3. final: one block per row concatenates the slices' survivors in slice
//     order (so still in index order) and selects exactly from them. When
//     the survivors are fewer than k (the threshold overshot) or more than
//     the block holds, it selects from the whole dense row instead, so the
//     result never depends on the sampling.

constexpr int kDecCandCap = 16384;  // survivors the final block holds in LDS
static_assert(kDecCandCap >= kBlkHistWords, "the final block's histograms overlay its key array");

// Exclusive block-wide scan that also returns the block total.
__device__ __forceinline__ uint32_t block_scan_total(SelShared& sh, uint32_t v, uint32_t* total) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t incl = (uint32_t)wave_incl_scan((int)v);
  if (lane == 63) sh.wave_tot[wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
  for (int w = 0; w < kSelWaves; ++w) {
    const uint32_t t = sh.wave_tot[w];
    base += w < wave ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

struct DecRow {
  int ncand;       // |C(p)|
  const float* s;  // dense score row
};
__device__ __forceinline__ DecRow dec_row(const SelectDecodeParams& P, int row) {
  const int b = row / P.Hkv;
  const int p = dec_len(P.seq_lens, b, P.max_len) - 1;
  return DecRow{imax(0, p - P.window + 1), P.sigma + (int64_t)row * P.sigma_stride};
}

__global__ __launch_bounds__(kSelThreads) void select_decode_threshold_kernel(SelectDecodeParams P) {
  __shared__ SelShared sh;
  __shared__ __attribute__((aligned(16))) uint32_t hist[kBlkHistWords];
  const int row = blockIdx.x;
  const DecRow r = dec_row(P, row);
  if (r.ncand <= kRegCap) return;  // selected directly by the final kernel
  const int shift = dec_sample_shift(r.ncand);
  const int nsamp = (r.ncand + (1 << shift) - 1) >> shift;
  const double mu = (double)P.top_k * nsamp / (double)r.ncand;
  const int m = (int)ceil(mu + 6.0 * sqrt(mu)) + 1;
  if (m >= nsamp) {  // the samples cannot bound the k-th key: no filter
    if (threadIdx.x == 0) P.theta_key[row] = 0u;
    return;
  }
  // thread t holds samples 4(t + 256e) .. +3: contiguous 16-byte loads
  constexpr int ES = kDecSamples / kSelThreads;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc_sized(P.samp + (int64_t)row * kDecSamples, 4u * (uint32_t)nsamp);
  u32x4 v[ES / 4];  // all loads first (past the samples: range-checked, read as 0), then the keys
#pragma unroll
  for (int e = 0; e < ES / 4; ++e) v[e] = buf_ld16(rs, 16u * (uint32_t)((int)threadIdx.x + kSelThreads * e));
  uint32_t skey[ES];
#pragma unroll
  for (int e = 0; e < ES / 4; ++e)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      skey[4 * e + q] = score_key_if(__uint_as_float(v[e][q]), 4 * ((int)threadIdx.x + kSelThreads * e) + q < nsamp);
  RadixResult rr;
  if (m <= 4 * kSelThreads) {  // the union of per-thread top fours (a lower bound, usually exact)
    uint32_t t4[4];
    top4_regs<ES>(skey, t4);
    rr = block_radix<4>(sh, hist, t4, 4, (uint32_t)m);
  } else {
    rr = block_radix<ES>(sh, hist, skey, ES, (uint32_t)m);
  }
  // keys >= prefix include the m largest samples (take_all leaves the low
  // bits of prefix zero: still a lower bound)
  if (threadIdx.x == 0) P.theta_key[row] = rr.prefix;
}

// One wave per slice (kDecSlice keys of a row; a block holds four slices of
// one row). Load j of lane l reads keys 256j + 4l .. +3 of the slice, so
// every load is one contiguous 1 KB piece of the row, and all 16 are issued
// up front. Survivors are emitted in index order (per load, then lane, then
// q; positions from four ballots) as soon as each load lands, while the later
// ones are still in flight: each slice has its own output segment, so no
// wave waits for another (a block-wide count exchange before the emission
// held every resident block in step, loads then emission, and cost 40% of the
// kernel). They pass through the wave's LDS ring in order and leave in runs
// of 64 consecutive entries (one coalesced store per array), not as one
// scattered store per survivor bit position. About 2% of the keys survive.
constexpr int kRing = 512;  // per-wave LDS ring of the filter's survivors

__global__ __launch_bounds__(kSelThreads) void select_decode_filter_kernel(SelectDecodeParams P) {
  __shared__ uint32_t ring_key[kSelWaves][kRing];
  __shared__ int32_t ring_idx[kSelWaves][kRing];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slice = (int)blockIdx.x * kSelWaves + wave, row = blockIdx.y;
  if (slice >= P.nslices) return;
  const DecRow r = dec_row(P, row);
  if (r.ncand <= kRegCap) return;  // selected directly by the final kernel
  const int i0 = slice * kDecSlice;
  const int n = imin(r.ncand, i0 + kDecSlice) - i0;
  const int64_t seg = (int64_t)row * P.nslices + slice;
  if (n <= 0) {
    if (lane == 0) P.seg_count[seg] = 0u;
    return;
  }
  const uint32_t theta = P.theta_key[row];
  constexpr int kLoads = kDecSlice / 256;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc_sized(r.s + i0, 4u * (uint32_t)n);
  u32x4 v[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j)  // past the slice's end: range-checked, read as 0 (only a row's last slice)
    v[j] = buf_ld16(rs, 4u * (uint32_t)(256 * j + 4 * lane));
  const int lim = n - 4 * lane;  // key 256j + q of this lane lies in the slice iff 256j + q < lim
  uint32_t* okey = P.seg_key + seg * kDecSlice;
  int32_t* oidx = P.seg_idx + seg * kDecSlice;
  uint32_t* rkey = ring_key[wave];
  int32_t* ridx = ring_idx[wave];
  uint32_t tail = 0, head = 0;  // entries appended to / written out of the ring (wave-uniform)
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    // survivor bits, branch-free (a short-circuit test per key became a
    // branch per key, and the branches made the first test wait for every load)
    uint32_t m4 = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      m4 |= ((uint32_t)(256 * j + q < lim) & (uint32_t)(score_key(__uint_as_float(v[j][q])) >= theta)) << q;
    if (ballot(m4 != 0u) == 0) continue;  // wave-uniform
    uint32_t pos = tail;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint64_t bq = ballot((m4 >> q) & 1u);
      pos += lane_prefix(bq);
      tail += (uint32_t)__popcll(bq);
    }
    const int e0 = i0 + 256 * j + 4 * lane;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if ((m4 >> q) & 1u) {
        rkey[pos & (kRing - 1)] = v[j][q];  // the score's bits (the final kernel takes their key)
        ridx[pos & (kRing - 1)] = e0 + q;
        ++pos;
      }
    }
    if (tail - head >= kRing / 2) {  // a load adds at most 256 < kRing / 2 entries: no overrun
#pragma unroll
      for (int c = 0; c < kRing / 128; ++c) {
        const uint32_t i = head + 64u * (uint32_t)c + (uint32_t)lane;
        okey[i] = rkey[i & (kRing - 1)];
        oidx[i] = ridx[i & (kRing - 1)];
      }
      head += kRing / 2;
    }
  }
  for (uint32_t i = head + (uint32_t)lane; i < tail; i += 64) {
    okey[i] = rkey[i & (kRing - 1)];
    oidx[i] = ridx[i & (kRing - 1)];
  }
  if (lane == 0) P.seg_count[seg] = tail;
}

struct DecLds {
  __attribute__((aligned(16))) uint32_t key[kDecCandCap];
  int32_t idx[kDecCandCap];
  uint32_t off[kMaxDecSlices + 1];
};

__global__ __launch_bounds__(kSelThreads) void select_decode_final_kernel(SelectDecodeParams P) {
  __shared__ SelShared sh;
  __shared__ DecLds lds;
  const int row = blockIdx.x;
  const DecRow r = dec_row(P, row);
  const int k = P.top_k;
  int32_t* out = P.idx + (int64_t)row * k;
  if (r.ncand <= k) {
    for (int i = threadIdx.x; i < k; i += kSelThreads) out[i] = i < r.ncand ? i : -1;
    return;
  }
  const DenseSrc dense{r.s};
  if (r.ncand <= kRegCap) {
    topk_regs_e<kE>(sh, lds.key, dense, r.ncand, k, out);
    return;
  }
  const int ns = (r.ncand + kDecSlice - 1) / kDecSlice;  // <= nslices <= kMaxDecSlices
  const uint32_t* cnt = P.seg_count + (int64_t)row * P.nslices;
  const int per = (ns + kSelThreads - 1) / kSelThreads;
  const int s0 = imin(ns, threadIdx.x * per), s1 = imin(ns, s0 + per);
  uint32_t local = 0;
  for (int i = s0; i < s1; ++i) local += cnt[i];
  uint32_t total;
  uint32_t base = block_scan_total(sh, local, &total);
  for (int i = s0; i < s1; ++i) {
    lds.off[i] = base;
    base += cnt[i];
  }
  if (threadIdx.x == 0) lds.off[ns] = total;
  __syncthreads();
  if (total < (uint32_t)k || total > (uint32_t)kDecCandCap) {
    topk_stream(sh, dense, r.ncand, k, out);
    return;
  }
  // Survivors into LDS, in concatenation order. With more than 16 per
  // thread (the 1M context): one slice per wave at a time, lanes e and
  // e + 64 copying the slice's survivors e and e + 64, so each read is one
  // coalesced run, and a wave has 16 slices' reads in flight before it
  // writes any (per-thread runs made every read touch a cache line per
  // lane there). Reads go to clamped in-segment positions; only lanes
  // inside a slice's count write.
  const int run = uniform((int)((total + kSelThreads - 1) / kSelThreads));
  if (run > 16) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    constexpr int kSl = 16;
    const int64_t seg0 = (int64_t)row * P.nslices * kDecSlice;
    for (int sb = wave * kSl; sb < ns; sb += (kSelThreads / 64) * kSl) {
      uint32_t kk[2][kSl], o[kSl], c[kSl];
      int32_t jj[2][kSl];
#pragma unroll
      for (int u = 0; u < kSl; ++u) {
        const int sl = imin(sb + u, ns - 1);
        o[u] = lds.off[sl];
        c[u] = sb + u < ns ? lds.off[sl + 1] - o[u] : 0u;
        const int last = imax((int)c[u] - 1, 0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int64_t p = seg0 + (int64_t)sl * kDecSlice + imin(lane + 64 * h, last);
          kk[h][u] = P.seg_key[p];
          jj[h][u] = P.seg_idx[p];
        }
      }
#pragma unroll
      for (int u = 0; u < kSl; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if ((uint32_t)(lane + 64 * h) < c[u]) {
            lds.key[o[u] + lane + 64 * h] = score_key(__uint_as_float(kk[h][u]));
            lds.idx[o[u] + lane + 64 * h] = jj[h][u];
          }
      // slices holding more than 128 survivors
#pragma unroll 1
      for (int u = 0; u < kSl; ++u) {
        const int sl = sb + u;
        for (uint32_t e = 128u + lane; sl < ns && e < c[u]; e += 64u) {
          const int64_t p = seg0 + (int64_t)sl * kDecSlice + e;
          lds.key[o[u] + e] = score_key(__uint_as_float(P.seg_key[p]));
          lds.idx[o[u] + e] = P.seg_idx[p];
        }
      }
    }
  } else {
    // Shorter runs (64 sequences): thread t copies the contiguous run
    // [t*run, t*run + run) of the concatenation (measured faster there). One
    // binary search over the slice offsets finds the run's first slice; a
    // walk then crosses slice boundaries in order, and every read of a group
    // is issued before the first is used (a binary search per element
    // chained about nine dependent LDS reads per survivor).
    const int beg = (int)threadIdx.x * run;
    int sl = 0;  // the last slice whose offset is <= the run's first position
    {
      const uint32_t b0 = (uint32_t)imin(beg, (int)total - 1);
      int hi = ns;
      while (hi - sl > 1) {
        const int mid = (sl + hi) >> 1;
        if (lds.off[mid] <= b0) sl = mid;
        else hi = mid;
      }
    }
    uint32_t sbase = lds.off[sl], next = lds.off[sl + 1];  // the slice's first position, the next slice's
    const int64_t seg0 = (int64_t)row * P.nslices * kDecSlice;
    constexpr int kCopyGroup = 16;
    for (int e0 = 0; e0 < run; e0 += kCopyGroup) {
      uint32_t src[kCopyGroup];
#pragma unroll
      for (int u = 0; u < kCopyGroup; ++u) {
        const uint32_t i = (uint32_t)imin(beg + e0 + u, (int)total - 1);  // past the run: re-read the last
        while (i >= next) {  // into the following slice (empty slices skipped; off[ns] = total ends it)
          ++sl;
          sbase = next;
          next = lds.off[sl + 1];
        }
        src[u] = (uint32_t)sl * kDecSlice + (i - sbase);
      }
      uint32_t kk[kCopyGroup];
      int32_t jj[kCopyGroup];
#pragma unroll
      for (int u = 0; u < kCopyGroup; ++u) {
        kk[u] = P.seg_key[seg0 + src[u]];
        jj[u] = P.seg_idx[seg0 + src[u]];
      }
#pragma unroll
      for (int u = 0; u < kCopyGroup; ++u) {
        const int i = beg + e0 + u;
        if (e0 + u < run && i < (int)total) {
          lds.key[i] = score_key(__uint_as_float(kk[u]));
          lds.idx[i] = jj[u];
        }
      }
    }
  }
  __syncthreads();
  const LdsSrc ls{lds.key, lds.idx};
  if (total == (uint32_t)k) {
    for (int i = threadIdx.x; i < k; i += kSelThreads) out[i] = lds.idx[i];
  } else if (total <= (uint32_t)kRegCap) {
    topk_regs_e<kE>(sh, lds.key, ls, (int)total, k, out);  // the histograms overlay the keys once in registers
  } else {
    topk_regs_e<kDecCandCap / kSelThreads>(sh, lds.key, ls, (int)total, k, out);
  }
}

// Decode probability-score row (after the full layer has produced lse):
// tiles of 16 keys x 16 columns (the group's G heads, zero columns beyond)
// on v_mfma_f32_16x16x32_bf16, each head's column turned into
// scale * s - lse_h (one rounding), the maximum across the G head lanes,
// one store per 4 keys. Each wave walks kDecScoreWaveKeys keys of one (b, g)
// row with four 16-key chunks (16 loads per lane) in flight.
constexpr int kDecScoreWaveKeys = 256;

template <int G>
__global__ __launch_bounds__(256) void decode_prob_score_kernel(DecodeScoreParams P) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = blockIdx.y;  // b * Hkv + g
  const int b = row / P.Hkv, g = row % P.Hkv;
  const int ncand = imax(0, dec_len(P.seq_lens, b, P.max_len) - P.window);  // p - W + 1 with p = seq_len - 1
  const int j0 = ((int)blockIdx.x * 4 + wave) * kDecScoreWaveKeys;
  if (j0 >= ncand) return;
  const int col = lane & 15, kg = lane >> 4;
  // B operand: head `col` of the group, dims 32s + 8kg .. +8 (zero past G)
  bf16x8 qb[4];
  const uint16_t* qrow = P.q + ((int64_t)b * P.Hq + g * G + (col < G ? col : 0)) * kHeadDim;
#pragma unroll
  for (int s = 0; s < 4; ++s) qb[s] = as_bf16x8(col < G ? ld16(qrow + 32 * s + 8 * kg) : u32x4{0u, 0u, 0u, 0u});
  const float lse_col = col < G && !P.per_head ? P.lse[(int64_t)b * P.Hq + g * G + col] : 0.f;
  const uint16_t* slab = P.kv.slab(b, g);
  float* srow = P.sigma + (int64_t)row * P.sigma_stride;
  // samples for the sliced threshold: scores at multiples of 2^s (jk is a multiple of 4)
  const int samp_shift = dec_sample_shift(ncand);
  const int samp_mask = (1 << samp_shift) - 1;
  const int jend = imin(ncand, j0 + kDecScoreWaveKeys);
  for (int c0 = j0; c0 < jend; c0 += 64) {
    // A operand: key c0 + 16ch + col, dims 32s + 8kg .. +8 (rows past the
    // last candidate read the last one; their scores are not stored)
    u32x4 kw[4][4];
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const int j = imin(c0 + 16 * ch + col, ncand - 1);
      const uint16_t* kr = slab + (uint32_t)(j * P.kv.st);
#pragma unroll
      for (int s = 0; s < 4; ++s) kw[ch][s] = ld16(kr + 32 * s + 8 * kg);
    }
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mfma16x16x32(as_bf16x8(kw[ch][s]), qb[s], acc);
      mfma_settle<kSettle16>(acc);
      // lane (kg, col) holds keys 4kg + i of the chunk for head col
      const int jk = c0 + 16 * ch + 4 * kg;
      if (P.per_head) {  // each head's own scaled logit, its own row
        if (col < G) {
          const int64_t hr = (int64_t)b * P.Hq + g * G + col;
          float* hrow = P.sigma + hr * P.sigma_stride;
          if (P.samp && jk < ncand && (jk & samp_mask) == 0) P.samp[hr * kDecSamples + (jk >> samp_shift)] = acc[0] * P.scale;
          if (jk + 3 < ncand) {
            *reinterpret_cast<f32x4*>(hrow + jk) =
                f32x4{acc[0] * P.scale, acc[1] * P.scale, acc[2] * P.scale, acc[3] * P.scale};
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (jk + i < ncand) hrow[jk + i] = acc[i] * P.scale;
          }
        }
        continue;
      }
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = group_max<G>(col < G ? fmaf(acc[i], P.scale, -lse_col) : kNegInf);
      if (col == 0) {
        if (P.samp && jk < ncand && (jk & samp_mask) == 0) P.samp[(int64_t)row * kDecSamples + (jk >> samp_shift)] = v[0];
        if (jk + 3 < ncand) {
          *reinterpret_cast<f32x4*>(srow + jk) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (jk + i < ncand) srow[jk + i] = v[i];
        }
      }
    }
  }
}

hipError_t launch_decode_prob_score(const DecodeScoreParams& p, hipStream_t s) {
  const unsigned gx = (unsigned)((std::max(p.max_cand, 1) + 4 * kDecScoreWaveKeys - 1) / (4 * kDecScoreWaveKeys));
  const dim3 grid(gx, (unsigned)(p.B * p.Hkv));
  switch (p.Hq / p.Hkv) {
    case 1: decode_prob_score_kernel<1><<<grid, dim3(256), 0, s>>>(p); break;
    case 2: decode_prob_score_kernel<2><<<grid, dim3(256), 0, s>>>(p); break;
    case 4: decode_prob_score_kernel<4><<<grid, dim3(256), 0, s>>>(p); break;
    case 8: decode_prob_score_kernel<8><<<grid, dim3(256), 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Block-level selection: the block scores of C(p) (one per aligned 64-token
// block) go through the same exact top-k as token scores (ties: lower block
// first), and the chosen blocks, ascending, are expanded to their candidate
// tokens (only the last block of C(p) can be partial, and it comes last, so
// the padding stays at the end).
struct BlockRow {
  int ncand, nblk, nb;
};
__device__ __forceinline__ BlockRow block_row(const BlockSelectParams& P, int64_t row) {
  int p;
  if (P.seq_lens) {
    p = dec_len(P.seq_lens, (int)(row / P.Hkv), P.max_len) - 1;
  } else {
    const int t = (int)((row / P.Hkv) % P.n_q);
    p = P.n_kv - P.n_q + t;
  }
  BlockRow r;
  r.ncand = imax(0, p - P.window + 1);
  r.nblk = (r.ncand + 63) / 64;
  r.nb = P.top_k / 64;
  return r;
}

// Rows of up to 64 * kBlkWaveE blocks: one wave per row, block scores in
// registers, the cut found by wave_radix, the chosen blocks listed in LDS in
// ascending order, then written out 64 tokens (one block) per store.
constexpr int kBlkWaveE = 16;
constexpr int kMaxSelBlocks = kMaxTopK / 64;
__global__ __launch_bounds__(256, 2) void select_blocks_wave_kernel(BlockSelectParams P, int64_t rows) {
  __shared__ __attribute__((aligned(16))) uint32_t hist_all[4][kHistCopies * kHistStride];
  __shared__ int32_t chosen_all[4][kMaxSelBlocks];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = uniform64((int64_t)blockIdx.x * 4 + wave);
  if (row >= rows) return;
  const BlockRow br = block_row(P, row);
  int32_t* out = P.idx + row * P.top_k;
  if (br.nblk <= br.nb) {
    for (int i = lane; i < P.top_k; i += 64) out[i] = i < br.ncand ? i : -1;
    return;
  }
  const float* bs = P.blk_score + row * (int64_t)P.blk_stride;
  uint32_t key[kBlkWaveE];
#pragma unroll
  for (int e = 0; e < kBlkWaveE; ++e) {
    const int i = 64 * e + lane;
    key[e] = i < br.nblk ? score_key(bs[i]) : 0u;
  }
  const RadixResult r = wave_radix<kBlkWaveE>(hist_all[wave], key, br.nblk, (uint32_t)br.nb);
  int32_t* chosen = chosen_all[wave];
  uint32_t out_run = 0, eq_run = 0;
#pragma unroll
  for (int e = 0; e < kBlkWaveE; ++e) {
    if (64 * e >= br.nblk) continue;
    const uint32_t kk = key[e];
    const uint32_t km = kk & r.mask;
    const bool gt = kk != 0u && km > r.prefix;
    const bool eq = kk != 0u && km == r.prefix;
    const uint64_t eqm = ballot(eq);
    const uint32_t eq_before = eq_run + lane_prefix(eqm);
    eq_run += (uint32_t)__popcll(eqm);
    const bool sel = gt || (eq && (r.take_all || eq_before < r.need));
    const uint64_t selm = ballot(sel);
    if (sel) chosen[out_run + lane_prefix(selm)] = 64 * e + lane;
    out_run += (uint32_t)__popcll(selm);
  }
  // the wave's LDS writes are complete before its reads below
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  for (int b = 0; b < P.top_k / 64; ++b) {
    const int j = b < br.nb ? chosen[b] * 64 + lane : br.ncand;
    out[64 * b + lane] = j < br.ncand ? j : -1;
  }
}

// Longer rows: one block per row, through the block-wide top-k.
__global__ __launch_bounds__(kSelThreads) void select_blocks_kernel(BlockSelectParams P) {
  __shared__ SelShared sh;
  __shared__ SelLds<true> lds;
  __shared__ int32_t chosen[kMaxSelBlocks];
  const int64_t row = blockIdx.x;
  const BlockRow br = block_row(P, row);
  int nsel = br.nblk;
  if (br.nblk <= br.nb) {
    for (int i = threadIdx.x; i < br.nblk; i += kSelThreads) chosen[i] = i;
  } else {
    topk_any<true>(sh, lds.key, lds.key, lds.idx, DenseSrc{P.blk_score + row * P.blk_stride}, br.nblk, br.nb, chosen);
    nsel = br.nb;
  }
  __syncthreads();
  int32_t* out = P.idx + row * P.top_k;
  for (int i = threadIdx.x; i < P.top_k; i += kSelThreads) {
    const int r = i >> 6;
    int v = -1;
    if (r < nsel) {
      const int j = chosen[r] * 64 + (i & 63);
      if (j < br.ncand) v = j;
    }
    out[i] = v;
  }
}

// Decode: block scores of each (b, g) row from its dense score row. A wave
// reads 1 KB (four blocks) per load, 16 lanes to a block, each lane's four
// scores reduced in registers and then across its 16 lanes; a 256-thread
// block covers 64 blocks.
__global__ __launch_bounds__(256) void block_max_kernel(BlockMaxParams P) {
  const int row = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ncand = imax(0, dec_len(P.seq_lens, row / P.Hkv, P.max_len) - P.window);
  const int blk0 = blockIdx.x * 64 + wave * 16;  // first of the wave's 16 blocks
  if (blk0 * 64 >= ncand) return;
  const float* s = P.sigma + (int64_t)row * P.sigma_stride;
  f32x4 x[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = (blk0 + 4 * u) * 64 + 4 * lane;  // first of this lane's four keys
    x[u] = j < ncand ? *reinterpret_cast<const f32x4*>(s + j) : f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = (blk0 + 4 * u) * 64 + 4 * lane;
    float v = kNegInf;
#pragma unroll
    for (int e = 0; e < 4; ++e) v = j + e < ncand ? fmaxf(v, x[u][e]) : v;
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    v = fmaxf(v, dpp<kDppMirror>(v));
    const int blk = blk0 + 4 * u + lane / 16;
    if ((lane & 15) == 0 && blk * 64 < ncand) P.blk_score[(int64_t)row * P.blk_stride + blk] = v;
  }
}

// Union of the G heads' top-k lists of one row: a bitmap over a window of
// kUnionWords * 32 token positions in LDS takes every listed token of the
// window (LDS atomic or), then the set bits are emitted in ascending order
// (each thread scans a contiguous run of words at its exclusive prefix of the
// bit counts); windows follow one another up to |C(p)|.
constexpr int kUnionWords = 8192;
__global__ __launch_bounds__(kSelThreads) void head_union_kernel(UnionParams P) {
  __shared__ uint32_t bits[kUnionWords];
  __shared__ SelShared sh;
  const int64_t row = blockIdx.x;
  int p;
  if (P.seq_lens) {
    p = dec_len(P.seq_lens, (int)(row / P.Hkv), P.max_len) - 1;
  } else {
    p = P.n_kv - P.n_q + (int)((row / P.Hkv) % P.n_q);
  }
  const int ncand = imax(0, p - P.window + 1);
  const int width = P.G * P.k;
  int32_t* out = P.out + row * width;
  const int tid = threadIdx.x;
  int emitted = 0;
  for (int w0 = 0; w0 < ncand; w0 += 32 * kUnionWords) {
    const int nw = imin(kUnionWords, (ncand - w0 + 31) / 32);
    const int wend = imin(ncand, w0 + 32 * kUnionWords);
    for (int i = tid; i < nw; i += kSelThreads) bits[i] = 0u;
    __syncthreads();
    for (int r = 0; r < P.G; ++r) {
      const int32_t* L = P.lists + row * P.row_stride + (int64_t)r * P.head_stride;
      for (int i = tid; i < P.k; i += kSelThreads) {
        const int x = L[i];
        if (x >= w0 && x < wend) atomicOr(&bits[(x - w0) >> 5], 1u << ((x - w0) & 31));
      }
    }
    __syncthreads();
    const int per = (nw + kSelThreads - 1) / kSelThreads;
    const int wb = imin(nw, tid * per), we = imin(nw, wb + per);
    uint32_t cnt = 0;
    for (int i = wb; i < we; ++i) cnt += (uint32_t)__popc(bits[i]);
    uint32_t total;
    int pos = emitted + (int)block_scan_total(sh, cnt, &total);
    for (int i = wb; i < we; ++i) {
      uint32_t m = bits[i];
      while (m) {
        out[pos++] = w0 + 32 * i + __builtin_ctz(m);
        m &= m - 1u;
      }
    }
    emitted += (int)total;
    __syncthreads();
  }
  for (int i = emitted + tid; i < width; i += kSelThreads) out[i] = -1;
}

__global__ __launch_bounds__(256) void head_slice_kernel(const uint16_t* src, uint16_t* dst, int64_t bt, int Hkv,
                                                         int G, int r, int gather) {
  const int64_t i = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // (bt, g) row
  if (i >= bt * Hkv) return;
  const int64_t t = i / Hkv;
  const int g = (int)(i % Hkv), c = threadIdx.x & 15;
  const int64_t narrow = i, wide = t * Hkv * G + (int64_t)g * G + r;
  const int64_t s_row = gather ? wide : narrow, d_row = gather ? narrow : wide;
  *reinterpret_cast<u32x4*>(dst + d_row * kHeadDim + 8 * c) =
      *reinterpret_cast<const u32x4*>(src + s_row * kHeadDim + 8 * c);
}

__global__ __launch_bounds__(256) void lse_scatter_kernel(const float* src, float* dst, int B, int Hkv, int G, int r,
                                                          int n) {
  const int bg = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  dst[((int64_t)b * Hkv * G + (int64_t)g * G + r) * n + t] = src[(int64_t)bg * n + t];
}

hipError_t launch_head_union(const UnionParams& p, int64_t rows, hipStream_t s) {
  head_union_kernel<<<dim3((unsigned)rows), dim3(kSelThreads), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_head_slice(const uint16_t* src, uint16_t* dst, int64_t bt, int Hkv, int G, int r, bool gather,
                             hipStream_t s) {
  const int64_t rows = bt * Hkv;
  head_slice_kernel<<<dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s>>>(src, dst, bt, Hkv, G, r, gather ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_lse_scatter(const float* src, float* dst, int B, int Hkv, int G, int r, int n, hipStream_t s) {
  lse_scatter_kernel<<<dim3((unsigned)((n + 255) / 256), (unsigned)(B * Hkv)), dim3(256), 0, s>>>(src, dst, B, Hkv, G,
                                                                                                  r, n);
  return hipGetLastError();
}

hipError_t launch_select_blocks(const BlockSelectParams& p, int64_t rows, hipStream_t s) {
  if (p.blk_stride <= 64 * kBlkWaveE)
    select_blocks_wave_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(p, rows);
  else
    select_blocks_kernel<<<dim3((unsigned)rows), dim3(kSelThreads), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_block_max(const BlockMaxParams& p, hipStream_t s) {
  const unsigned gx = (unsigned)((std::max(p.blk_stride, 1) + 63) / 64);
  block_max_kernel<<<dim3(gx, (unsigned)(p.B * p.Hkv)), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_select_prefill(const SelectParams& p, int64_t rows, hipStream_t s) {
  // Sampled rows keep about 1.77 k candidates: past what 80 slots per lane
  // hold from k ~ 2600 on (k = 4096 at the 1M context: ~7300), where every
  // row would otherwise go to the block-wide path.
  if (p.top_k > 2560)
    select_prefill_wave_kernel<kWaveEBig><<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(p, rows);
  else
    select_prefill_wave_kernel<kWaveE><<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(p, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)std::min<int64_t>(rows, 1024);
  if (p.cap > kRegCap)
    select_prefill_deferred_kernel<true><<<dim3(grid), dim3(kSelThreads), 0, s>>>(p);
  else
    select_prefill_deferred_kernel<false><<<dim3(grid), dim3(kSelThreads), 0, s>>>(p);
  return hipGetLastError();
}
hipError_t launch_threshold(const ThresholdParams& p, int64_t rows, hipStream_t s) {
  const dim3 g((unsigned)((rows + 3) / 4));
  if (p.max_samples <= 64 * 16)
    threshold_wave_kernel<16><<<g, dim3(256), 0, s>>>(p, rows);
  else if (p.max_samples <= 64 * 32)
    threshold_wave_kernel<32><<<g, dim3(256), 0, s>>>(p, rows);
  else if (p.max_samples <= 64 * kWaveE)
    threshold_wave_kernel<kWaveE><<<g, dim3(256), 0, s>>>(p, rows);
  else
    threshold_kernel<<<dim3((unsigned)rows), dim3(kSelThreads), 0, s>>>(p);
  return hipGetLastError();
}
hipError_t launch_select_decode(const SelectDecodeParams& p, int rows, hipStream_t s) {
  if (p.nslices <= 0) {
    select_decode_kernel<<<dim3((unsigned)rows), dim3(kSelThreads), 0, s>>>(p);
    return hipGetLastError();
  }
  select_decode_threshold_kernel<<<dim3((unsigned)rows), dim3(kSelThreads), 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  select_decode_filter_kernel<<<dim3((unsigned)((p.nslices + kSelWaves - 1) / kSelWaves), (unsigned)rows),
                                dim3(kSelThreads), 0, s>>>(p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  select_decode_final_kernel<<<dim3((unsigned)rows), dim3(kSelThreads), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace hs
