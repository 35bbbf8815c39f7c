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
// each score (8-bit digits, per-wave LDS histograms). It finds the exact k-th
// key T and how many elements equal to T are still needed; when more elements
// tie at T than are needed, a second radix select over the token indices of the
// tied elements keeps the lowest ones. Selected indices are gathered in LDS and
// bitonic-sorted ascending. One 256-thread block handles one row.
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
__device__ void pick_digit(SelShared& sh, bool descending) {
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
    uint32_t need = sh.need;
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
    float kv[kHeadDim];
#pragma unroll
    for (int c = 0; c < kHeadDim / 8; ++c) {
      u32x4 w = ld16(kr + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kv[8 * c + 2 * e] = bf16lo(w[e]);
        kv[8 * c + 2 * e + 1] = bf16hi(w[e]);
      }
    }
    float best = kNegInf;
    for (int h = 0; h < G; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < kHeadDim; ++e) acc = fmaf(qs[h * kHeadDim + e], kv[e], acc);
      best = fmaxf(best, acc * scale);
    }
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
    pick_digit(sh, true);
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

// Among elements with key == T, find the largest index bound J such that
// exactly `need` tied elements have index <= J (indices are distinct).
template <class Src>
__device__ uint32_t find_tie_bound(SelShared& sh, const Src& src, int n, uint32_t T, uint32_t need) {
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if (threadIdx.x == 0) { sh.prefix = 0; sh.need = need; }
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t pmask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
    clear_hist(sh);
    __syncthreads();
    const uint32_t prefix = sh.prefix;
    for (int i = threadIdx.x; i < n; i += kSelThreads) {
      if (src.key(i) != T) continue;
      uint32_t ix = (uint32_t)src.index(i);
      if ((ix & pmask) == prefix) atomicAdd(&sh.hist[wave][(ix >> shift) & 255u], 1u);
    }
    __syncthreads();
    pick_digit(sh, false);
    __syncthreads();
    if (threadIdx.x == 0) {
      sh.prefix = prefix | (sh.found_digit << shift);
      sh.need -= sh.found_gt;
    }
    __syncthreads();
  }
  return sh.prefix;
}

// Sorts list[0, n) ascending in LDS (n <= cap_pow2, cap_pow2 a power of two),
// padding with INT32_MAX, then writes k entries (-1 padded) to out.
__device__ void sort_and_emit(int32_t* list, int n, int k, int32_t* out) {
  int P = 1;
  while (P < n) P <<= 1;
  for (int i = n + threadIdx.x; i < P; i += kSelThreads) list[i] = 0x7fffffff;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < P / 2; t += kSelThreads) {
        int lo = 2 * t - (t & (stride - 1));
        int hi = lo + stride;
        bool up = (lo & size) == 0;
        int32_t a = list[lo], b = list[hi];
        if ((a > b) == up) { list[lo] = b; list[hi] = a; }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < k; i += kSelThreads) out[i] = i < n ? list[i] : -1;
}

template <class Src>
__device__ void topk_from_source(SelShared& sh, int32_t* list, const Src& src, int n, int k, int32_t* out) {
  if (n <= k) {
    // Every candidate is selected (reading: fewer than k candidates -> all).
    for (int i = threadIdx.x; i < n; i += kSelThreads) list[i] = src.index(i);
    __syncthreads();
    sort_and_emit(list, n, k, out);
    return;
  }
  find_kth_key(sh, src, n, (uint32_t)k);
  const uint32_t T = sh.prefix;
  const uint32_t need_eq = (uint32_t)k - sh.found_gt;  // tied elements to keep
  const uint32_t n_eq = sh.eq_count;
  uint32_t J = 0xffffffffu;
  if (n_eq > need_eq) J = find_tie_bound(sh, src, n, T, need_eq);
  __syncthreads();
  if (threadIdx.x == 0) sh.nsel = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kSelThreads) {
    uint32_t key = src.key(i);
    bool sel = key > T;
    if (key == T) sel = (uint32_t)src.index(i) <= J;
    if (sel) {
      uint32_t slot = atomicAdd(&sh.nsel, 1u);
      if (slot < (uint32_t)k) list[slot] = src.index(i);
    }
  }
  __syncthreads();
  sort_and_emit(list, k, k, out);
}

// ---------------------------------------------------------------- kernels

// Top-k over the candidate buffer of each (b, t, g) row of a prefill call.
__global__ __launch_bounds__(kSelThreads) void select_prefill_kernel(SelectParams P) {
  __shared__ SelShared sh;
  __shared__ int32_t list[kMaxTopK];
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
    for (int i = threadIdx.x; i < P.top_k; i += kSelThreads) out[i] = i < ncand ? i : -1;
    return;
  }
  const int cnt = P.counts[row];
  const bool ok = !P.force_rescan && cnt >= P.top_k && cnt <= P.cap;
  if (ok) {
    BufSrc src{P.buf_sigma + row * (int64_t)P.cap, P.buf_j + row * (int64_t)P.cap};
    topk_from_source(sh, list, src, cnt, P.top_k, out);
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
  RescanSrc src{qs, P.kv.k_row(b, g, 0), P.kv.st, G, P.scale};
  topk_from_source(sh, list, src, ncand, P.top_k, out);
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
  find_kth_key(sh, src, nsamp, (uint32_t)m);
  if (threadIdx.x == 0) P.theta[row] = key_to_score(sh.prefix);
}

// Decode: top-k over the dense score row of each (b, g).
__global__ __launch_bounds__(kSelThreads) void select_decode_kernel(SelectDecodeParams P) {
  __shared__ SelShared sh;
  __shared__ int32_t list[kMaxTopK];
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
  topk_from_source(sh, list, src, ncand, P.top_k, out);
}

hipError_t launch_select_prefill(const SelectParams& p, int64_t rows, hipStream_t s) {
  select_prefill_kernel<<<dim3((unsigned)rows), dim3(kSelThreads), 0, s>>>(p);
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
