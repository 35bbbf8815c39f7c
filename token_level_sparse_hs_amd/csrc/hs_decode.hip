// Gather-based attention for the sparse-reuse layers and for decode (gfx950).
//
// Sparse-reuse layers ("HySparse2 od Xiaomi zkracuje zpracovani dlouheho
// kontextu", section "Proc neni nutne znovu zpracovat cely dlouhy vstup";
// DAIR.AI weekly, bullet "Two levels of KV sharing"): every sparse layer reuses
// the full layer's KV cache and selection, attending from its own queries to
// S = (selected tokens) U (forced recent window). Decode full attention
// ("HySparse2 Cuts the Prefill Path for Tool-Using Agents", section "Tool
// Responses Turn Prefill Into the Bottleneck": decoding reuses the cache that
// prefill wrote) streams a sequence's whole cache once and also emits the
// group score row that the decode selection ranks. Split partials (m, l, acc)
// are merged by the log-sum-exp correction ("Simplified Sparse Attention via
// Gist Tokens", section 3.6, three-kernel split-K decode).
//
// Design (MI355X): one wave per work item (row or split), so thousands of
// independent waves keep enough 16-byte gathers in flight to cover HBM
// latency; no block-level synchronisation.
//  * A work item walks a virtual key list in chunks of 32 keys. FULL: keys
//    [k0, k1) of a decode row. SPARSE: the idx row (entries < 0 are padding)
//    followed by the window Win(p).
//  * K and V rows are gathered 4 keys x 8 dims per lane, so consecutive
//    lanes read consecutive bytes of a row (full cache lines, one address
//    quad per row segment: the texture addresser, not the memory, was the
//    limit with operand-shaped gathers), and staged in row-major per-wave LDS
//    tiles. S^T = K Q^T on v_mfma_f32_16x16x32_bf16 reads its A operand from
//    the K tile; the G query heads of the group occupy MFMA columns 0..G-1,
//    so one K/V row read serves all heads. V is read back transposed
//    (ds_read_b64_tr_b16) as the A operand of O^T = V^T P^T on
//    v_mfma_f32_16x16x16_bf16; P^T is already in B-operand layout.
//  * Softmax state is per lane (query column = lane%16) with two cross-lane
//    exchanges (lane^16, lane^32) per chunk; accumulation is fp32.
#include "hs_common.hpp"
#include "hs_kernels.hpp"

namespace hs {

namespace {

constexpr int kVS16 = 144;  // per-wave V tile row stride in bf16 (128 dims + pad: 288 B)
constexpr int kKS16 = 136;  // per-wave K tile row stride in bf16 (272 B: 16-B reads of 16 rows hit distinct banks)

__device__ __forceinline__ void lds_wait() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

template <bool SPARSE>
struct KeyList {
  // SPARSE: virtual v < k -> idx[v] (if >= 0), else window token w0 + (v-k).
  // FULL: v -> v.
  // Selected entries outside [0, lim] (padding, or a malformed row) are
  // skipped, so no gather leaves the sequence's valid rows.
  const int32_t* sel;
  int k;
  int w0;
  int lim;
  int end;  // virtual end (exclusive)
  __device__ __forceinline__ int key(int v) const {
    if (v >= end) return -1;
    if constexpr (!SPARSE) return v;
    if (v >= k) return w0 + (v - k);
    const int j = sel[v];
    return (j >= 0 && j <= lim) ? j : -1;
  }
};

constexpr int kSeg = 2048;  // idx-row entries staged per wave (refilled only when k > kSeg)

// One 16-key chunk in flight: K rows as MFMA A operands (lane: key l%16, dims
// 32s + 8(l/16)..+8) and V rows for the LDS transpose (lane: keys
// 4(l/16)..+3, dims 8(l%16)..+7), plus the validity mask of its 16 keys.
struct Chunk {
  u32x4 kw[4];     // K rows 4gq + r, dims 8n..8n+7 (row-coalesced gather)
  u32x4 vw[4];     // V rows, same keys
  uint32_t valid;  // bit r: key 4gq + r is valid
};

template <int G, bool SPARSE>
__global__ __launch_bounds__(256) void flash_gather_kernel(DecodeParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t Vt_all[4][16 * kVS16];
  __shared__ __attribute__((aligned(16))) uint16_t Kt_all[4][16 * kKS16];
  __shared__ __attribute__((aligned(16))) int32_t klist_all[4][SPARSE ? kSeg : 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar control flow
  const int n = lane & 15, gq = lane >> 4;
  uint16_t* Vt = Vt_all[wave];
  uint16_t* Kt = Kt_all[wave];
  int32_t* klist = klist_all[wave];

  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  const bool decode = P.seq_lens != nullptr;
  int b, t, g, split, p;
  int64_t total;
  if (decode) {
    total = (int64_t)P.B * P.Hkv * P.splits;
    if (item >= total) return;
    split = (int)(item % P.splits);
    const int64_t bg = item / P.splits;
    g = (int)(bg % P.Hkv);
    b = (int)(bg / P.Hkv);
    t = 0;
    p = imin(P.seq_lens[b], P.n_kv) - 1;  // n_kv carries the host bound max_seq_len
    if (p < 0) return;
  } else {
    // A block holds four consecutive query rows of one KV group, and the group
    // varies fastest over blocks: with blocks dealt round-robin to the XCDs,
    // each XCD's L2 then serves one group, and neighbouring rows (which share
    // their window and often popular keys) run side by side.
    split = 0;
    g = (int)(blockIdx.x % P.Hkv);
    const int64_t bt = (int64_t)(blockIdx.x / P.Hkv) * 4 + wave;
    if (bt >= (int64_t)P.B * P.n_q) return;
    t = (int)(bt % P.n_q);
    b = (int)(bt / P.n_q);
    p = P.n_kv - P.n_q + t;
  }
  const int64_t qrow = (int64_t)b * P.n_q + t;  // decode: n_q == 1

  KeyList<SPARSE> kl;
  int vbeg, vend;
  if (SPARSE) {
    kl.sel = P.idx + (qrow * P.Hkv + g) * (int64_t)P.top_k;
    kl.k = P.top_k;
    kl.w0 = imax(0, p - P.window + 1);
    kl.lim = p - P.window;
    const int nv = P.top_k + (p - kl.w0 + 1);
    vbeg = split * P.split_len;
    vend = imin(nv, vbeg + P.split_len);
  } else {
    kl.sel = nullptr;
    kl.k = 0;
    kl.w0 = 0;
    kl.lim = p;
    vbeg = split * P.split_len;
    vend = imin(p + 1, vbeg + P.split_len);
  }
  kl.end = vend;
  if (vbeg >= vend) return;  // split beyond this row: the combine skips it

  // Query operand: column n = head g*G + n (n < G), dims 32s + 8*gq .. +8.
  bf16x8 qb[4];
  {
    const uint16_t* qp = P.q + (qrow * P.Hq + (int64_t)g * G + (n < G ? n : 0)) * kHeadDim + 8 * gq;
#pragma unroll
    for (int s = 0; s < 4; ++s) qb[s] = as_bf16x8(n < G ? ld16(qp + 32 * s) : u32x4{0u, 0u, 0u, 0u});
  }

  const uint16_t* slab = P.kv.slab(b, g);
  f32x4 oacc[8] = {};
  float m_run = kNegInf, l_part = 0.f;
  const float cexp = P.scale * kLog2e;
  const int cand_end = p - P.window;  // last candidate position (FULL score row)
  float* sig_row = nullptr;
  if (!SPARSE && P.sigma) sig_row = P.sigma + ((int64_t)b * P.Hkv + g) * P.sigma_stride;

  // SPARSE: the idx row is staged in LDS, kSeg entries at a time; window
  // tokens (virtual keys >= k) are computed.
  int seg0 = -kSeg;
  auto refill = [&](int base) {
    seg0 = base;
    const int cnt = imin(kSeg, kl.k - base);  // >= 1
    const int32_t* src = kl.sel + base;
    // All loads are issued before any is consumed (clamped, unconditional);
    // entries beyond cnt are never looked up as selected tokens.
    constexpr int kBatch = 8;
#pragma unroll 1
    for (int i0 = 0; i0 < cnt; i0 += 64 * kBatch) {
      int32_t vals[kBatch];
#pragma unroll
      for (int it = 0; it < kBatch; ++it) vals[it] = src[imin(i0 + lane + 64 * it, cnt - 1)];
#pragma unroll
      for (int it = 0; it < kBatch; ++it) klist[imin(i0 + lane + 64 * it, kSeg - 1)] = vals[it];
    }
    lds_wait();
  };
  if constexpr (SPARSE) {
    if (vbeg < kl.k) refill(vbeg - (vbeg % kSeg));
  }

  // Issues the gathers of the chunk starting at virtual key v0.
  auto load = [&](Chunk& ch, int v0) {
    if constexpr (SPARSE) {
      if (v0 < kl.k && v0 + 16 > seg0 + kSeg) refill(v0 - (v0 % kSeg));
    }
    // Each lane gathers keys 4gq..4gq+3 of the chunk (consecutive virtual
    // keys: one 16-byte LDS read of the staged idx row), 16 bytes of K and of
    // V per key, so that consecutive lanes read consecutive bytes of one row
    // (row-coalesced, full cache lines). Invalid slots read row 0 (always a
    // valid row); their scores are masked to -inf, so their probabilities
    // are exactly 0. Keeping every gather unconditional lets the compiler
    // wait only for the chunk it consumes.
    int jv[4];
    const int vb = v0 + 4 * gq;
    if constexpr (SPARSE) {
      const int vi = imin(imax(vb - seg0, 0), kSeg - 4);
      const int4 e4 = *reinterpret_cast<const int4*>(&klist[vi]);
      const int e[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = vb + r;
        const int js = (e[r] >= 0 && e[r] <= kl.lim) ? e[r] : -1;
        const int j = v < kl.k ? js : kl.w0 + (v - kl.k);
        jv[r] = v < vend ? j : -1;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) jv[r] = vb + r < vend ? vb + r : -1;
    }
    uint32_t valid = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint16_t* row = slab + (uint32_t)((jv[r] >= 0 ? jv[r] : 0) * P.kv.st + 8 * n);
      ch.kw[r] = ld16(row);
      ch.vw[r] = ld16(row + P.kv.voff);
      valid |= (jv[r] >= 0 ? 1u : 0u) << r;
    }
    ch.valid = valid;
  };

  // Attention update with the chunk starting at virtual key v0.
  auto compute = [&](const Chunk& ch, int v0) {
    // K and V rows into the per-wave LDS tiles (row-major, key 4gq + r)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      st16(&Kt[(4 * gq + r) * kKS16 + 8 * n], ch.kw[r]);
      st16(&Vt[(4 * gq + r) * kVS16 + 8 * n], ch.vw[r]);
    }
    lds_wait();
    // S^T = K Q^T: A operand lane (n, gq) = K[key n][32s + 8gq .. +8]
    f32x4 acc = {};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma16x16x32(as_bf16x8(ld16(&Kt[n * kKS16 + 32 * s + 8 * gq])), qb[s], acc);
    // lane holds query column n, chunk keys 4*gq + i: the keys it gathered
    if (ch.valid != 0xfu) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!((ch.valid >> i) & 1u)) acc[i] = kNegInf;
    }
    if (!SPARSE && sig_row && v0 <= cand_end) {
      f32x4 mxh;
#pragma unroll
      for (int i = 0; i < 4; ++i) mxh[i] = group_max<G>(acc[i]) * P.scale;
      const int j = v0 + 4 * gq;
      if (n == 0) {
        if (j + 3 <= cand_end && ((j & 3) == 0)) {
          *reinterpret_cast<f32x4*>(sig_row + j) = mxh;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (j + i <= cand_end) sig_row[j + i] = mxh[i];
        }
      }
    }
    // online softmax
    float mx = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
    mx = xor32_max(xor16_max(mx));
    // Deferred rescaling: the reference maximum moves only when a score
    // exceeds it by more than 2^kRescaleLog2, so P stays <= 2^8 and O, l are
    // rarely touched; numerator and denominator share the reference, so the
    // normalised result is the same.
    const float m_cand = mx * cexp;
    if (ballot(m_cand > m_run + kRescaleLog2)) {
      const float m_new = fmaxf(m_run, m_cand);
      const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == kNegInf ? 0.f : m_new));  // -inf -> 0
      l_part *= alpha;
#pragma unroll
      for (int bk = 0; bk < 8; ++bk) oacc[bk] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = __builtin_amdgcn_exp2f(fmaf(acc[i], cexp, -m_use));
      acc[i] = pv;
      psum += pv;
    }
    l_part += psum;
    u32x2 pb;
    pb[0] = pack_bf16x2(acc[0], acc[1]);
    pb[1] = pack_bf16x2(acc[2], acc[3]);
    lds_wait();
    // A operand of O^T = V^T P^T: lane (n, gq) needs V[4gq + e][16bk + n];
    // lane n of group gq addresses V[4gq + n/4][16bk + 4(n%4)].
    const uint16_t* vrd = &Vt[(4 * gq + (n >> 2)) * kVS16 + 4 * (n & 3)];
#pragma unroll
    for (int bk = 0; bk < 8; ++bk) oacc[bk] = mfma16x16x16(lds_read_tr16(vrd + 16 * bk), pb, oacc[bk]);
  };

  // Two chunks in flight: the next chunk's gathers are issued before the
  // current chunk is consumed.
  // Later chunks are always issued (past the end their slots are invalid and
  // read row 0), so every path carries the same loads in flight and the
  // compiler waits only for the chunk being consumed.
  // sched_barrier keeps each batch of gathers ahead of the previous chunk's
  // math, so the waits before that math cover only the previous chunk.
  // Three chunks in flight.
  Chunk A, B, C;
  load(A, vbeg);
  load(B, vbeg + 16);
  for (int v0 = vbeg;; v0 += 48) {
    load(C, v0 + 32);
    __builtin_amdgcn_sched_barrier(0);
    compute(A, v0);
    if (v0 + 16 >= vend) break;
    load(A, v0 + 48);
    __builtin_amdgcn_sched_barrier(0);
    compute(B, v0 + 16);
    if (v0 + 32 >= vend) break;
    load(B, v0 + 64);
    __builtin_amdgcn_sched_barrier(0);
    compute(C, v0 + 32);
    if (v0 + 48 >= vend) break;
  }

  const float l_tot = xor32_sum(xor16_sum(l_part));
  if (n >= G) return;
  const int head = g * G + n;
  if (P.splits == 1) {
    const float inv = 1.f / l_tot;
    uint16_t* op = P.o + (qrow * P.Hq + head) * kHeadDim;
#pragma unroll
    for (int bk = 0; bk < 8; ++bk) {
      u32x2 w;
      w[0] = pack_bf16x2(oacc[bk][0] * inv, oacc[bk][1] * inv);
      w[1] = pack_bf16x2(oacc[bk][2] * inv, oacc[bk][3] * inv);
      *reinterpret_cast<u32x2*>(op + 16 * bk + 4 * gq) = w;
    }
    if (P.lse && gq == 0) P.lse[((int64_t)b * P.Hq + head) * P.n_q + t] = m_run * kLn2 + __logf(l_tot);
  } else {
    float* pp = P.part + ((((int64_t)b * P.Hkv + g) * P.splits + split) * G + n) * (kHeadDim + 2);
#pragma unroll
    for (int bk = 0; bk < 8; ++bk)
      *reinterpret_cast<f32x4*>(pp + 16 * bk + 4 * gq) = oacc[bk];
    if (gq == 0) {
      pp[kHeadDim] = m_run;
      pp[kHeadDim + 1] = l_tot;
    }
  }
}

// Decode: write kv_new[b] into cache slot seq_lens[b]-1.
__global__ void append_kernel(AppendParams P) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 16-byte piece
  const int64_t total = (int64_t)P.B * P.Hkv * 2 * 16;
  if (i >= total) return;
  const int c = (int)(i & 15);
  const int kvsel = (int)((i >> 4) & 1);
  const int64_t bg = i >> 5;
  const int g = (int)(bg % P.Hkv);
  const int b = (int)(bg / P.Hkv);
  const int slot = P.seq_lens[b] - 1;
  if (slot < 0 || slot >= P.cap) return;  // out-of-range length: nothing written
  const u32x4 w = ld16(P.kv_new + ((bg * 2 + kvsel) * kHeadDim) + 8 * c);
  uint16_t* dst = P.kv + (int64_t)b * P.sb + (int64_t)g * P.sh + (int64_t)slot * P.st + (kvsel ? P.voff : 0) + 8 * c;
  st16(dst, w);
}

// Log-sum-exp merge of split partials; one 128-thread block per (b, head).
// Pass 1 (threads over splits): M = max m_s, then weights w_s = 2^(m_s - M)
// into LDS and l = sum w_s l_s. Pass 2 (threads over dims): o = sum w_s acc_s / l
// with independent loads.
constexpr int kMaxCombineSplits = 4096;
__global__ __launch_bounds__(128) void combine_kernel(CombineParams P) {
  __shared__ float wsh[kMaxCombineSplits];
  __shared__ float red[2][4];
  const int bh = blockIdx.x;
  const int head = bh % P.Hq, b = bh / P.Hq;
  const int G = P.Hq / P.Hkv;
  const int g = head / G, n = head % G;
  const int L = imin(P.seq_lens[b], P.max_len);
  if (L < 1) return;
  const int nv = P.sparse_k >= 0 ? P.sparse_k + (L < P.window ? L : P.window) : L;
  const int ns = imin(imin(P.splits, (nv + P.split_len - 1) / P.split_len), kMaxCombineSplits);
  const float* base = P.part + (((int64_t)b * P.Hkv + g) * P.splits * G + n) * (kHeadDim + 2);
  const int64_t sstride = (int64_t)G * (kHeadDim + 2);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float M = kNegInf;
  for (int s = tid; s < ns; s += 128) M = fmaxf(M, base[s * sstride + kHeadDim]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  if (lane == 0) red[0][wave] = M;
  __syncthreads();
  M = fmaxf(red[0][0], red[0][1]);
  const float Mu = M == kNegInf ? 0.f : M;
  float l = 0.f;
  for (int s = tid; s < ns; s += 128) {
    const float w = __builtin_amdgcn_exp2f(base[s * sstride + kHeadDim] - Mu);
    wsh[s] = w;
    l += w * base[s * sstride + kHeadDim + 1];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
  if (lane == 0) red[1][wave] = l;
  __syncthreads();
  l = red[1][0] + red[1][1];
  float acc = 0.f;
  const float* pd = base + tid;
  int s = 0;
  for (; s + 8 <= ns; s += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = pd[(s + u) * sstride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += wsh[s + u] * v[u];
  }
  for (; s < ns; ++s) acc += wsh[s] * pd[s * sstride];
  P.o[((int64_t)b * P.Hq + head) * kHeadDim + tid] = (uint16_t)f32_to_bf16_bits(acc / l);
  if (P.lse && tid == 0) P.lse[(int64_t)b * P.Hq + head] = M * kLn2 + __logf(l);
}

template <int G, bool SPARSE>
hipError_t launch_gather_g(const DecodeParams& p, hipStream_t s) {
  const int64_t blocks = p.seq_lens ? ((int64_t)p.B * p.Hkv * p.splits + 3) / 4
                                    : (((int64_t)p.B * p.n_q + 3) / 4) * p.Hkv;
  flash_gather_kernel<G, SPARSE><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

template <bool SPARSE>
hipError_t launch_gather(const DecodeParams& p, hipStream_t s) {
  switch (p.Hq / p.Hkv) {
    case 1: return launch_gather_g<1, SPARSE>(p, s);
    case 2: return launch_gather_g<2, SPARSE>(p, s);
    case 4: return launch_gather_g<4, SPARSE>(p, s);
    case 8: return launch_gather_g<8, SPARSE>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_full(const DecodeParams& p, hipStream_t s) { return launch_gather<false>(p, s); }
hipError_t launch_sparse(const DecodeParams& p, hipStream_t s) { return launch_gather<true>(p, s); }

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  const int64_t total = (int64_t)p.B * p.Hkv * 32;
  append_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  combine_kernel<<<dim3((unsigned)(p.B * p.Hq)), dim3(128), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace hs
