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
// Design (MI355X): one wave per work item (a query row, or a split of a
// decode row), so thousands of independent waves keep enough 16-byte gathers
// in flight to cover memory latency.
//  * A work item walks a virtual key list in chunks of 16 keys, three chunks
//    in flight. FULL: keys [k0, k1) of a decode row. SPARSE: the idx row
//    (entries < 0 are padding) followed by the window Win(p), compacted into
//    a per-wave LDS list of byte offsets.
//  * Each lane gathers 16 bytes of four K and four V rows, so consecutive
//    lanes read consecutive bytes of a row (full cache lines, one address
//    quad per row segment: the texture addresser, not the memory, was the
//    limit with operand-shaped gathers). K goes through a per-wave LDS tile
//    into S^T = K Q^T on v_mfma_f32_16x16x32_bf16, the G query heads of the
//    group in MFMA columns 0..G-1, so one K/V row read serves all heads.
//    V never leaves the lane: O^T = V^T P^T on v_mfma_f32_16x16x16_bf16 runs
//    with the head dimension permuted, and P^T already is the B operand.
//  * Softmax state is per lane (query column = lane%16) with two cross-lane
//    exchanges (lane^16, lane^32) per chunk; accumulation is fp32.
//  * Block-level cooperation only where rows share data: in prefill the four
//    rows of a block gather their common forced window once; in decode the
//    four splits of one row may merge their partials in LDS.
#include "hs_common.hpp"
#include "hs_kernels.hpp"

namespace hs {

namespace {

constexpr int kKS16 = 136;  // per-wave K tile row stride in bf16 (272 B: 16-B reads of 16 rows hit distinct banks)
constexpr int kList = 2048;     // staged key offsets per wave (SPARSE)
constexpr int kListPad = 64;    // zero tail read by the chunks issued past the end
constexpr int kSigStage = 2048; // score-row keys staged per wave (FULL segment length)

__device__ __forceinline__ void lds_wait() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// One 16-key chunk in flight. Lane (n = l%16, gq = l/16) gathers keys
// 4gq..4gq+3 of the chunk, dims 8n..8n+7 of each K and V row (consecutive
// lanes read consecutive bytes of a row: full cache lines, one address quad
// per row segment).
template <bool FP8>
struct ChunkT {
  u32x4 kw[4];  // K rows 4gq + r
  u32x4 vw[4];  // V rows 4gq + r
  int nv;       // wave-uniform: keys 0..nv-1 of the chunk are real, the rest masked
};
// FP8 cache: the same eight dims per row as e4m3 codes (8 bytes), widened to
// bf16 when consumed.
template <>
struct ChunkT<true> {
  u32x2 kw[4];
  u32x2 vw[4];
  int nv;
};

// SIGMA (full rows only): also write the group score row of the candidates.
// FP8: keys and values from the FP8 copy of the cache (sparse layers, and the
// decode full layer).
template <int G, bool SPARSE, bool SIGMA, bool FP8 = false>
__global__ __launch_bounds__(256) void flash_gather_kernel(DecodeParams P) {
  using Chunk = ChunkT<FP8>;
  // Per-wave K tiles and key lists; in prefill SPARSE mode the block's
  // shared window tiles alias this region before the lists are built.
  constexpr int kKtBytes = 16 * kKS16 * 2;
  constexpr int kListBytes = (SPARSE ? kList + kListPad : 4) * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[4 * (kKtBytes + kListBytes)];
  __shared__ __attribute__((aligned(16))) float sig_all[4][SIGMA ? kSigStage : 4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar control flow
  const int n = lane & 15, gq = lane >> 4;
  uint16_t* Kt = reinterpret_cast<uint16_t*>(lds_raw + wave * kKtBytes);
  uint32_t* klist = reinterpret_cast<uint32_t*>(lds_raw + 4 * kKtBytes + wave * kListBytes);

  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  const bool decode = P.seq_lens != nullptr;
  int b, t, g, split, p;
  bool row_ok = true, win_shared = false;  // prefill: row exists; window gathered by the block
  int b0 = 0, t0 = 0;
  if (decode) {
    const int64_t total = (int64_t)P.B * P.Hkv * P.splits;
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
    row_ok = bt < (int64_t)P.B * P.n_q;  // rows past the end join the block's shared phase only
    const int64_t btc = row_ok ? bt : (int64_t)P.B * P.n_q - 1;
    t = (int)(btc % P.n_q);
    b = (int)(btc / P.n_q);
    p = P.n_kv - P.n_q + t;
    // the block's first row: the rows of its batch entry share one window
    const int64_t bt0 = (int64_t)(blockIdx.x / P.Hkv) * 4;
    b0 = (int)(bt0 / P.n_q);
    t0 = (int)(bt0 % P.n_q);
    win_shared = SPARSE && !FP8 && row_ok && b == b0;  // FP8: window keys gathered per wave
  }
  const int64_t qrow = (int64_t)b * P.n_q + t;  // decode: n_q == 1

  // Key source. SPARSE: source position i < k is idx entry i (kept when it
  // lies in [0, p - W], dropped otherwise: padding or a malformed entry);
  // i >= k is window token w0 + (i - k). A split covers source positions
  // [sbeg, send); its kept keys are compacted, in source order, into the
  // wave's LDS list as byte offsets of their cache rows. FULL: keys
  // [sbeg, send) of the row, in order.
  const int k = SPARSE ? P.top_k : 0;
  const int w0 = imax(0, p - P.window + 1);
  const int lim = p - P.window;  // last selectable token
  const int ns = SPARSE ? k + (win_shared ? 0 : p - w0 + 1) : p + 1;
  const int sbeg = uniform(split * P.split_len);
  const int send = uniform(imin(ns, sbeg + P.split_len));
  // A split beyond this row: the global merge skips it; a block merge needs
  // the wave at its barrier, contributing an empty partial (m = -inf, l = 0).
  const bool empty = sbeg >= send;
  if (decode && empty && !P.combine_in_block) return;

  // Query operand: column n = head g*G + n (n < G), dims 32s + 8*gq .. +8.
  bf16x8 qb[4];
  {
    const uint16_t* qp = P.q + (qrow * P.Hq + (int64_t)g * G + (n < G ? n : 0)) * kHeadDim + 8 * gq;
#pragma unroll
    for (int s = 0; s < 4; ++s) qb[s] = as_bf16x8(n < G ? ld16(qp + 32 * s) : u32x4{0u, 0u, 0u, 0u});
  }

  b = uniform(b);
  g = uniform(g);
  __amdgpu_buffer_rsrc_t krs, vrs;
  uint32_t rowb, colb;  // bytes per token; this lane's bytes of a row (dims 8n .. 8n+7)
  float kscale = 1.f, vscale = 1.f;
  if constexpr (FP8) {
    const uint8_t* slab8 = P.kv8 + ((int64_t)b * P.Hkv + g) * P.kv8_cap * kFp8RowBytes;
    krs = make_rsrc(slab8);
    vrs = make_rsrc(slab8 + kHeadDim);
    rowb = kFp8RowBytes;
    colb = 8u * (uint32_t)n;
    // power-of-two scales: K's folds into the logit scale, V's into P (exact)
    kscale = P.kv8_scale[((int64_t)b * P.Hkv + g) * 2];
    vscale = P.kv8_scale[((int64_t)b * P.Hkv + g) * 2 + 1];
  } else {
    krs = make_rsrc(P.kv.slab(b, g));
    vrs = make_rsrc(P.kv.slab(b, g) + P.kv.voff);
    rowb = 2u * (uint32_t)P.kv.st;
    colb = 16u * (uint32_t)n;
  }
  f32x4 oacc[8] = {};
  float m_run = kNegInf, l_part = 0.f;
  const float cexp = P.scale * kscale * kLog2e;
  const float sig_scale = P.scale * kscale;  // exact product: kscale is a power of two
  const int cand_end = lim;  // last candidate position (FULL score row)
  // Score row: the group maxima of each chunk are staged in the wave's LDS
  // segment buffer and written out once the segment's gathers are done: a
  // store among the gathers would hold up every later wait on them (vector
  // memory operations retire in order). 16-byte pieces are written when they
  // start at a candidate of this split; such a piece may run into the window
  // or the row padding (sigma_stride is a multiple of 64 and at least the
  // longest row): entries the selection never reads.
  float* const sig_row = SIGMA ? P.sigma + ((int64_t)b * P.Hkv + g) * P.sigma_stride : nullptr;

  // SPARSE list state (wave-uniform): klist[0 .. cnt) holds the offsets of
  // virtual keys vseg0 .. vseg0 + cnt - 1; keys below lend are published to
  // the chunk loop; spos is the next source position.
  int vseg0 = 0, cnt = 0, lend = 0, spos = sbeg;
  const int32_t* sel = SPARSE ? P.idx + (qrow * P.Hkv + g) * (int64_t)P.top_k : nullptr;
  // Stages the next segment while no gathers are in flight: carries the
  // unpublished tail [lend, vseg0 + cnt) (fewer than 16 entries) to the
  // front, appends compacted source entries until the list is nearly full or
  // the source is exhausted, and publishes whole chunks (all entries once the
  // source is exhausted). kListPad zero offsets (row 0) follow the entries:
  // chunks issued past the end read them.
  auto refill = [&]() {
    const int keep = vseg0 + cnt - lend;
    const uint32_t kept = klist[imin(lend - vseg0 + lane, kList + kListPad - 1)];
    if (lane < keep) klist[lane] = kept;  // one wave: LDS ops stay in order
    vseg0 = lend;
    cnt = keep;
    constexpr int kBatch = 16;
#pragma unroll 1
    while (spos < send && cnt <= kList - 64 * kBatch) {
      int ent[kBatch];
      if (spos < k) {
#pragma unroll
        for (int it = 0; it < kBatch; ++it) ent[it] = sel[imin(spos + lane + 64 * it, k - 1)];
      }
#pragma unroll
      for (int it = 0; it < kBatch; ++it) {
        const int i = spos + lane + 64 * it;
        int e = 0;
        bool ok = i < send;
        if (i < k) {
          e = ent[it];
          ok = ok && lim >= 0 && (unsigned)e <= (unsigned)lim;
        } else {
          e = w0 + (i - k);
        }
        const uint64_t m = ballot(ok);
        if (ok) klist[cnt + (int)lane_prefix(m)] = (uint32_t)e * rowb;
        cnt = uniform(cnt + __popcll(m));
      }
      spos = uniform(spos + 64 * kBatch);
    }
    klist[cnt + lane] = 0u;
    lend = uniform(vseg0 + (spos >= send ? cnt : (cnt & ~15)));
    lds_wait();
  };

  // Issues the gathers of the chunk starting at virtual key v (keys below
  // vend are real).
  auto load = [&](Chunk& ch, int v, int vend) {
    uint32_t off[4];
    if constexpr (SPARSE) {
      const u32x4 e4 = *reinterpret_cast<const u32x4*>(&klist[v - vseg0 + 4 * gq]);
#pragma unroll
      for (int r = 0; r < 4; ++r) off[r] = e4[r] + colb;
    } else {
      const int vb = sbeg + v;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = vb + 4 * gq + r;
        off[r] = (uint32_t)(j < send ? j : 0) * rowb + colb;
      }
    }
    ch.nv = uniform(imin(imax(vend - v, 0), 16));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (FP8) {
        ch.kw[r] = buf_ld8(krs, off[r]);
        ch.vw[r] = buf_ld8(vrs, off[r]);
      } else {
        ch.kw[r] = buf_ld16(krs, off[r]);
        ch.vw[r] = buf_ld16(vrs, off[r]);
      }
    }
  };

  // Attention update with the chunk starting at virtual key v.
  float* const sig_stage = sig_all[wave];
  const int sig_last = imin(cand_end, send - 1);  // last key this split may start a piece at
  int sig_v0 = 0;                                 // first key of the staged segment
  // Writes the staged scores of keys [sig_v0, ve) (relative to sbeg).
  // Pieces start at multiples of 4 (splits and segments are), so a sample
  // (every 2^s-th candidate, s >= 2) can only be a piece's first key.
  float* const samp_row = SIGMA && P.samp ? P.samp + ((int64_t)b * P.Hkv + g) * kDecSamples : nullptr;
  const int samp_shift = dec_sample_shift(cand_end + 1);
  const int samp_mask = (1 << samp_shift) - 1;
  auto sig_flush = [&](int ve) {
    for (int i = 4 * lane; i < ve - sig_v0; i += 256) {
      const int j = sbeg + sig_v0 + i;
      if (j <= sig_last) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(&sig_stage[i]);
        *reinterpret_cast<f32x4*>(sig_row + j) = v;
        if (samp_row && (j & samp_mask) == 0) samp_row[j >> samp_shift] = v[0];
      }
    }
  };
  // Online-softmax update and O^T += V^T P^T for one 16-key chunk: acc holds
  // its raw dot products (masked keys at -inf) as S^T (lane: query column n,
  // keys 4gq + i), vw its V rows (keys 4gq + r, dims 8n..8n+7).
  auto finish = [&](f32x4 acc, const u32x4* vw) __attribute__((always_inline)) {
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
    if constexpr (FP8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= vscale;  // exact: a power of two
    }
    u32x2 pb;
    pb[0] = pack_bf16x2(acc[0], acc[1]);
    pb[1] = pack_bf16x2(acc[2], acc[3]);
    // O^T = V^T P^T with the head dimension permuted: tile bk, row r stands
    // for dim 8r + bk, so the A operand (row n, keys 4gq..4gq+3) is element
    // bk of this lane's own four V rows; no data leaves the lane.
#pragma unroll
    for (int bk = 0; bk < 8; ++bk) {
      const uint32_t sel2 = (bk & 1) ? 0x07060302u : 0x05040100u;
      u32x2 a;
      a[0] = __builtin_amdgcn_perm(vw[1][bk >> 1], vw[0][bk >> 1], sel2);
      a[1] = __builtin_amdgcn_perm(vw[3][bk >> 1], vw[2][bk >> 1], sel2);
      oacc[bk] = mfma16x16x16(a, pb, oacc[bk]);
    }
  };
  auto compute = [&](const Chunk& ch, int v) __attribute__((always_inline)) {
    // K rows into the per-wave LDS tile (row-major, key 4gq + r)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (FP8)
        st16(&Kt[(4 * gq + r) * kKS16 + 8 * n], fp8x8_to_bf16x8(ch.kw[r]));
      else
        st16(&Kt[(4 * gq + r) * kKS16 + 8 * n], ch.kw[r]);
    }
    lds_wait();
    // S^T = K Q^T: A operand lane (n, gq) = K[key n][32s + 8gq .. +8]
    f32x4 acc = {};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma16x16x32(as_bf16x8(ld16(&Kt[n * kKS16 + 32 * s + 8 * gq])), qb[s], acc);
    mfma_settle<kSettle16>(acc);
    // lane holds query column n, chunk keys 4*gq + i: the keys it gathered
    if (ch.nv < 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * gq + i >= ch.nv) acc[i] = kNegInf;
    }
    if constexpr (SIGMA) {
      f32x4 mxh;
#pragma unroll
      for (int i = 0; i < 4; ++i) mxh[i] = group_max<G>(acc[i]) * sig_scale;
      if (n == 0) *reinterpret_cast<f32x4*>(&sig_stage[v - sig_v0 + 4 * gq]) = mxh;
    }
    if constexpr (FP8) {
      u32x4 vw[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) vw[r] = fp8x8_to_bf16x8(ch.vw[r]);
      finish(acc, vw);
    } else {
      finish(acc, ch.vw);
    }
  };

  // Prefill: the forced windows of the block's rows (consecutive tokens of
  // one batch entry and KV group) overlap in all but a few keys, so the four
  // waves gather their union once, in 32-key tiles loaded straight into LDS
  // (buffer_load ... lds; three buffers, two tiles in flight, one barrier
  // per tile), and each wave scores its own window from there; the selected
  // keys follow, gathered per wave. K rows sit with their 16-byte chunks
  // permuted (chunk c of row r at c ^ (r % 16)) so that the score operand
  // reads of 16 rows hit distinct banks.
  if constexpr (SPARSE) {
    if (!decode && !FP8) {
      constexpr int kWinKeys = 32;
      constexpr int kWinTile = 2 * kWinKeys * 256;  // K then V, 256-byte rows
      static_assert(3 * kWinTile <= 4 * (kKtBytes + kListBytes), "window tiles exceed the aliased LDS");
      const int t_last = imin(t0 + 3, P.n_q - 1);
      const int off = P.n_kv - P.n_q;
      const int lo = imax(0, off + t0 - P.window + 1), hi = off + t_last;
      const int ntw = uniform((hi - lo + kWinKeys) / kWinKeys);
      const __amdgpu_buffer_rsrc_t krs0 = make_rsrc(P.kv.slab(uniform(b0), g));
      const __amdgpu_buffer_rsrc_t vrs0 = make_rsrc(P.kv.slab(uniform(b0), g) + P.kv.voff);
      typedef __attribute__((address_space(3))) void lds_void;
      // wave w loads tile rows 8w + 4h + l/16 (h = 0, 1), 16 bytes each lane
      auto fetch = [&](int j) __attribute__((always_inline)) {
        uint8_t* tb = lds_raw + (j % 3) * kWinTile;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r0 = 8 * wave + 4 * h;
          const int row = r0 + (lane >> 4);
          const int key = imin(lo + j * kWinKeys + row, hi);  // past the union: clamped, masked
          const uint32_t base = (uint32_t)key * rowb;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(krs0, (lds_void*)(tb + r0 * 256), 16,
                                                   base + 16u * (uint32_t)(n ^ (row & 15)), 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs0, (lds_void*)(tb + kWinKeys * 256 + r0 * 256), 16,
                                                   base + 16u * (uint32_t)n, 0, 0, 0);
        }
      };
      fetch(0);
      if (ntw > 1) {
        fetch(1);
        __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4): tile 0 landed
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      }
      __syncthreads();
#pragma unroll 1
      for (int j = 0; j < ntw; ++j) {
        if (j + 2 < ntw) fetch(j + 2);  // into tile j-1's buffer, free since the last barrier
        if (win_shared) {
          const uint8_t* tb = lds_raw + (j % 3) * kWinTile;
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int kb = lo + j * kWinKeys + 16 * c;  // first key of the chunk
            if (kb > p || kb + 15 < w0) continue;       // wave-uniform
            f32x4 acc = {};
            const uint8_t* krow = tb + (16 * c + n) * 256;
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
              acc = mfma16x16x32(as_bf16x8(ld16(krow + 16 * ((4 * s2 + gq) ^ n))), qb[s2], acc);
            mfma_settle<kSettle16>(acc);
            if (kb < w0 || kb + 15 > p) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int jk = kb + 4 * gq + i;
                if (jk < w0 || jk > p) acc[i] = kNegInf;
              }
            }
            u32x4 vw[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) vw[r] = ld16(tb + kWinKeys * 256 + (16 * c + 4 * gq + r) * 256 + 16 * n);
            finish(acc, vw);
          }
        }
        // tile j+1 landed (the loads of tile j+2, if any, may still fly)
        if (j + 2 < ntw)
          __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
        else
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
      }
    }
    if (!row_ok) return;
  }

  // Three chunks in flight: chunks are issued two ahead of the one consumed
  // (unconditionally: past the end they are masked and read row 0), and
  // sched_barrier keeps each batch of gathers ahead of the previous chunk's
  // math. The steady-state loop runs whole triples and has a single
  // exit at its end (a mid-loop exit would make the compiler assume gathers
  // still in flight at the loop head and wait for all of them there); the
  // last one or two chunks are consumed after it. SPARSE rows run segment by
  // segment (the pipeline drains at each refill).
  if (!empty) for (;;) {
    int vs = 0, ve = send - sbeg;
    if constexpr (SPARSE) {
      refill();
      vs = vseg0;
      ve = lend;
    } else if constexpr (SIGMA) {
      vs = sig_v0;
      ve = imin(send - sbeg, sig_v0 + kSigStage);
    }
    const int nch = uniform((ve - vs + 15) >> 4);
    const int ntrip = uniform(nch / 3);
    Chunk A, B, C;
    load(A, vs, ve);
    load(B, vs + 16, ve);
    int v = vs;
#pragma unroll 1
    for (int it = 0; it < ntrip; ++it, v += 48) {
      load(C, v + 32, ve);
      __builtin_amdgcn_sched_barrier(0);
      compute(A, v);
      load(A, v + 48, ve);
      __builtin_amdgcn_sched_barrier(0);
      compute(B, v + 16);
      load(B, v + 64, ve);
      __builtin_amdgcn_sched_barrier(0);
      compute(C, v + 32);
    }
    const int rem = nch - 3 * ntrip;
    if (rem >= 1) compute(A, v);
    if (rem >= 2) compute(B, v + 16);
    if constexpr (SPARSE) {
      if (spos >= send) break;
    } else if constexpr (SIGMA) {
      sig_flush(ve);
      sig_v0 = ve;
      if (sig_v0 >= send - sbeg) break;
    } else {
      break;
    }
  }

  mfma_settle8<kSettle16>(oacc);
  const float l_tot = xor32_sum(xor16_sum(l_part));
  if (decode && P.combine_in_block) {
    // The block's waves are splits 0..3 of one (b, g) row. Each wave leaves
    // its partial (acc[G][128], m, l) in its own K tile, then thread
    // (head hn, dims 4c..4c+3) merges the four: M = max m_s,
    // o = sum 2^(m_s - M) acc_s / sum 2^(m_s - M) l_s.
    constexpr int kPartStride = kHeadDim + 4;  // floats per head; 16-byte aligned rows
    static_assert(G * kPartStride * 4 <= kKtBytes, "block-merge partials exceed the K tile");
    float* mine = reinterpret_cast<float*>(Kt);
    if (n < G) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float* d = mine + n * kPartStride + 32 * gq + 8 * i;
        *reinterpret_cast<f32x4*>(d) = f32x4{oacc[0][i], oacc[1][i], oacc[2][i], oacc[3][i]};
        *reinterpret_cast<f32x4*>(d + 4) = f32x4{oacc[4][i], oacc[5][i], oacc[6][i], oacc[7][i]};
      }
      if (gq == 0) {
        mine[n * kPartStride + kHeadDim] = m_run;
        mine[n * kPartStride + kHeadDim + 1] = l_tot;
      }
    }
    __syncthreads();
    if (tid >= G * 32) return;
    const int hn = tid >> 5, d0 = 4 * (tid & 31);
    float ms[4], ls[4];
    f32x4 av[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const float* src = reinterpret_cast<const float*>(lds_raw + s2 * kKtBytes) + hn * kPartStride;
      ms[s2] = src[kHeadDim];
      ls[s2] = src[kHeadDim + 1];
      av[s2] = *reinterpret_cast<const f32x4*>(src + d0);
    }
    const float M = fmaxf(fmaxf(ms[0], ms[1]), fmaxf(ms[2], ms[3]));
    const float Mu = M == kNegInf ? 0.f : M;
    float lsum = 0.f;
    f32x4 o4 = {};
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const float w = __builtin_amdgcn_exp2f(ms[s2] - Mu);  // empty split: 0
      lsum += w * ls[s2];
      o4 += w * av[s2];
    }
    const float inv = 1.f / lsum;
    const int head = g * G + hn;
    u32x2 ow;
    ow[0] = pack_bf16x2(o4[0] * inv, o4[1] * inv);
    ow[1] = pack_bf16x2(o4[2] * inv, o4[3] * inv);
    *reinterpret_cast<u32x2*>(P.o + (qrow * P.Hq + head) * kHeadDim + d0) = ow;
    if (P.lse && (tid & 31) == 0) P.lse[((int64_t)b * P.Hq + head) * P.n_q + t] = Mu * kLn2 + __logf(lsum);
    return;
  }
  if (n >= G) return;
  const int head = g * G + n;
  // oacc[bk][i] is dim 8(4gq + i) + bk: eight consecutive dims per i.
  if (P.splits == 1) {
    const float inv = 1.f / l_tot;
    uint16_t* op = P.o + (qrow * P.Hq + head) * kHeadDim + 32 * gq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 w;
#pragma unroll
      for (int c = 0; c < 4; ++c) w[c] = pack_bf16x2(oacc[2 * c][i] * inv, oacc[2 * c + 1][i] * inv);
      st16(op + 8 * i, w);
    }
    if (P.lse && gq == 0) P.lse[((int64_t)b * P.Hq + head) * P.n_q + t] = m_run * kLn2 + __logf(l_tot);
  } else {
    float* pp = P.part + ((((int64_t)b * P.Hkv + g) * P.splits + split) * G + n) * (kHeadDim + 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<f32x4*>(pp + 32 * gq + 8 * i) = f32x4{oacc[0][i], oacc[1][i], oacc[2][i], oacc[3][i]};
      *reinterpret_cast<f32x4*>(pp + 32 * gq + 8 * i + 4) = f32x4{oacc[4][i], oacc[5][i], oacc[6][i], oacc[7][i]};
    }
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

// ---------------------------------------------------------------- FP8 cache copy
// A token row is 32 pieces of 8 dims: piece c < 16 holds K dims 8c .. 8c+7,
// piece c >= 16 V dims 8(c-16) ...; thread t takes piece t % 32 of rows
// t / 32, t / 32 + 8, ... of its block's rows.
constexpr int kFp8RowsPerBlock = 256;

// Smallest e with amax <= 448 * 2^e (0 for an all-zero head).
__device__ __forceinline__ int fp8_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int e;
  (void)frexpf(amax, &e);
  e -= 9;
  while (amax > ldexpf(448.f, e)) ++e;
  while (amax <= ldexpf(448.f, e - 1)) --e;
  return e;
}

// Eight bf16 values times inv (a power of two), clamped to +-448, to e4m3
// codes rounded to nearest even (byte i = element i).
__device__ __forceinline__ u32x2 bf16x8_to_fp8x8(u32x4 w, float inv) {
  float x[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x[2 * q] = fminf(fmaxf(bf16lo(w[q]) * inv, -448.f), 448.f);
    x[2 * q + 1] = fminf(fmaxf(bf16hi(w[q]) * inv, -448.f), 448.f);
  }
  uint32_t a = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0u, false);
  a = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], a, true);
  uint32_t c = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0u, false);
  c = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], c, true);
  return u32x2{a, c};
}

__global__ void fp8_zero_kernel(uint32_t* amax, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) amax[i] = 0u;
}

// Per-(b, g) maxima of |K| and |V| over rows [0, n_kv): per block, then one
// atomic max per block (non-negative floats order like their bit patterns).
__global__ __launch_bounds__(256) void fp8_amax_kernel(Fp8ConvertParams P) {
  __shared__ float red[2][4];
  const int bg = blockIdx.y, b = bg / P.Hkv, g = bg % P.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid & 31, vsel = c >> 4, d0 = 8 * (c & 15);
  const int r0 = blockIdx.x * kFp8RowsPerBlock;
  const int r1 = imin(P.n_kv, r0 + kFp8RowsPerBlock);
  float m = 0.f;
  for (int r = r0 + (tid >> 5); r < r1; r += 8) {
    const u32x4 w = ld16((vsel ? P.kv.v_row(b, g, r) : P.kv.k_row(b, g, r)) + d0);
#pragma unroll
    for (int q = 0; q < 4; ++q) m = fmaxf(m, fmaxf(fabsf(bf16lo(w[q])), fabsf(bf16hi(w[q]))));
  }
  // lanes with bit 4 clear hold K pieces, the others V pieces
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  if (lane == 0) red[0][wave] = m;
  if (lane == 16) red[1][wave] = m;
  __syncthreads();
  if (tid < 2) {
    const float mm = fmaxf(fmaxf(red[tid][0], red[tid][1]), fmaxf(red[tid][2], red[tid][3]));
    uint32_t* amax = reinterpret_cast<uint32_t*>(P.kv8 + kv8_codes_bytes(P.B, P.Hkv, P.cap));
    atomicMax(&amax[bg * 2 + tid], __float_as_uint(mm));
  }
}

__global__ __launch_bounds__(256) void fp8_convert_kernel(Fp8ConvertParams P) {
  const int bg = blockIdx.y, b = bg / P.Hkv, g = bg % P.Hkv;
  const int tid = threadIdx.x;
  const int c = tid & 31, vsel = c >> 4, d0 = 8 * (c & 15);
  const uint32_t* amax = reinterpret_cast<const uint32_t*>(P.kv8 + kv8_codes_bytes(P.B, P.Hkv, P.cap));
  float* scale = reinterpret_cast<float*>(P.kv8 + kv8_codes_bytes(P.B, P.Hkv, P.cap) + (int64_t)P.B * P.Hkv * 8);
  const int e = fp8_exponent(__uint_as_float(amax[bg * 2 + vsel]));
  const float inv = ldexpf(1.f, -e);
  if (blockIdx.x == 0 && (tid == 0 || tid == 16)) scale[bg * 2 + vsel] = ldexpf(1.f, e);
  const int r0 = blockIdx.x * kFp8RowsPerBlock;
  const int r1 = imin(P.n_kv, r0 + kFp8RowsPerBlock);
  uint8_t* dst = P.kv8 + (int64_t)bg * P.cap * kFp8RowBytes + vsel * kHeadDim + d0;
  for (int r = r0 + (tid >> 5); r < r1; r += 8) {
    const u32x4 w = ld16((vsel ? P.kv.v_row(b, g, r) : P.kv.k_row(b, g, r)) + d0);
    *reinterpret_cast<u32x2*>(dst + (int64_t)r * kFp8RowBytes) = bf16x8_to_fp8x8(w, inv);
  }
}

// Decode: the row appended at slot seq_lens[b] - 1, with the stored scales.
__global__ __launch_bounds__(256) void fp8_append_kernel(Fp8ConvertParams P) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= P.B * P.Hkv * 32) return;
  const int bg = i >> 5, c = i & 31, vsel = c >> 4, d0 = 8 * (c & 15);
  const int b = bg / P.Hkv, g = bg % P.Hkv;
  const int r = P.seq_lens[b] - 1;
  if (r < 0 || r >= P.cap) return;
  const float* scale = reinterpret_cast<const float*>(P.kv8 + kv8_codes_bytes(P.B, P.Hkv, P.cap) + (int64_t)P.B * P.Hkv * 8);
  const float inv = 1.f / scale[bg * 2 + vsel];  // exact: a power of two
  const u32x4 w = ld16((vsel ? P.kv.v_row(b, g, r) : P.kv.k_row(b, g, r)) + d0);
  *reinterpret_cast<u32x2*>(P.kv8 + ((int64_t)bg * P.cap + r) * kFp8RowBytes + vsel * kHeadDim + d0) =
      bf16x8_to_fp8x8(w, inv);
}

// Log-sum-exp merge of split partials; one block per (b, head) of
// kCombGroups groups of 128 threads. Pass 1 (threads over splits): M = max
// m_s, then weights w_s = 2^(m_s - M) into LDS and l = sum w_s l_s. Pass 2:
// group i takes the i-th quarter of the splits, thread d of a group sums
// w_s acc_s[d] over them with independent loads; the groups' sums add in LDS
// and o = sum / l.
constexpr int kMaxCombineSplits = 4096;
constexpr int kCombGroups = 4;
constexpr int kCombThreads = 128 * kCombGroups;
__global__ __launch_bounds__(kCombThreads) void combine_kernel(CombineParams P) {
  __shared__ float wsh[kMaxCombineSplits];
  __shared__ float red[2][kCombThreads / 64];
  __shared__ float part[kCombGroups][kHeadDim];
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
  for (int s = tid; s < ns; s += kCombThreads) M = fmaxf(M, base[s * sstride + kHeadDim]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  if (lane == 0) red[0][wave] = M;
  __syncthreads();
  M = red[0][0];
#pragma unroll
  for (int w = 1; w < kCombThreads / 64; ++w) M = fmaxf(M, red[0][w]);
  const float Mu = M == kNegInf ? 0.f : M;
  float l = 0.f;
  for (int s = tid; s < ns; s += kCombThreads) {
    const float w = __builtin_amdgcn_exp2f(base[s * sstride + kHeadDim] - Mu);
    wsh[s] = w;
    l += w * base[s * sstride + kHeadDim + 1];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
  if (lane == 0) red[1][wave] = l;
  __syncthreads();
  l = 0.f;
#pragma unroll
  for (int w = 0; w < kCombThreads / 64; ++w) l += red[1][w];
  const int grp = tid >> 7, d = tid & 127;
  const int s0 = (ns * grp) / kCombGroups, s1 = (ns * (grp + 1)) / kCombGroups;
  // 32 loads in flight per thread: with a few hundred splits per head the
  // sum is a chain of memory round trips, not of arithmetic
  float acc = 0.f;
  const float* pd = base + d;
  int s = s0;
  for (; s + 32 <= s1; s += 32) {
    float v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) v[u] = pd[(s + u) * sstride];
#pragma unroll
    for (int u = 0; u < 32; ++u) acc += wsh[s + u] * v[u];
  }
  for (; s + 8 <= s1; s += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = pd[(s + u) * sstride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += wsh[s + u] * v[u];
  }
  for (; s < s1; ++s) acc += wsh[s] * pd[s * sstride];
  part[grp][d] = acc;
  __syncthreads();
  if (tid < kHeadDim) {
    float o = part[0][tid];
#pragma unroll
    for (int q = 1; q < kCombGroups; ++q) o += part[q][tid];
    P.o[((int64_t)b * P.Hq + head) * kHeadDim + tid] = (uint16_t)f32_to_bf16_bits(o / l);
  }
  if (P.lse && tid == 0) P.lse[(int64_t)b * P.Hq + head] = M * kLn2 + __logf(l);
}

// Gather-rate probe (diagnostics): the memory access pattern of the sparse
// layers without their arithmetic. Wave w stages its keys idx[w * per_wave
// ..) in LDS as byte offsets (as the sparse kernel stages its compacted key
// list), then walks them in 16-key chunks, three in flight; lane (n = l % 16,
// gq = l / 16) loads 16 bytes of the K half and 16 bytes of the V half of
// token rows 4gq..4gq+3 of a chunk (512-byte rows, K then V, as in the
// default cache layout). The loaded words are folded into one value per lane
// and stored, so no load is dead.
constexpr int kProbeMaxKeys = 2048;
__global__ __launch_bounds__(256) void gather_probe_kernel(ProbeParams P) {
  __shared__ uint32_t offs[4][kProbeMaxKeys];
  const int lane = threadIdx.x & 63, n = lane & 15, gq = lane >> 4;
  const int wv = threadIdx.x >> 6;
  const int64_t wave = (int64_t)blockIdx.x * 4 + wv;
  const int64_t k0 = wave * P.per_wave;
  if (k0 >= P.n) return;
  const int nk = (int)(P.n - k0 < P.per_wave ? P.n - k0 : P.per_wave);
  uint32_t* lst = offs[wv];
  for (int i = lane; i < nk; i += 64) lst[i] = (uint32_t)P.idx[k0 + i] * 512u;
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): one wave, LDS operations in order
  const __amdgpu_buffer_rsrc_t rs = make_rsrc_sized(P.src, P.src_bytes);  // reads past the buffer return 0
  uint32_t acc = 0;
  auto issue = [&](u32x4* kw, u32x4* vw, int c) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t off = lst[imin(16 * c + 4 * gq + r, nk - 1)] + 16u * (uint32_t)n;
      kw[r] = buf_ld16(rs, off);
      vw[r] = buf_ld16(rs, off + 256u);
    }
  };
  auto fold = [&](const u32x4* kw, const u32x4* vw) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc += (kw[r][0] ^ kw[r][1] ^ kw[r][2] ^ kw[r][3]) + (vw[r][0] ^ vw[r][3]);
  };
  const int nch = (nk + 15) / 16;
  u32x4 ka[4], va[4], kb[4], vb[4], kc[4], vc[4];
  issue(ka, va, 0);
  if (nch > 1) issue(kb, vb, 1);
  int c = 0;
#pragma unroll 1
  for (; c + 2 < nch; c += 3) {
    issue(kc, vc, c + 2);
    fold(ka, va);
    if (c + 3 < nch) issue(ka, va, c + 3);
    fold(kb, vb);
    if (c + 4 < nch) issue(kb, vb, c + 4);
    fold(kc, vc);
  }
  if (c < nch) fold(ka, va);
  if (c + 1 < nch) fold(kb, vb);
  P.out[wave * 64 + lane] = acc;
}

template <int G, bool SPARSE>
hipError_t launch_gather_g(const DecodeParams& p, hipStream_t s) {
  const int64_t blocks = p.seq_lens ? ((int64_t)p.B * p.Hkv * p.splits + 3) / 4
                                    : (((int64_t)p.B * p.n_q + 3) / 4) * p.Hkv;
  if (!SPARSE && p.kv8 && p.sigma)
    flash_gather_kernel<G, false, true, true><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p);
  else if (!SPARSE && p.kv8)
    flash_gather_kernel<G, false, false, true><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p);
  else if (!SPARSE && p.sigma)
    flash_gather_kernel<G, false, true><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p);
  else if (SPARSE && p.kv8)
    flash_gather_kernel<G, true, false, true><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p);
  else
    flash_gather_kernel<G, SPARSE, false><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p);
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

hipError_t launch_kv_convert_fp8(const Fp8ConvertParams& p, hipStream_t s) {
  const int bg = p.B * p.Hkv;
  if (p.seq_lens) {
    fp8_append_kernel<<<dim3((unsigned)((bg * 32 + 255) / 256)), dim3(256), 0, s>>>(p);
    return hipGetLastError();
  }
  uint32_t* amax = reinterpret_cast<uint32_t*>(p.kv8 + kv8_codes_bytes(p.B, p.Hkv, p.cap));
  fp8_zero_kernel<<<dim3((unsigned)((2 * bg + 255) / 256)), dim3(256), 0, s>>>(amax, 2 * bg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((p.n_kv + kFp8RowsPerBlock - 1) / kFp8RowsPerBlock), (unsigned)bg);
  fp8_amax_kernel<<<grid, dim3(256), 0, s>>>(p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  fp8_convert_kernel<<<grid, dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_gather_probe(const ProbeParams& p, hipStream_t s) {
  const int64_t waves = (p.n + p.per_wave - 1) / p.per_wave;
  gather_probe_kernel<<<dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  combine_kernel<<<dim3((unsigned)(p.B * p.Hq)), dim3(kCombThreads), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace hs
