// Prefill full-attention layer with fused token selection (gfx950).
//
// Computes, for a chunk of n_q query rows at the end of an n_kv-token cache,
// causal GQA attention (o, lse) and the per-(row, KV group) candidate set for
// token-level top-k selection: the full-attention layer of a hybrid block
// whose selection the following sparse layers reuse ("HySparse2 od Xiaomi
// zkracuje zpracovani dlouheho kontextu", section "Proc neni nutne znovu
// zpracovat cely dlouhy vstup"; DAIR.AI weekly, bullets "Two levels of KV
// sharing" and "Prefill exits early").
//
// Design (MI355X):
//  * One block = 8 waves (two per SIMD, one block per CU; 4 waves for G = 1)
//    = one KV group g and 8*(32/G) query tokens. Each wave owns 32 MFMA rows
//    = 32/G tokens x the G query heads of group g, so the group's heads and
//    all eight waves share every K/V tile staged in LDS, and the
//    group maximum over heads (the selection score) is a reduction across
//    lanes: a token's heads sit 16/G lanes apart inside one 16-lane row, and
//    masked DPP steps halve the values each lane carries.
//  * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16: with the key
//    axis on MFMA rows and the query rows on lanes, every per-row softmax
//    quantity (running max, sum, rescale) is lane-local apart from one
//    lane^32 exchange, and the S^T accumulator is already laid out as the B
//    operand of the PV product. K and V tiles go from global memory straight
//    into LDS (buffer loads with the lds modifier, two stages, the next tile
//    in flight during the current one), 256-byte rows with their 16-byte
//    chunks XOR-permuted by row so operand reads hit distinct banks; K
//    operands are read two steps ahead of their products, and V is read back
//    with LDS transpose reads (ds_read_b64_tr_b16) as the A operand of
//    O^T = V^T P^T.
//  * Online softmax in fp32 on exp2 with the scale folded into one FMA.
//  * Selection: the per-lane scaled logits are maxed over the G head lanes
//    (DPP), staged per wave in LDS, and every candidate (j <= p - W) whose
//    score reaches the row's threshold is appended, in ascending key order,
//    to the row's candidate buffer with a wave ballot + mbcnt compaction.
//    Thresholds come from sampled scores (below); rows whose candidates all
//    fit the buffer use -inf, i.e. the buffer is then the full score row.
//  * Blocks run late (long) query tiles first; the group index varies
//    fastest over blockIdx so that, with blocks dealt round-robin to the 8
//    XCDs, each XCD's L2 serves one KV head.
#include <type_traits>

#include "hs_common.hpp"
#include "hs_kernels.hpp"

namespace hs {

namespace {

constexpr int kKS = 136;  // sampled-key tile row stride in bf16 (272 B: conflict-free 16-B reads)
constexpr int kRowB = 256;                 // attention tiles: unpadded 256-byte rows
constexpr int kTileB = 64 * kRowB;         // one 64-key K or V tile

// s_waitcnt immediate for vmcnt(n) alone (gfx9 encoding; n <= 63).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ void lds_wait() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// S^T tile (64 keys x 32 query rows) of this wave: acc[c][i] holds the raw
// dot product of key 32c + 8(i/4) + 4h + i%4 with query row l%32.
__device__ __forceinline__ void qk_tile(const uint16_t* Ks, const bf16x8* qb, f32x16* acc) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, n = lane & 31;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    f32x16 a = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 kop = as_bf16x8(ld16(&Ks[(32 * c + n) * kKS + 16 * s + 8 * h]));
      a = mfma32x32x16(kop, qb[s], a);
    }
    acc[c] = a;
  }
}

// MFMA row n (= lane % 32) of a wave stands for token tok_of(n) of the
// wave's 32/G tokens and head g*G + head_of(n). Each 16-lane row of the wave
// holds 16/G tokens, and a token's G heads sit 16/G lanes apart inside one
// row, so the group maximum runs on DPP within rows.
template <int G>
__device__ __forceinline__ int tok_of(int n) {
  constexpr int TR = 16 / (G > 16 ? 16 : G);
  return (n >> 4) * TR + (n & 15) % TR;
}
template <int G>
__device__ __forceinline__ int head_of(int n) {
  constexpr int TR = 16 / (G > 16 ? 16 : G);
  return (n & 15) / TR;
}

// Loads this lane's query operand: row n = l%32 of the wave (token
// tok_of(n), head g*G + head_of(n)), dims 16s + 8h .. +8 for s = 0..7.
template <int G>
__device__ __forceinline__ void load_q(const uint16_t* q, int b, int n_q, int Hq, int g, int tok, bf16x8* qb) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, n = lane & 31;
  const bool ok = tok < n_q;
  const int head = g * G + head_of<G>(n);
  const uint16_t* qp = q + (((int64_t)b * n_q + (ok ? tok : 0)) * Hq + head) * kHeadDim + 8 * h;
#pragma unroll
  for (int s = 0; s < 8; ++s) qb[s] = as_bf16x8(ok ? ld16(qp + 16 * s) : u32x4{0u, 0u, 0u, 0u});
}

// dst = max(src[partner], src) in the lanes of the DPP banks (4-lane groups
// of a row) named by BANKS; the other lanes of dst keep their value. Row
// rotations: ror:8 pairs lane i with i^8; ror:4 feeds lane i from i-4,
// ror:12 from i+4. The first form defines dst, the second updates it.
// One bank-masked v_max_f32_dpp per value and half-row: the compiler's DPP
// builtins cannot keep the other lanes of dst without a copy of it (three
// instructions per value instead of two; measured 5% slower on this kernel).
// Wait states the compiler cannot see here are placed by hand:
//  * matrix results: every caller settles the accumulators first
//    (mfma_settle, the count the CDNA4 rules give for these instructions);
//  * a DPP read needs two wait states after a vector write of its source:
//    scores rewritten by vector code (the causal mask, the probability
//    score's rescaling) are followed by a two-state pause tied to them, the
//    statements below read r and r2 at least eight instructions after
//    writing them (volatile asm keeps their order; the compiler can only add
//    instructions between them), and `dep` orders the first read after the
//    caller's last use of the scores.
#define HS_DPP_MAX_DEF(dst, src, ROR, BANKS, dep)                                                        \
  asm volatile("v_max_f32_dpp %0, %1, %1 row_ror:" #ROR " row_mask:0xf bank_mask:" #BANKS : "=v"(dst) \
               : "v"(src), "v"(dep))
#define HS_DPP_MAX_UPD(dst, src, ROR, BANKS, dep)                                                        \
  asm volatile("v_max_f32_dpp %0, %1, %1 row_ror:" #ROR " row_mask:0xf bank_mask:" #BANKS : "+v"(dst) \
               : "v"(src), "v"(dep))

// The group maximum reads the scores through DPP from inline assembly, so
// the compiler does not insert the two wait states a DPP read needs after a
// vector write of its source: callers that have just rewritten the scores
// with vector code pause here first.
__device__ __forceinline__ void dpp_read_pause(f32x16& a, f32x16& b) { asm volatile("s_nop 1" : "+v"(a), "+v"(b)); }

// Writes the group-max scores of the wave's tile into sig[TPW][64] (raw,
// unscaled). acc[c][i] holds key 32c + 8(i/4) + 4h + i%4 of MFMA row n.
// Transposing steps halve the values each lane carries instead of
// reducing all 32 in every lane: across lane^8 (banks 0-1 keep the keys of
// acc[0], banks 2-3 those of acc[1]), then across lane^4 (even banks keep
// i < 8, odd banks i >= 8), then a plain step across lane^2 for G = 8. `dep`
// is any value computed after the last use of acc by ordinary code (the
// DPP sources must not be read before the matrix results have landed).
template <int G>
__device__ __forceinline__ void stage_group_max(const f32x16* acc, float* sig, float dep) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, q = lane & 15;
  if constexpr (G == 1) {
    float* row = sig + (lane & 31) * 64;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(row + 32 * c + 8 * q4 + 4 * h) =
            f32x4{acc[c][4 * q4], acc[c][4 * q4 + 1], acc[c][4 * q4 + 2], acc[c][4 * q4 + 3]};
  } else {
    const int c = (q >> 3) & 1;
    float r[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      HS_DPP_MAX_DEF(r[i], acc[1][i], 8, 0xc, dep);
      HS_DPP_MAX_UPD(r[i], acc[0][i], 8, 0x3, dep);
    }
    float* trow = sig + tok_of<G>(lane & 31) * 64 + 32 * c + 4 * h;
    if constexpr (G == 2) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(trow + 8 * q4) = f32x4{r[4 * q4], r[4 * q4 + 1], r[4 * q4 + 2], r[4 * q4 + 3]};
    } else {
      const int ih = (q >> 2) & 1;
      float r2[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        HS_DPP_MAX_DEF(r2[i], r[8 + i], 4, 0xa, dep);
        HS_DPP_MAX_UPD(r2[i], r[i], 12, 0x5, dep);
      }
      if constexpr (G == 8) {  // in order after every write of r2 above (8+ statements back)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          asm volatile("v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf" : "+v"(r2[i]));
      }
      f32x4 v0 = {r2[0], r2[1], r2[2], r2[3]}, v1 = {r2[4], r2[5], r2[6], r2[7]};
      asm volatile("" : "+v"(v0), "+v"(v1));  // computed by all lanes before the writer branch
      if (G == 4 || (q & 2) == 0) {
        *reinterpret_cast<f32x4*>(trow + 16 * ih) = v0;
        *reinterpret_cast<f32x4*>(trow + 16 * ih + 8) = v1;
      }
    }
  }
}

// The group maximum of stage_group_max in pieces, so that its steps can sit
// between matrix instructions. gm_fold8 folds lane^8 for values [I0, I0+N)
// into r, gm_fold4 lane^4 into r2, gm_fold2 lane^2 (G = 8); gm_store writes
// the wave's rows of sig. Within a piece all first-form steps precede the
// second-form ones, so no step reads a register written right before it;
// callers keep each piece's sources at least one chunk (an MFMA, its operand
// reads and a piece) behind their writes.
template <int I0, int N>
__device__ __forceinline__ void gm_fold8(const f32x16* acc, float* r, float dep) {
#pragma unroll
  for (int i = I0; i < I0 + N; ++i) HS_DPP_MAX_DEF(r[i], acc[1][i], 8, 0xc, dep);
#pragma unroll
  for (int i = I0; i < I0 + N; ++i) HS_DPP_MAX_UPD(r[i], acc[0][i], 8, 0x3, dep);
}
template <int I0, int N>
__device__ __forceinline__ void gm_fold4(const float* r, float* r2, float dep) {
#pragma unroll
  for (int i = I0; i < I0 + N; ++i) HS_DPP_MAX_DEF(r2[i], r[8 + i], 4, 0xa, dep);
#pragma unroll
  for (int i = I0; i < I0 + N; ++i) HS_DPP_MAX_UPD(r2[i], r[i], 12, 0x5, dep);
}
__device__ __forceinline__ void gm_fold2(float* r2) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    asm volatile("v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf" : "+v"(r2[i]));
}
// Row layout as in stage_group_max. For G = 8 the lanes q and q^2 hold equal
// values for the same sig entries after gm_fold2, so every lane writes (the
// duplicate writes store the same bytes) and no branch splits the schedule.
template <int G>
__device__ __forceinline__ void gm_store(const f32x16* acc, const float* r, const float* r2, float* sig) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, q = lane & 15;
  if constexpr (G == 1) {
    float* row = sig + (lane & 31) * 64;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(row + 32 * c + 8 * q4 + 4 * h) =
            f32x4{acc[c][4 * q4], acc[c][4 * q4 + 1], acc[c][4 * q4 + 2], acc[c][4 * q4 + 3]};
  } else {
    const int c = (q >> 3) & 1;
    float* trow = sig + tok_of<G>(lane & 31) * 64 + 32 * c + 4 * h;
    if constexpr (G == 2) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(trow + 8 * q4) = f32x4{r[4 * q4], r[4 * q4 + 1], r[4 * q4 + 2], r[4 * q4 + 3]};
    } else {
      const int ih = (q >> 2) & 1;
      *reinterpret_cast<f32x4*>(trow + 16 * ih) = f32x4{r2[0], r2[1], r2[2], r2[3]};
      *reinterpret_cast<f32x4*>(trow + 16 * ih + 8) = f32x4{r2[4], r2[5], r2[6], r2[7]};
    }
  }
}

// Waves per block of the full layer: eight (two per SIMD, one block per CU)
// share every K/V tile; one query head per group (G = 1) needs more
// registers than two waves per SIMD allow and keeps four.
template <int G>
constexpr int attn_waves() { return G == 1 ? 4 : 8; }

// SEL: 0 no selection, 1 token-level candidates, 2 block-level maxima.
//
// Software pipeline over 64-key tiles (one wave's view of tile i):
//   A: S_i = K_i Q^T (16 MFMAs) beside the candidate compaction of tile
//      i-1 (from the group maxima staged in LDS);
//   B: causal mask and row maximum of S_i, then O += V_{i-1}^T P_{i-1}^T
//      (16 MFMAs) beside the group maximum of S_i and P_i = exp2(...),
//      summed and packed to bf16.
// Each wave thus keeps its matrix pipe busy with vector work of its own
// instead of relying on the other wave of its SIMD. V tiles are consumed one
// tile after their K tiles: at tile i, K_{i+1} and V_i are fetched (into the
// stages that K_{i-1} and V_{i-2} left), and one barrier per tile orders
// everything. Rows whose maximum rises past the deferred-rescale slack finish
// O += V_{i-1}^T P_{i-1}^T first, rescale, and let B add a zero P.
template <int G, int SEL>
__global__ __launch_bounds__(64 * attn_waves<G>(), G == 1 ? 2 : 1) void prefill_attn_kernel(PrefillParams P) {
  constexpr int NW = attn_waves<G>();
  constexpr int TPW = 32 / G;
  constexpr int TPB = NW * TPW;
  constexpr int RPW = 64 / NW;  // tile rows each wave fetches
  constexpr int NLD = RPW / 4;  // 16-byte loads per lane and tile, for K and for V
  // K and V tiles of 64 keys, two stages each, unpadded 256-byte rows written
  // by direct global->LDS loads. 16-byte chunks are XOR-permuted within a row
  // so that both operand read patterns hit distinct banks: chunk c of K row r
  // sits at c ^ (r % 16) (16 rows read the same chunk), chunk c of V row r at
  // c ^ 4(r % 4) (the transpose reads take 4 rows x 64 bytes at a time).
  __shared__ __attribute__((aligned(1024))) uint8_t kv_st0[2][kTileB];
  __shared__ __attribute__((aligned(1024))) uint8_t kv_st1[2][kTileB];
  __shared__ __attribute__((aligned(16))) float sig[NW][TPW * 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, n = lane & 31;
  const int ntq = (P.n_q + TPB - 1) / TPB;
  int L = blockIdx.x;
  const int g = L % P.Hkv;
  L /= P.Hkv;
  const int b = L % P.B;
  L /= P.B;
  const int t0 = (ntq - 1 - L) * TPB;
  const int off = P.n_kv - P.n_q;

  const int wt0 = t0 + wave * TPW;
  const int tok = wt0 + tok_of<G>(n);
  const bool tok_ok = tok < P.n_q;
  const int head = g * G + head_of<G>(n);
  const int p_lane = tok_ok ? off + tok : -1;
  const int p_wlo = off + wt0;
  const int p_whi = off + imin(wt0 + TPW, P.n_q) - 1;
  const bool wave_live = wt0 < P.n_q;

  bf16x8 qb[8];
  load_q<G>(P.q, b, P.n_q, P.Hq, g, tok, qb);

  // Selection state of the wave's tokens, all wave-uniform (scalar
  // registers): threshold (+inf past the chunk: nothing passes) and count.
  // Row (b, wt0 + u, g) is row0 + u * Hkv; its last selectable key is
  // off + wt0 + u - W.
  const int64_t row0 = uniform64(((int64_t)b * P.n_q + wt0) * P.Hkv + g);
  float theta[TPW];
  int cnt[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const bool ok = SEL == 1 && wt0 + u < P.n_q;
    theta[u] = ok ? __builtin_bit_cast(float, uniform(__builtin_bit_cast(int, P.theta[row0 + (int64_t)u * P.Hkv])))
                  : kPosInf;
    cnt[u] = 0;
  }

  f32x16 oacc[4] = {};
  float m_run = kNegInf, l_run = 0.f;
  const float cexp = P.scale * kLog2e;

  const int p_bhi = off + imin(t0 + TPB, P.n_q) - 1;
  const int ntiles = p_bhi / 64 + 1;

  // Tile loads: wave w fetches tile rows RPW w + 4i + lane/16 (i < NLD) of K
  // and of V, 16 bytes per lane, straight into LDS (lane l lands at byte 16l
  // of a 1 KB run of 4 rows, i.e. chunk position l % 16); each lane reads the
  // global chunk that belongs at its position. Rows past the cache's valid
  // rows read as zeros (range-checked), and causality masks them.
  const uint16_t* slab = reinterpret_cast<const uint16_t*>(uniform64(reinterpret_cast<int64_t>(P.kv.slab(b, g))));
  const uint32_t rowb = 2u * (uint32_t)P.kv.st;
  const uint32_t span = (uint32_t)(P.n_kv - 1) * rowb + 2u * kHeadDim;  // bytes up to the last valid row's end
  const u32x4 krs = rsrc_words(slab, span);
  const u32x4 vrs = rsrc_words(slab + P.kv.voff, span);
  uint32_t dk[NLD], dv[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const uint32_t r = (uint32_t)RPW * wave + 4u * i + (lane >> 4);
    dk[i] = r * rowb + 16u * ((lane & 15) ^ (r & 15));
    dv[i] = r * rowb + 16u * ((lane & 15) ^ (4u * (r & 3)));
  }
  // The loads are issued from inline assembly, so the compiler does not
  // treat them as LDS writes in flight; the tile wait and the barrier order
  // them explicitly.
  auto fetch_k = [&](int kt, auto stage_c) __attribute__((always_inline)) {
    constexpr int S = decltype(stage_c)::value;
    const uint32_t soff = (uint32_t)uniform(kt * 64) * rowb;
    const uint32_t base = lds_addr(S ? kv_st1[0] : kv_st0[0]) + (uint32_t)(RPW * wave) * kRowB;
#pragma unroll
    for (int i = 0; i < NLD; ++i) lds_dma16(base + 4u * i * kRowB, dk[i], krs, soff);
  };
  auto fetch_v = [&](int kt, auto stage_c) __attribute__((always_inline)) {
    constexpr int S = decltype(stage_c)::value;
    const uint32_t soff = (uint32_t)uniform(kt * 64) * rowb;
    const uint32_t base = lds_addr(S ? kv_st1[1] : kv_st0[1]) + (uint32_t)(RPW * wave) * kRowB;
#pragma unroll
    for (int i = 0; i < NLD; ++i) lds_dma16(base + 4u * i * kRowB, dv[i], vrs, soff);
  };
  // Operand read offsets within a tile. K (S^T = K Q^T, A operand): lane
  // (n, h) reads dims 16s + 8h .. +8 of key n (+32 for the second MFMA block).
  // V (O^T = V^T P^T, A operand, transpose reads): lane l reads 4 dims of key
  // row kb + (l % 16) / 4 + 4h, dims 32bk + 16((l / 16) % 2) + 4(l % 4).
  uint32_t kad[8], vad[4];
#pragma unroll
  for (int s2 = 0; s2 < 8; ++s2) kad[s2] = n * kRowB + 16u * ((2u * s2 + h) ^ (n & 15));
#pragma unroll
  for (int bk = 0; bk < 4; ++bk)
    vad[bk] = (((lane & 15) >> 2) + 4 * h) * kRowB +
              16u * (4u * (bk ^ ((lane >> 2) & 3)) + 2u * ((lane >> 4) & 1) + ((lane & 3) >> 1)) + 8u * (lane & 1);

  // bf16 P of the last two tiles (B operands of O^T += V^T P^T), in turn.
  u32x4 pbA[4], pbB[4];
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) pbA[s2] = pbB[s2] = u32x4{0u, 0u, 0u, 0u};

  // Schedule variant, chosen by measurement. With selection, P of a tile is
  // pinned beside the products of its own tile (otherwise the compiler
  // sinks half of it into the next tile, out of the products' shadow) and
  // waves keep one priority: raising the priority of waves in step A made
  // blocks drift apart, and at a 1M-token context the blocks streaming one
  // group's cache then lost L2 locality (97% -> 28% hits, the clock fell
  // with the extra HBM traffic). Without selection the unpinned schedule
  // with step A at raised priority measured faster.
  constexpr bool kPinP = SEL != 0;

  // Stores per tile of the compaction; the wait for a tile's loads lets them
  // remain outstanding (vector memory operations complete in order).
  constexpr int kStores = SEL == 1 ? 2 * TPW : 0;
  constexpr int kTileWait = kStores < 63 ? kStores : 63;

  // O^T += V^T P^T for one tile: MFMA m = 4 s2 + bk, A operand from two
  // transpose reads (issued four products ahead), B = pb[s2]. FILL(m) places
  // vector work of the caller after product m; each product and its work
  // form one scheduling chunk.
  auto pv = [&](const uint8_t* Vb, const u32x4* pb, auto&& fill) __attribute__((always_inline)) {
    u32x2 vf[5][2];
    auto vread = [&](int m, u32x2* dst) __attribute__((always_inline)) {
      const int s2 = m >> 2, bk = m & 3;
      const int kb = 32 * (s2 >> 1) + 16 * (s2 & 1);
      dst[0] = lds_read_tr16(reinterpret_cast<const uint16_t*>(Vb + kb * kRowB + vad[bk]));
      dst[1] = lds_read_tr16(reinterpret_cast<const uint16_t*>(Vb + (kb + 8) * kRowB + vad[bk]));
    };
    vread(0, vf[0]);
    vread(1, vf[1]);
    vread(2, vf[2]);
    vread(3, vf[3]);
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      if (m + 4 < 16) vread(m + 4, vf[(m + 4) % 5]);
      const int s2 = m >> 2, bk = m & 3;
      const u32x4 w = {vf[m % 5][0][0], vf[m % 5][0][1], vf[m % 5][1][0], vf[m % 5][1][1]};
      oacc[bk] = mfma32x32x16(as_bf16x8(w), as_bf16x8(pb[s2]), oacc[bk]);
      fill(m);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Candidate compaction of the tile at key0p for row u (token-level
  // selection): every candidate key whose score reaches the row's threshold
  // is appended, in ascending key order, to the row's buffer. Past a token's
  // last candidate key (and for tiles without candidates: lim = -1) the lane
  // compares against +inf, so the ballot is the compare's own lane mask.
  // Exactly two range-checked stores: failing lanes and positions past the
  // buffer's capacity aim beyond the row and are dropped.
  auto compact_row = [&](int u, float sv, int key0p, int lim) __attribute__((always_inline)) {
    const float v = sv * P.scale;
    const float th = lane <= lim ? theta[u] : kPosInf;
    const bool pass = v >= th;
    const uint64_t m = ballot(pass);
    const uint32_t so = pass ? 4u * lane_prefix(m) : kDropOffset;
    const int c = uniform(cnt[u]);
    const int64_t rb = (row0 + (int64_t)u * P.Hkv) * P.cap + c;
    const uint32_t room = 4u * (uint32_t)imax(0, P.cap - c);
    buf_st4(make_rsrc_sized(P.buf_sigma + rb, room), so, __float_as_uint(v));
    buf_st4(make_rsrc_sized(P.buf_j + rb, room), so, (uint32_t)(key0p + lane));
    cnt[u] = uniform(c + __popcll(m));
  };
  // Block-level selection of the tile at key0p: the best scaled score among
  // the tile's candidates of each row (the tile is one 64-key block). Row
  // u's 64 scores are spread over 64 / TPW consecutive lanes, TPW scores
  // each, then reduced across those lanes (DPP within a 16-lane row).
  auto block_max = [&](int key0p) __attribute__((always_inline)) {
    constexpr int LPR = 64 / TPW;
    const int u = lane / LPR, c0 = (lane % LPR) * TPW;
    const int lim = off + wt0 + u - P.window - key0p;  // last candidate, tile-relative
    const float* ws = sig[wave] + u * 64 + c0;
    float v = kNegInf;
#pragma unroll
    for (int i = 0; i < TPW; i += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(ws + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) v = c0 + i + e <= lim ? fmaxf(v, x[e]) : v;
    }
    if constexpr (LPR >= 2) v = fmaxf(v, dpp<kDppXor1>(v));
    if constexpr (LPR >= 4) v = fmaxf(v, dpp<kDppXor2>(v));
    if constexpr (LPR >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
    if constexpr (LPR >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
    if (lane % LPR == 0 && wt0 + u < P.n_q)
      P.blk_score[(row0 + (int64_t)u * P.Hkv) * P.blk_stride + (key0p >> 6)] = v * P.scale;
  };
  // Selection of a finished tile (its group maxima in sig): the compaction
  // rows go into chunks 2..7 of the caller's schedule (chunk < 0: all).
  float sv[TPW];
  auto select_part = [&](int key0p, bool live, int chunk) __attribute__((always_inline)) {
    if constexpr (SEL == 1) {
      // up to 8 rows: their scores are read two chunks ahead of their use
      if (TPW <= 8 && chunk <= 0) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) sv[u] = sig[wave][u * 64 + lane];
      }
#pragma unroll
      for (int u = 0; u < TPW; ++u)
        if (chunk < 0 || chunk == 2 + (u * 6) / TPW)
          compact_row(u, TPW <= 8 ? sv[u] : sig[wave][u * 64 + lane], key0p,
                      live ? off + wt0 + u - P.window - key0p : -1);
    } else if constexpr (SEL == 2) {
      if ((chunk < 0 || chunk == 2) && live) block_max(key0p);
    }
  };

  fetch_k(0, std::integral_constant<int, 0>{});
  // V stage 1 is read (times a zero P) before its first tile arrives, and
  // the first tile's selection step reads the group maxima of a tile that
  // does not exist (with no candidates, but finite scores are assumed)
#pragma unroll
  for (int e = 0; e < NLD; ++e) st16(&kv_st1[1][(tid + 64 * NW * e) * 16], u32x4{0u, 0u, 0u, 0u});
  if constexpr (SEL != 0) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) sig[wave][u * 64 + lane] = kNegInf;
  }
  lds_wait();
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  auto tile = [&](int kt, auto stage_c) __attribute__((always_inline)) {
    constexpr int S = decltype(stage_c)::value;
    u32x4* pb_prev = S ? pbA : pbB;
    u32x4* pb_cur = S ? pbB : pbA;
    const int key0 = kt * 64, key0p = key0 - 64;
    const bool sel_prev = SEL != 0 && wave_live && kt > 0 && key0p <= p_whi - P.window;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kTileWait));
    // every wave's part of K_kt and V_{kt-1} has landed, and every wave is
    // done with K_{kt-1} and V_{kt-2}, whose stages the next loads overwrite
    asm volatile("s_barrier" ::: "memory");
    if (kt + 1 < ntiles) fetch_k(kt + 1, std::integral_constant<int, 1 - S>{});
    fetch_v(kt, std::integral_constant<int, S>{});
    const uint8_t* Kb = S ? kv_st1[0] : kv_st0[0];
    const uint8_t* Vp = S ? kv_st0[1] : kv_st1[1];  // V_{kt-1}

    // ---- A: S^T = K Q^T beside the previous tile's selection
    f32x16 acc[2] = {};
    if constexpr (!kPinP) __builtin_amdgcn_s_setprio(1);
    {
      u32x4 kf[3][2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int c = 0; c < 2; ++c) kf[s2][c] = ld16(Kb + c * 32 * kRowB + kad[s2]);
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        if (s2 + 2 < 8)
#pragma unroll
          for (int c = 0; c < 2; ++c) kf[(s2 + 2) % 3][c] = ld16(Kb + c * 32 * kRowB + kad[s2 + 2]);
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[c] = mfma32x32x16(as_bf16x8(kf[s2 % 3][c]), qb[s2], acc[c]);
        select_part(key0p, sel_prev, s2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    mfma_settle<kSettle32>(acc[0], acc[1]);
    if constexpr (!kPinP) __builtin_amdgcn_s_setprio(0);

    // ---- B: mask, row maximum, rescale; then O += V_{kt-1}^T P_{kt-1}^T
    // beside the group maximum and P of this tile
    if (key0 + 63 > p_wlo) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = key0 + 32 * c + 8 * (i >> 2) + 4 * h + (i & 3);
          if (j > p_lane) acc[c][i] = kNegInf;
        }
      // the group maximum reads the masked scores through DPP from inline
      // assembly: two wait states after their vector writes
      asm volatile("s_nop 1" : "+v"(acc[0]), "+v"(acc[1]));
    }
    float mx = kNegInf;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[c][i]);
    const float dep = mx;
    mx = xor32_max(mx);
    // deferred rescaling (see the gather kernel): P <= 2^kRescaleLog2
    const float m_cand = mx * cexp;
    if (ballot(m_cand > m_run + kRescaleLog2)) {
      pv(Vp, pb_prev, [](int) {});
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) pb_prev[s2] = u32x4{0u, 0u, 0u, 0u};
      mfma_settle4<kSettle32>(oacc);
      const float m_new = fmaxf(m_run, m_cand);
      const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == kNegInf ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int bk = 0; bk < 4; ++bk)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[bk][i] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    float r[16], r2[8];
    float ps[2] = {0.f, 0.f};
    pv(Vp, pb_prev, [&](int m) __attribute__((always_inline)) {
      if constexpr (SEL != 0) {
        if constexpr (G == 1) {
          if (m == 0) gm_store<G>(acc, r, r2, sig[wave]);
        } else {
          if (m == 0) gm_fold8<0, 4>(acc, r, dep);
          if (m == 1) gm_fold8<4, 4>(acc, r, dep);
          if (m == 2) gm_fold8<8, 4>(acc, r, dep);
          if (m == 3) gm_fold8<12, 4>(acc, r, dep);
          if constexpr (G == 2) {
            if (m == 5) gm_store<G>(acc, r, r2, sig[wave]);
          } else {
            if (m == 4) gm_fold4<0, 4>(r, r2, dep);
            if (m == 5) gm_fold4<4, 4>(r, r2, dep);
            if constexpr (G == 8) {
              if (m == 7) gm_fold2(r2);
              if (m == 9) gm_store<G>(acc, r, r2, sig[wave]);
            } else {
              if (m == 7) gm_store<G>(acc, r, r2, sig[wave]);
            }
          }
        }
      }
      // P = exp2(s * scale * log2e - m) for four values per product from
      // product 6 on (after the group maximum has read the raw scores),
      // summed in fp32 and packed to bf16 pairs as they complete
      if (m >= 6 && m < 14) {
        const int v0 = 4 * (m - 6);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = v0 + e, c = v >> 4, i = v & 15;
          acc[c][i] = __builtin_amdgcn_exp2f(fmaf(acc[c][i], cexp, -m_use));
          ps[e & 1] += acc[c][i];
        }
        const int c = v0 >> 4, i0 = v0 & 15, s2 = v0 >> 3, w0 = (v0 & 7) >> 1;
        pb_cur[s2][w0] = pack_bf16x2(acc[c][i0], acc[c][i0 + 1]);
        pb_cur[s2][w0 + 1] = pack_bf16x2(acc[c][i0 + 2], acc[c][i0 + 3]);
        // computed here, beside product m (with selection; see kPinP)
        if constexpr (kPinP)
          asm volatile("" : "+v"(pb_cur[s2][w0]), "+v"(pb_cur[s2][w0 + 1]), "+v"(ps[0]), "+v"(ps[1]));
      }
    });
    l_run += ps[0] + ps[1];
  };

  // two tiles per trip, so that every LDS address is a constant offset
  int kt = 0;
#pragma unroll 1
  for (; kt + 1 < ntiles; kt += 2) {
    tile(kt, std::integral_constant<int, 0>{});
    tile(kt + 1, std::integral_constant<int, 1>{});
  }
  if (kt < ntiles) tile(kt, std::integral_constant<int, 0>{});

  // the last tile's O += V^T P^T, row sums and selection
  auto finish = [&](auto stage_c) __attribute__((always_inline)) {
    constexpr int S = decltype(stage_c)::value;
    const u32x4* pb_last = S ? pbB : pbA;
    const int key0p = (ntiles - 1) * 64;
    const bool sel_last = SEL != 0 && wave_live && key0p <= p_whi - P.window;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kTileWait));
    asm volatile("s_barrier" ::: "memory");
    pv(S ? kv_st1[1] : kv_st0[1], pb_last, [](int) {});
    select_part(key0p, sel_last, -1);
  };
  if (ntiles & 1)
    finish(std::integral_constant<int, 0>{});
  else
    finish(std::integral_constant<int, 1>{});

  mfma_settle4<kSettle32>(oacc);
  const float l_tot = xor32_sum(l_run);
  if (tok_ok) {
    const float inv = 1.f / l_tot;
    uint16_t* op = P.o + (((int64_t)b * P.n_q + tok) * P.Hq + head) * kHeadDim;
#pragma unroll
    for (int bk = 0; bk < 4; ++bk)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[bk][4 * q4] * inv, oacc[bk][4 * q4 + 1] * inv);
        w[1] = pack_bf16x2(oacc[bk][4 * q4 + 2] * inv, oacc[bk][4 * q4 + 3] * inv);
        *reinterpret_cast<u32x2*>(op + 32 * bk + 8 * q4 + 4 * h) = w;
      }
    if (P.lse && h == 0) P.lse[((int64_t)b * P.Hq + head) * P.n_q + tok] = m_run * kLn2 + __logf(l_tot);
  }
  if (SEL == 1 && lane == 0) {
#pragma unroll
    for (int u = 0; u < TPW; ++u)
      if (wt0 + u < P.n_q) P.counts[row0 + (int64_t)u * P.Hkv] = cnt[u];
  }
}

// Scores of sampled keys j = s*stride (s = 0..nsamp(p)-1, nsamp(p) =
// ceil(|C(p)|/stride)) for every (b, t, g) row, computed with the same MFMA
// sequence as the attention kernel, into samples[row][s].
template <int G>
__global__ __launch_bounds__(256, 2) void sample_scores_kernel(SampleParams P) {
  constexpr int TPW = 32 / G;
  constexpr int TPB = 4 * TPW;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * kKS];
  __shared__ __attribute__((aligned(16))) float sig[4][TPW * 64];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31;
  const int ntq = (P.n_q + TPB - 1) / TPB;
  int L = blockIdx.x;
  const int g = L % P.Hkv;
  L /= P.Hkv;
  const int b = L % P.B;
  L /= P.B;
  const int t0 = (ntq - 1 - L) * TPB;
  const int off = P.n_kv - P.n_q;
  const int wt0 = t0 + wave * TPW;
  const int tok = wt0 + tok_of<G>(n);

  bf16x8 qb[8];
  load_q<G>(P.q, b, P.n_q, P.Hq, g, tok, qb);
  // probability score: each lane's column subtracts its head's log-sum-exp
  const bool prob = P.lse != nullptr;
  const float lse_col =
      prob && tok < P.n_q ? P.lse[((int64_t)b * P.Hq + g * G + head_of<G>(n)) * P.n_q + tok] : 0.f;

  const int p_bhi = off + imin(t0 + TPB, P.n_q) - 1;
  const int ncand_hi = imax(0, p_bhi - P.window + 1);
  const int ns_hi = (ncand_hi + P.stride - 1) / P.stride;
  const int ntiles = (ns_hi + 63) / 64;
  const int wlast = imin(wt0 + TPW, P.n_q) - 1;
  const int ns_whi = wt0 < P.n_q ? (imax(0, off + wlast - P.window + 1) + P.stride - 1) / P.stride : 0;

  const int dq = tid & 15, kq = tid >> 4;
  const uint16_t* slab = P.kv.slab(b, g);
  for (int st = 0; st < ntiles; ++st) {
    const int s0 = st * 64;
    {
      u32x4 kw[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int sidx = imin(s0 + 4 * kq + r, ns_hi - 1);
        kw[r] = ld16(slab + (uint32_t)(sidx * P.stride * P.kv.st + 8 * dq));
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) st16(&Ks[(4 * kq + r) * kKS + 8 * dq], kw[r]);
    }
    __syncthreads();
    if (s0 < ns_whi) {
      f32x16 acc[2];
      qk_tile(Ks, qb, acc);
      mfma_settle<kSettle32>(acc[0], acc[1]);
      if (prob) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[c][i] = fmaf(acc[c][i], P.scale, -lse_col);
        dpp_read_pause(acc[0], acc[1]);
      }
      float* ws = sig[wave];
      stage_group_max<G>(acc, ws, fmaxf(acc[0][15], acc[1][15]));
      lds_wait();
      const int s = s0 + lane;
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int tk = wt0 + u;
        if (tk >= P.n_q) continue;
        const int ncand = imax(0, off + tk - P.window + 1);
        const int ns = (ncand + P.stride - 1) / P.stride;
        if (s < ns) {
          const int64_t row = ((int64_t)b * P.n_q + tk) * P.Hkv + g;
          P.samples[row * P.max_samples + s] = prob ? ws[u * 64 + lane] : ws[u * 64 + lane] * P.scale;
        }
      }
    }
    __syncthreads();
  }
}

// Probability-score candidates, after the attention pass has produced lse:
// the selection of the prefill attention kernel on its own. Per 64-key tile,
// S^T = K Q^T, each lane's column turned into scale * s - lse of its head
// (one rounding), the group maximum over the G heads staged in LDS, and every
// candidate j <= p - W at or above its row's threshold appended in ascending
// key order (same buffers and counts as the fused path). K tiles go through
// registers into padded LDS tiles, the next tile's rows in flight while the
// current one is scored.
template <int G>
__global__ __launch_bounds__(256, 2) void score_pass_kernel(PrefillParams P) {
  constexpr int TPW = 32 / G;
  constexpr int TPB = 4 * TPW;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][64 * kKS];
  __shared__ __attribute__((aligned(16))) float sig[4][TPW * 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int ntq = (P.n_q + TPB - 1) / TPB;
  int L = blockIdx.x;
  const int g = L % P.Hkv;
  L /= P.Hkv;
  const int b = L % P.B;
  L /= P.B;
  const int t0 = (ntq - 1 - L) * TPB;
  const int off = P.n_kv - P.n_q;
  const int wt0 = t0 + wave * TPW;
  const int tok = wt0 + tok_of<G>(n);
  const bool wave_live = wt0 < P.n_q;

  bf16x8 qb[8];
  load_q<G>(P.q, b, P.n_q, P.Hq, g, tok, qb);
  const float lse_col = tok < P.n_q ? P.lse[((int64_t)b * P.Hq + g * G + head_of<G>(n)) * P.n_q + tok] : 0.f;

  const int64_t row0 = uniform64(((int64_t)b * P.n_q + wt0) * P.Hkv + g);
  float theta[TPW];
  int cnt[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const bool ok = wt0 + u < P.n_q;
    theta[u] = ok ? __builtin_bit_cast(float, uniform(__builtin_bit_cast(int, P.theta[row0 + (int64_t)u * P.Hkv])))
                  : kPosInf;
    cnt[u] = 0;
  }
  // last candidate key of the block and of this wave (< 0: none)
  const int jb = off + imin(t0 + TPB, P.n_q) - 1 - P.window;
  const int jw = wave_live ? off + imin(wt0 + TPW, P.n_q) - 1 - P.window : -1;
  const int ntiles = jb >= 0 ? jb / 64 + 1 : 0;

  // tile loader: thread (kq, dq) moves rows 4kq .. 4kq+3, 16-byte chunk dq
  const int dq = tid & 15, kq = tid >> 4;
  const uint16_t* slab = P.kv.slab(b, g);
  u32x4 kw[4];
  auto load = [&](int kt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = imin(kt * 64 + 4 * kq + r, jb);  // rows past the last candidate: any valid row
      kw[r] = ld16(slab + (uint32_t)(j * P.kv.st) + 8 * dq);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) st16(&Ks[buf][(4 * kq + r) * kKS + 8 * dq], kw[r]);
  };
  if (ntiles > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ntiles) load(kt + 1);
    const int key0 = kt * 64;
    if (key0 <= jw) {
      f32x16 acc[2];
      qk_tile(Ks[buf], qb, acc);
      mfma_settle<kSettle32>(acc[0], acc[1]);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[c][i] = fmaf(acc[c][i], P.scale, -lse_col);
      dpp_read_pause(acc[0], acc[1]);
      float* ws = sig[wave];
      stage_group_max<G>(acc, ws, fmaxf(acc[0][15], acc[1][15]));
      lds_wait();
      const int j = key0 + lane;
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const float v = ws[u * 64 + lane];
        const bool pass = j <= off + wt0 + u - P.window && v >= theta[u];
        const uint64_t m = ballot(pass);
        const uint32_t o = pass ? 4u * ((uint32_t)cnt[u] + lane_prefix(m)) : kDropOffset;
        const int64_t rb = (row0 + (int64_t)u * P.Hkv) * P.cap;  // wave-uniform row base
        buf_st4(make_rsrc_sized(P.buf_sigma + rb, 4u * (uint32_t)P.cap), o, __float_as_uint(v));
        buf_st4(make_rsrc_sized(P.buf_j + rb, 4u * (uint32_t)P.cap), o, (uint32_t)j);
        cnt[u] = uniform(cnt[u] + __popcll(m));
      }
    }
    if (kt + 1 < ntiles) store(buf ^ 1);
    __syncthreads();
  }
  if (lane == 0) {
#pragma unroll
    for (int u = 0; u < TPW; ++u)
      if (wt0 + u < P.n_q) P.counts[row0 + (int64_t)u * P.Hkv] = cnt[u];
  }
}

template <int G>
hipError_t launch_prefill_g(const PrefillParams& p, hipStream_t s) {
  constexpr int TPB = attn_waves<G>() * (32 / G);
  const int64_t blocks = (int64_t)((p.n_q + TPB - 1) / TPB) * p.B * p.Hkv;
  const dim3 grid((unsigned)blocks), block(64 * attn_waves<G>());
  switch (p.select) {
    case 0: prefill_attn_kernel<G, 0><<<grid, block, 0, s>>>(p); break;
    case 1: prefill_attn_kernel<G, 1><<<grid, block, 0, s>>>(p); break;
    case 2: prefill_attn_kernel<G, 2><<<grid, block, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int G>
hipError_t launch_sample_g(const SampleParams& p, hipStream_t s) {
  constexpr int TPB = 4 * (32 / G);
  const int64_t blocks = (int64_t)((p.n_q + TPB - 1) / TPB) * p.B * p.Hkv;
  sample_scores_kernel<G><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

template <int G>
hipError_t launch_score_pass_g(const PrefillParams& p, hipStream_t s) {
  constexpr int TPB = 4 * (32 / G);
  const int64_t blocks = (int64_t)((p.n_q + TPB - 1) / TPB) * p.B * p.Hkv;
  score_pass_kernel<G><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_pass(const PrefillParams& p, hipStream_t s) {
  switch (p.Hq / p.Hkv) {
    case 1: return launch_score_pass_g<1>(p, s);
    case 2: return launch_score_pass_g<2>(p, s);
    case 4: return launch_score_pass_g<4>(p, s);
    case 8: return launch_score_pass_g<8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t s) {
  switch (p.Hq / p.Hkv) {
    case 1: return launch_prefill_g<1>(p, s);
    case 2: return launch_prefill_g<2>(p, s);
    case 4: return launch_prefill_g<4>(p, s);
    case 8: return launch_prefill_g<8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_sample_scores(const SampleParams& p, hipStream_t s) {
  switch (p.Hq / p.Hkv) {
    case 1: return launch_sample_g<1>(p, s);
    case 2: return launch_sample_g<2>(p, s);
    case 4: return launch_sample_g<4>(p, s);
    case 8: return launch_sample_g<8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hs
