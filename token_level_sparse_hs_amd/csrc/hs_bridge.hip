// KV Bridging: the cross-decoder's full-attention K/V rows built from the
// self-decoder's hidden states ("HySparse2 od Xiaomi zkracuje zpracovani
// dlouheho kontextu", section "Proc neni nutne znovu zpracovat cely dlouhy
// vstup"; DAIR.AI weekly, bullets "Two levels of KV sharing" and "Prefill
// exits early"). Because these rows come from the self-decoder alone, a
// prefill can stop once the self-decoder is done: this projection, written
// straight into the cache, is all the cross-decoder's full-attention layer
// needs of a prefill chunk.
//
// For every batch entry b, chunk token t and KV head g:
//   K[b][g][n_kv - n_q + t] = h[b][t] W_K,g^T,  V likewise with W_V,g,
// with W laid out as a linear layer's weight, [Hkv][2][128][d_model].
//
// Design (MI355X): a bf16 MFMA GEMM in the transposed form C^T = W H^T on
// v_mfma_f32_32x32x16_bf16, so that both operands are rows contiguous in the
// reduction dimension and each lane's results are four consecutive head
// dimensions of one token (8-byte stores into the cache row). One 256-thread
// block = 128 tokens x one (KV head, K or V) output of 128 dimensions; the
// four waves take 64 x 64 quadrants. 64-wide reduction tiles of W and h go
// through registers into LDS (rows padded to 144 bytes: the 16-byte operand
// reads of 16 consecutive rows hit distinct banks), the next tile's loads in
// flight while the current one is multiplied. The eight (head, K|V) blocks of
// a token tile are adjacent in the grid, so they share the tile's hidden
// states in L2. fp32 accumulation; results rounded to bf16 (nearest even).
#include "hs_common.hpp"
#include "hs_kernels.hpp"

namespace hs {

namespace {

constexpr int kBT = 128;     // tokens per block
constexpr int kBK = 64;      // reduction tile
constexpr int kRow = kBK + 8;  // LDS row stride in bf16 (144 bytes)

__global__ __launch_bounds__(256, 2) void kv_bridge_kernel(BridgeParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][128 * kRow];  // W rows (dims) x k
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBT * kRow];  // h rows (tokens) x k
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  int L = blockIdx.x;
  const int hs2 = L % (2 * P.Hkv);  // (head, K|V) fastest: blocks of one token tile are adjacent
  L /= 2 * P.Hkv;
  const int ntt = (P.n_q + kBT - 1) / kBT;
  const int tt = L % ntt;
  const int b = L / ntt;
  const int g = hs2 >> 1, s = hs2 & 1;
  const int t0 = tt * kBT;

  // Loader: thread (row r = tid / 8 + 32 i, chunk c = tid % 8) moves 16 bytes.
  const int lr = tid >> 3, lc = tid & 7;
  const uint16_t* wsrc = P.w + ((int64_t)(g * 2 + s) * 128) * P.d_model + 8 * lc;
  const uint16_t* hsrc = P.h + ((int64_t)b * P.n_q) * P.d_model + 8 * lc;
  u32x4 ra[4], rb[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lr + 32 * i;
      ra[i] = ld16(wsrc + (int64_t)r * P.d_model + k0);
      const int tok = imin(t0 + r, P.n_q - 1);  // rows past the chunk: any valid row, not stored
      rb[i] = ld16(hsrc + (int64_t)tok * P.d_model + k0);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lr + 32 * i;
      st16(&As[buf][r * kRow + 8 * lc], ra[i]);
      st16(&Bs[buf][r * kRow + 8 * lc], rb[i]);
    }
  };

  f32x16 acc[2][2] = {};
  const int n = lane & 31, kh = lane >> 5;
  const int nk = P.d_model / kBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8 a[2], bb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = as_bf16x8(ld16(&As[buf][(64 * wm + 32 * i + n) * kRow + 16 * ks + 8 * kh]));
        bb[i] = as_bf16x8(ld16(&Bs[buf][(64 * wn + 32 * i + n) * kRow + 16 * ks + 8 * kh]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], bb[j], acc[i][j]);
    }
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }
  mfma_settle4<kSettle32>(&acc[0][0]);

  // acc[i][j], register r: dim 64 wm + 32 i + 8 (r / 4) + 4 kh + r % 4, token
  // t0 + 64 wn + 32 j + n: four consecutive dims per 8-byte store.
  uint16_t* slab = P.kv + (int64_t)b * P.sb + (int64_t)g * P.sh + (s ? P.voff : 0);
  const int row0 = P.n_kv - P.n_q;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tok = t0 + 64 * wn + 32 * j + n;
    if (tok >= P.n_q) continue;
    uint16_t* dst = slab + (int64_t)(row0 + tok) * P.st;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int dim = 64 * wm + 32 * i + 8 * q4 + 4 * kh;
        u32x2 w;
        w[0] = pack_bf16x2(acc[i][j][4 * q4], acc[i][j][4 * q4 + 1]);
        w[1] = pack_bf16x2(acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]);
        *reinterpret_cast<u32x2*>(dst + dim) = w;
      }
  }
}

}  // namespace

hipError_t launch_kv_bridge(const BridgeParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)((p.n_q + kBT - 1) / kBT) * p.B * p.Hkv * 2;
  kv_bridge_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace hs
