// Device-side building blocks shared by the libhysparse kernels (gfx950).
//
// Lane layouts of the bf16 matrix-core instructions used below (wave64):
//   v_mfma_f32_32x32x16_bf16  A[m][k]: lane l holds row m = l%32, k = 8*(l/32)+e
//                             B[k][n]: lane l holds col n = l%32, k = 8*(l/32)+e
//                             C[m][n]: lane l, reg i -> m = 8*(i/4)+4*(l/32)+i%4,
//                                                     n = l%32
//   v_mfma_f32_16x16x32_bf16  A: m = l%16, k = 8*(l/16)+e;  B: n = l%16,
//                             k = 8*(l/16)+e;  C: reg i -> m = 4*(l/16)+i,
//                             n = l%16
//   v_mfma_f32_16x16x16_bf16  as 16x16x32 with k = 4*(l/16)+e, e = 0..3
// (e = 0..7 indexes the eight bf16 of an operand register quad.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();
constexpr float kRescaleLog2 = 8.f;  // deferred-rescale slack of the online softmax (log2 units)

// ---------------------------------------------------------------- bf16 data

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even float pair -> packed bf16 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// ---------------------------------------------------------------- matrix core

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x16_bf16: A: m = l%16, k = 4*(l/16)+e; B: n = l%16,
// k = 4*(l/16)+e (e = 0..3); C as for 16x16x32.
// Pause before VALU code reads matrix results. On gfx950 the results of
// v_mfma_f32_{32x32x16,16x16x32}_bf16 arrive later than the wait states the
// compiler inserts before a dependent VALU read: a read a few instructions
// after the last MFMA of a chain (across a branch) returned partly written
// accumulators. Measured on the decode sparse layer: the row maximum read
// right after its score tile varied from run to run while the scores read
// later did not (repeated calls then differed by one bf16 ulp); 8 extra wait
// states removed it. The accumulators are tied to an explicit pause of
// kSettle16 (16x16 tiles) or kSettle32 (32x32 tiles) wait states, so every
// later read is ordered after it.
constexpr int kSettle16 = 12;
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x2;
constexpr int kSchedMfma = 0x8;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedDsWrite = 0x200;
constexpr int kSettle32 = 20;
#define HS_NOPS_12 "s_nop 11"
#define HS_NOPS_20 "s_nop 15\n\ts_nop 3"
template <int N, typename A>
__device__ __forceinline__ void mfma_settle(A& a) {
  static_assert(N == 12 || N == 20, "settle length");
  if constexpr (N == 12) asm volatile(HS_NOPS_12 : "+v"(a));
  else asm volatile(HS_NOPS_20 : "+v"(a));
}
template <int N, typename A, typename B>
__device__ __forceinline__ void mfma_settle(A& a, B& b) {
  static_assert(N == 12 || N == 20, "settle length");
  if constexpr (N == 12) asm volatile(HS_NOPS_12 : "+v"(a), "+v"(b));
  else asm volatile(HS_NOPS_20 : "+v"(a), "+v"(b));
}
template <int N, typename A>
__device__ __forceinline__ void mfma_settle4(A* a) {
  static_assert(N == 12 || N == 20, "settle length");
  if constexpr (N == 12) asm volatile(HS_NOPS_12 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
  else asm volatile(HS_NOPS_20 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
}
template <int N, typename A>
__device__ __forceinline__ void mfma_settle8(A* a) {
  static_assert(N == 12 || N == 20, "settle length");
  if constexpr (N == 12)
    asm volatile(HS_NOPS_12 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]),
                 "+v"(a[7]));
  else
    asm volatile(HS_NOPS_20 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]),
                 "+v"(a[7]));
}

__device__ __forceinline__ f32x4 mfma16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c,
                                                    0, 0, 0);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, the lanes' 8-byte
// pieces (4 bf16 each, read at each lane's own address, in lane order) form a
// 4 x 16 matrix; lane i of the group receives column i. With a row-major tile
// T[row][col] and lane j = 4r + c of a group addressing T[row0 + r][col0 + 4c],
// lane i receives T[row0 + 0..3][col0 + i].
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// ---------------------------------------------------------------- cross-lane

// DPP controls (gfx9 encoding).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16
constexpr int kDppRowRor8 = 0x128;    // row_ror:8: lane i <-> lane i ^ 8 within 16

// With NaN-free, non-IEEE-mode compilation (see the build flags) a DPP move
// feeding a max folds into a single v_max_f32_dpp.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(v), CTRL, 0xF, 0xF, true));
}

// Max over aligned groups of N consecutive lanes (N in {1,2,4,8}); every lane
// of a group receives the group maximum.
template <int N>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp<kDppXor1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp<kDppXor2>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
  return v;
}

// Combine lane l with lane l^32 (max / sum).
// Transposing max across lane rows: with rows of 16 lanes, returns
// max(a[l], a[l ^ 16]) in even rows and max(b[l], b[l ^ 16]) in odd rows
// (one v_permlane16_swap and one max for two values).
__device__ __forceinline__ float row_pair_max(float a, float b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xor32_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Combine lane l with lane l^16.
__device__ __forceinline__ float xor16_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }
// Marks a wave-uniform value as such (keeps it in a scalar register, so that
// branches on it stay scalar).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Raw buffer over [base, base + 4 GiB): 16-byte loads at a 32-bit byte
// offset with no per-lane 64-bit address arithmetic (gfx9 resource word 3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xffffffff, 0x00020000);
}
__device__ __forceinline__ uint32_t buf_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ u32x2 buf_ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}

// Eight e4m3 codes (byte i = element i) to eight bf16 (element 2i in the low
// half of word i): every e4m3 value is a bf16 value, so this is exact.
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(u32x2 w) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true));
  return r;
}
// Buffer over [base, base + bytes): a store at an offset at or past `bytes`
// is discarded and a load there returns 0 (hardware range check), so lanes
// that must not access memory still execute the instruction (no divergent
// branch around it). The check is per 4-byte element: a 16-byte load that
// runs past `bytes` returns its elements below `bytes` and 0 for the rest
// (the decode selection's ragged-tail test relies on it).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_sized(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void buf_st16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_st4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}
constexpr uint32_t kDropOffset = 0x80000000u;

// Raw buffer descriptor (base, range in bytes, no stride) as four scalar
// words, for inline assembly.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)uniform((int)(uint32_t)a), (uint32_t)uniform((int)(uint32_t)(a >> 32)) & 0xffffu,
               (uint32_t)uniform((int)bytes), 0x00020000u};
}
// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Direct global->LDS load of 16 bytes per lane (buffer_load_dwordx4 ... lds):
// lane l's bytes land at LDS address lds + 16 l. The compiler does not see an
// LDS write here: callers order it with s_waitcnt vmcnt and barriers.
__device__ __forceinline__ void lds_dma16(uint32_t lds, uint32_t voff, u32x4 rsrc, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"((uint32_t)uniform((int)lds)), "v"(voff), "s"(rsrc), "s"(soff)
               : "m0");
}  // past every buffer range: the store is dropped
__device__ __forceinline__ uint32_t lane_prefix(uint64_t mask) {  // set bits below this lane
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// ---------------------------------------------------------------- score keys

// Monotone map of a finite float to uint32 (larger float -> larger key), with
// -0.0 mapped like +0.0 so that the two zeros tie.
// Branch-free (selects and bit operations only): under a condition, a branch
// here made the compiler wait for every outstanding load before each key.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  u = u == 0x80000000u ? 0u : u;
  const uint32_t neg = (uint32_t)((int32_t)u >> 31);  // all ones for a negative score
  return u ^ (neg | 0x80000000u);
}
// score_key(x) where `valid`, else 0 (the empty key).
__device__ __forceinline__ uint32_t score_key_if(float x, bool valid) { return score_key(x) & (0u - (uint32_t)valid); }
__device__ __forceinline__ float key_to_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------- misc

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
__device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }

// Decode length of sequence b as the kernels read it: seq_lens[b] clamped to
// the host bound the launch was sized for, so that a caller's length beyond
// that bound (an error, or a graph replayed past its bucket) yields a wrong
// but in-bounds result rather than accesses past the workspace rows.
__device__ __forceinline__ int dec_len(const int32_t* seq_lens, int b, int max_len) {
  return imin(seq_lens[b], max_len);
}

// Cache addressing. One (b, g) slab spans fewer than 2^31 elements (checked
// on the host), so rows inside a slab use 32-bit offsets from a 64-bit slab
// base computed once.
struct KvView {
  const uint16_t* base;
  int64_t sb, sh;
  int32_t st, voff;
  __device__ __forceinline__ const uint16_t* slab(int b, int g) const {
    return base + (int64_t)b * sb + (int64_t)g * sh;
  }
  __device__ __forceinline__ const uint16_t* k_row(int b, int g, int t) const {
    return slab(b, g) + (uint32_t)(t * st);
  }
  __device__ __forceinline__ const uint16_t* v_row(int b, int g, int t) const {
    return slab(b, g) + (uint32_t)(t * st + voff);
  }
};

}  // namespace hs
