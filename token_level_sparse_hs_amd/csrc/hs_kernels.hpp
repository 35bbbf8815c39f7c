// Kernel parameter blocks and launchers of libhysparse (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hs_common.hpp"

namespace hs {

constexpr int kMaxTopK = 8192;   // largest supported top_k

// Library-owned device scratch of hs_decode_step_noalloc: one array per GPU
// (a file-scope __device__ array), its address looked up once per device.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
hipError_t static_scratch(void** ptr);
constexpr int kPrefillKeyTile = 64;

// ----------------------------------------------------------- prefill attention
struct PrefillParams {
  const uint16_t* q;  // [B][n_q][Hq][128]
  KvView kv;
  uint16_t* o;        // [B][n_q][Hq][128]
  float* lse;         // [B][Hq][n_q] or null
  int B, n_q, n_kv, Hq, Hkv, window;
  float scale;
  // selection (select == 0: no selection, buffers unused; 1: token-level
  // candidates into buf_sigma / buf_j; 2: block level, the best scaled score
  // of each 64-key block's candidates into blk_score)
  int select;
  float* blk_score;    // [rows][blk_stride]
  int blk_stride;
  const float* theta;  // [rows] scaled-score threshold per (b,t,g) row
  float* buf_sigma;    // [rows][cap]
  int32_t* buf_j;      // [rows][cap]
  int32_t* counts;     // [rows]
  int cap;
};

// Sampled scores for the per-row filter thresholds.
struct SampleParams {
  const uint16_t* q;
  KvView kv;
  int B, n_q, n_kv, Hq, Hkv, window;
  float scale;
  int stride;       // sampled keys j = s * stride
  int max_samples;  // row stride of `samples`
  float* samples;   // [rows][max_samples]
  const float* lse; // probability score: [B][Hq][n_q] log-sum-exp; null for the logit score
};

hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t s);
hipError_t launch_sample_scores(const SampleParams& p, hipStream_t s);
// Probability-score candidate pass: the selection part of the prefill
// attention kernel alone (QK, group maximum of scale*s - lse, threshold
// compaction into buf_sigma / buf_j / counts), reading lse from p.lse.
hipError_t launch_score_pass(const PrefillParams& p, hipStream_t s);

// ------------------------------------------------------------------ selection
struct SelectParams {
  const uint16_t* q;
  KvView kv;
  int B, n_q, n_kv, Hq, Hkv, top_k, window;
  float scale;
  const float* buf_sigma;
  const int32_t* buf_j;
  const int32_t* counts;
  int cap;
  int force_rescan;
  int32_t* idx;            // [rows][top_k]
  uint32_t* rescan_count;  // optional counter of rows that took the rescan
  int32_t* defer_rows;     // [rows] rows left to the block-wide path
  uint32_t* defer_count;   // zeroed by the threshold kernel of the same call
  const float* lse;        // probability score: [B][Hq][n_q] for the exact rescan; null: logit score
};

struct ThresholdParams {
  int B, n_q, n_kv, Hkv, top_k, window, cap, stride, max_samples;
  uint32_t* defer_count;  // [2]: queued rows, rescanned rows; zeroed here (block 0)
                          // for the selection that follows
  const float* samples;
  float* theta;
};

struct SelectDecodeParams {
  int B, Hkv, top_k, window;
  const int32_t* seq_lens;
  int max_len;         // host bound on seq_lens (longer lengths are read as max_len)
  const float* sigma;  // [B*Hkv][sigma_stride]
  int64_t sigma_stride;
  int32_t* idx;        // [B][Hkv][top_k]
  // Sliced path (nslices > 0) for rows longer than one block holds in
  // registers: per-row threshold, a filter over row slices of kDecSlice keys
  // (one wave each), then one block per row on the survivors.
  int nslices;         // slices per row (covers the longest row)
  uint32_t* theta_key; // [rows] filter threshold (score key; 0 = no filter)
  const float* samp;   // [rows][kDecSamples] every 2^dec_sample_shift-th score of the row
  uint32_t* seg_count; // [rows][nslices] survivors per slice
  uint32_t* seg_key;   // [rows][nslices][kDecSlice] survivors' scores (fp32 bits), index order
  int32_t* seg_idx;    // [rows][nslices][kDecSlice] survivors' token indices
};
// Sliced decode selection: keys per filter wave; rows of up to kSelRegKeys
// candidates are selected directly from registers by one block.
constexpr int kDecSlice = 4096;
constexpr int kSelRegKeys = 8192;
constexpr int kMaxDecSlices = 4096;
// The kernel that writes a decode score row also writes its samples for the
// sliced threshold: scores at j = 2^s * i for i < ceil(|C| / 2^s), with s the
// smallest shift of at least 2 leaving at most kDecSamples of them. A shift
// of at least 2 puts each sample at the start of an aligned 4-key piece.
constexpr int kDecSamples = 16384;
__host__ __device__ __forceinline__ int dec_sample_shift(int ncand) {
  int s = 2;
  while (((ncand + (1 << s) - 1) >> s) > kDecSamples) ++s;
  return s;
}

// Decode probability-score row: sigma[(b,g)][j] = max over the group's heads
// of fl(scale * <q_h, k_j>) - lse_h for j in C(p), fp32 dot products in
// dimension order.
struct DecodeScoreParams {
  const uint16_t* q;  // [B][Hq][128]
  KvView kv;
  const int32_t* seq_lens;
  const float* lse;   // [B][Hq]
  int B, Hq, Hkv, window;
  float scale;
  float* sigma;       // [B*Hkv][sigma_stride]
  int64_t sigma_stride;
  int max_cand;       // bound on |C(p)| over the batch (grid size)
  int max_len;        // host bound on seq_lens (longer lengths are read as max_len)
  int per_head;       // 1: each head's scaled logit into row b*Hq + h (lse unused)
  float* samp;        // [rows][kDecSamples] the rows' samples (null: none)
};
hipError_t launch_decode_prob_score(const DecodeScoreParams& p, hipStream_t s);

// Union of per-head top-k lists: output row `row` (a (b, t, g) or (b, g)
// row) merges lists lists + row*row_stride + r*head_stride, r < G, each k
// entries ascending and -1 padded, into G*k entries ascending, -1 padded.
struct UnionParams {
  const int32_t* lists;
  int64_t row_stride, head_stride;
  int G, k;
  int B, n_q, n_kv, Hkv, window;
  const int32_t* seq_lens;  // decode rows; null for prefill rows
  int max_len;              // decode rows: host bound on seq_lens
  int32_t* out;
};
hipError_t launch_head_union(const UnionParams& p, int64_t rows, hipStream_t s);
// Head slices: dst row (bt, g) <- src row (bt, g*G + r) (gather) or dst row
// (bt, g*G + r) <- src row (bt, g) (scatter), 128 bf16 each; lse scatter:
// dst [B][Hkv*G][n] row (b, g*G + r) <- src [B][Hkv][n] row (b, g).
hipError_t launch_head_slice(const uint16_t* src, uint16_t* dst, int64_t bt, int Hkv, int G, int r, bool gather,
                             hipStream_t s);
hipError_t launch_lse_scatter(const float* src, float* dst, int B, int Hkv, int G, int r, int n, hipStream_t s);

// Block-level selection: the top top_k/64 blocks of each row by block score
// (ties: lower block), expanded to their candidate tokens.
struct BlockSelectParams {
  int B, n_q, n_kv, Hkv, top_k, window;
  const int32_t* seq_lens;  // decode rows; null for prefill rows
  int max_len;              // decode rows: host bound on seq_lens
  const float* blk_score;   // [rows][blk_stride]
  int blk_stride;
  int32_t* idx;             // [rows][top_k]
};
hipError_t launch_select_blocks(const BlockSelectParams& p, int64_t rows, hipStream_t s);
// Decode: block scores from the dense score rows.
struct BlockMaxParams {
  const float* sigma;
  int64_t sigma_stride;
  const int32_t* seq_lens;
  int max_len;  // host bound on seq_lens
  int B, Hkv, window;
  float* blk_score;
  int blk_stride;
};
hipError_t launch_block_max(const BlockMaxParams& p, hipStream_t s);

hipError_t launch_select_prefill(const SelectParams& p, int64_t rows, hipStream_t s);
hipError_t launch_threshold(const ThresholdParams& p, int64_t rows, hipStream_t s);
hipError_t launch_select_decode(const SelectDecodeParams& p, int rows, hipStream_t s);

// --------------------------------------------------------- flash-decode family
// One wave per work item. FULL: contiguous keys [k0, k1) of a decode row,
// writes the group score row. SPARSE: keys = idx row U forced window.
struct DecodeParams {
  const uint16_t* q;  // prefill: [B][n_q][Hq][128]; decode: [B][Hq][128]
  KvView kv;
  int B, n_q, n_kv, Hq, Hkv, top_k, window;
  float scale;
  const int32_t* seq_lens;  // decode: [B]; prefill: null
  const int32_t* idx;       // SPARSE: [B][n_q][Hkv][top_k]
  int splits;               // key splits per (b, g) (decode only)
  int split_len;            // keys per split (FULL) / virtual keys per split (SPARSE)
  // outputs
  uint16_t* o;              // used when splits == 1
  float* lse;               // [B][Hq][n_q] or null (splits == 1)
  float* part;              // splits > 1 (global merge): [B][Hkv][splits][G][128 + 2]
  int combine_in_block;     // decode, splits == 4: a block's four waves are the four
                            // splits of one (b, g) row and merge in LDS (part unused)
  float* sigma;             // FULL: [B*Hkv][sigma_stride]
  int64_t sigma_stride;
  float* samp;              // FULL with sigma: [B*Hkv][kDecSamples] samples of the score rows (or null)
  // SPARSE from the FP8 cache copy (kv8 != null; kv unused): rows of
  // [B][Hkv][kv8_cap] tokens, K then V codes, and per-(b, g) scales.
  const uint8_t* kv8;
  const float* kv8_scale;   // [B][Hkv][2]: 2^e of K and of V
  int64_t kv8_cap;
};

// FP8 (e4m3) copy of a bf16 cache for the sparse gathers. Buffer layout:
// codes [B][Hkv][cap][2][128] (256 bytes per token: K then V), then amax bits
// [B][Hkv][2] (uint32, scratch of the conversion), then scales [B][Hkv][2]
// (float, 2^e of K and of V). Prefill form: per (b, g), e = the smallest
// exponent with max|x| over rows [0, n_kv) <= 448 * 2^e, separately for K
// and V, then every row converted as e4m3(clamp(x / 2^e, +-448)) rounded to
// nearest even. Decode form (seq_lens given): row seq_lens[b] - 1 converted
// with the stored scales.
constexpr int kFp8RowBytes = 256;
struct Fp8ConvertParams {
  KvView kv;
  uint8_t* kv8;
  int B, Hkv, n_kv;
  int64_t cap;
  const int32_t* seq_lens;
};
__host__ __device__ inline int64_t kv8_codes_bytes(int B, int Hkv, int64_t cap) {
  return (int64_t)B * Hkv * cap * kFp8RowBytes;
}
__host__ __device__ inline int64_t kv8_total_bytes(int B, int Hkv, int64_t cap) {
  return kv8_codes_bytes(B, Hkv, cap) + (int64_t)B * Hkv * 16;
}
hipError_t launch_kv_convert_fp8(const Fp8ConvertParams& p, hipStream_t s);

struct AppendParams {
  const uint16_t* kv_new;  // [B][Hkv][2][128]
  uint16_t* kv;
  int64_t sb, sh, st, voff;
  const int32_t* seq_lens;
  int B, Hkv, cap;
};

struct CombineParams {
  const float* part;
  uint16_t* o;   // [B][Hq][128]
  float* lse;    // [B][Hq] or null
  const int32_t* seq_lens;
  int B, Hq, Hkv, splits, split_len;
  int sparse_k;  // SPARSE: top_k (virtual keys = top_k + |Win|); FULL: -1
  int window;
  int max_len;   // host bound on seq_lens
};

// KV Bridging: rows [n_kv - n_q, n_kv) of every (b, g) of the cache from
// hidden states h [B][n_q][d_model] and weights w [Hkv][2][128][d_model].
struct BridgeParams {
  const uint16_t* h;
  const uint16_t* w;
  uint16_t* kv;
  int64_t sb, sh, st, voff;  // cache strides (elements)
  int B, n_q, n_kv, Hkv, d_model;
};
hipError_t launch_kv_bridge(const BridgeParams& p, hipStream_t s);

// Gather-rate probe: 512-byte token rows of src at the indices idx[0..n),
// per_wave keys per wave; out gets one folded word per lane.
struct ProbeParams {
  const uint8_t* src;
  uint32_t src_bytes;
  const int32_t* idx;
  int64_t n;
  int per_wave;
  uint32_t* out;  // [waves * 64]
};
hipError_t launch_gather_probe(const ProbeParams& p, hipStream_t s);

hipError_t launch_decode_full(const DecodeParams& p, hipStream_t s);
hipError_t launch_sparse(const DecodeParams& p, hipStream_t s);
hipError_t launch_append(const AppendParams& p, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, hipStream_t s);

}  // namespace hs
