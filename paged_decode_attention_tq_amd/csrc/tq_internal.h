// Internal structures shared by the host code (tq_host.cpp) and the HIP
// kernels (tq_write.hip, tq_decompress.hip, tq_decode.hip, tq_decode_wave.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

constexpr int kHeadDim = 128;    // the kernels are built for head_dim 128
constexpr int kBlockSize = 16;   // decode page size (tokens per page)
constexpr int kDecodeLdsBytes = 160 * 1024;  // LDS of one gfx950 CU, all of it used by the decode
constexpr int kMaxGroup = 64;    // query heads per KV head (groups of 8 per wave)

// Arguments of the row-writer kernel (passed by value as kernel arguments).
struct WriteArgs {
  const void* raw;          // [num_tokens, num_kv_heads, 128]
  uint8_t* pages;           // [num_blocks, block_size, num_kv_heads, row_bytes]
  const int64_t* slots;     // [num_tokens]
  int32_t* err_count;       // nullable
  int64_t num_rows;         // num_tokens * num_kv_heads
  int64_t num_slots;        // num_blocks * block_size
  int64_t page_bytes;       // block_size * num_kv_heads * row_bytes
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t row_bytes;
  uint32_t sign_bits[kHeadDim / 32];   // bit i set <=> sign_i = -1
  float pos_bounds[16];     // the 2^(b-1) - 1 positive boundaries, increasing
};

// Arguments of the prod key writer (tq_write.hip): the MSE part of w uses
// bits - 1 (pos_bounds are that codebook's), sketch is the d x d matrix S
// (row-major fp32, device), cpos the 2^(bits-2) positive centroids of the
// bits - 1 codebook, increasing.
struct ProdWriteArgs {
  WriteArgs w;
  const float* sketch;
  float cpos[16];
};

// Arguments of the prod-key score kernels (tq_qjl.hip): estimated inner
// products of each query head with every key row of its sequence.
struct ProdScoreArgs {
  const void* q;                 // [B, Hq, 128] of q_dtype
  const uint8_t* pages;          // prod rows [num_blocks, 16, Hkv, row_bytes]
  const int32_t* block_table;    // [B, max_blocks_per_seq]
  const int32_t* seq_lens;       // [B], clamped to 0 .. max_len
  const float* sketch;           // [128, 128] row-major
  float* qr;                     // [B, Hq, 128] workspace: rht(q)
  float* sq;                     // [B, Hq, 128] workspace: S rht(q)
  float* scores;                 // [B, Hq, max_seq_len]
  int64_t page_bytes;
  int64_t num_blocks;            // block ids outside [0, num_blocks) read as zero rows
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t max_seq_len;           // columns of scores
  int32_t max_len;               // lengths are clamped to this (the block table's reach)
  int32_t row_bytes;
  int32_t q_dtype;
  int32_t chunk_pages;           // pages per workgroup (a multiple of 4)
  int32_t chunks;                // ceil(pages of max_seq_len / chunk_pages)
  int32_t vec_store;             // scores rows 16-byte aligned (max_seq_len % 4 == 0, aligned base)
  int32_t head_group;            // H: KV heads of one workgroup (a divisor of num_kv_heads)
  int32_t phases;                // P = 4 / H: the waves of one head split its pages P ways
  uint32_t sign_bits[kHeadDim / 32];
  float cent[16];                // the 2^(bits-1) centroids of the index codebook, times 16
};

// Arguments of the dense readback kernel (tq_decompress.hip).
struct ReadArgs {
  const uint8_t* pages;     // [num_blocks, block_size, num_kv_heads, row_bytes]
  const int64_t* slots;     // [num_tokens]
  void* out;                // [num_tokens, num_kv_heads, 128] of the output dtype, 16-byte aligned
  int32_t* err_count;       // nullable
  int64_t num_slots;        // num_blocks * block_size
  int64_t page_bytes;       // block_size * num_kv_heads * row_bytes (< 2^31)
  uint32_t num_rows;        // num_tokens * num_kv_heads (< 2^31)
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t row_bytes;
  int32_t hkv_shift;        // log2(num_kv_heads), or -1 when not a power of two
  int32_t bs_shift;         // log2(block_size), or -1 when not a power of two
  float cent[32];           // the 2^bits fp32 centroids
  // Sign of coordinate 32 q + j as held by quad lane q: bit j of neg_bits[q]
  // is set when the rotation sign s_(32q+j) times the parity sign
  // (-1)^popcount(q) that the quad butterflies leave is negative.
  uint32_t neg_bits[4];
};

// The new row of every sequence appended by the decode itself
// (tq_paged_decode_append): the K and V rows of sequence b's last token
// (position L_b - 1, L_b its clamped length) are encoded as the row writer
// encodes them and stored in that token's page, by the staged decode's
// workgroup that reads the page before any of its waves reads it, or by the
// appending row writer ahead of the wave-private decode.  on == 0: nothing
// is written.
struct AppendArgs {
  const void* k_new;             // [B, Hkv, 128] of new_dtype
  const void* v_new;
  int32_t* err_count;            // nullable: sequences whose last page has a block id outside the pages
  int32_t on;
  int32_t new_dtype;             // tq_dtype of k_new and v_new
  float k_bounds[16];            // the 2^(b_k - 1) - 1 positive boundaries of the K codebook, increasing
  float v_bounds[16];
};

// Arguments of the appending row writer (tq_write.hip), used where the decode
// kernel does not append the rows itself: row r = 2 (b Hkv + head) + comp of
// the launch encodes component comp (0 K, 1 V) of sequence b's new row for
// head `head` at its last token, found on the device from seq_lens and the
// block table exactly as the decode finds it.
struct AppendWriteArgs {
  AppendArgs app;
  uint8_t* k_pages;
  uint8_t* v_pages;
  const int32_t* block_table;    // [B, max_blocks_per_seq]
  const int32_t* seq_lens;       // [B]
  int64_t k_page_bytes;
  int64_t v_page_bytes;
  int64_t num_blocks;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t max_len;               // lengths are clamped to this, as by the decode
  int32_t k_row_bytes;
  int32_t v_row_bytes;
  uint32_t sign_bits[kHeadDim / 32];
};

// Arguments of the decode split kernel.  One workgroup handles one
// (sequence, group of kv_per_wg KV heads, split of pages_per_split pages)
// with waves = kv_per_wg * q_groups * streams waves: each wave owns one KV
// head, one group of up to 8 of its query heads, and one page of every
// stage (streams consecutive pages).  The workgroup copies each stage
// straight into one of two LDS slots, one stage ahead of the compute.
struct DecodeArgs {
  const void* q;                 // [B, Hq, 128]
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const int32_t* block_table;    // [B, max_blocks_per_seq]
  const int32_t* seq_lens;       // [B]
  float* part_acc;               // [B, Hq, S, 128]  rotated, normalised, x v_scale
  float* part_lse;               // [B, Hq, S]       log2-sum-exp2 of the split
  int64_t k_page_bytes;
  int64_t v_page_bytes;
  int64_t num_blocks;            // block ids outside [0, num_blocks) read as zero rows
  int32_t max_len;               // lengths are clamped to this (the block table and split coverage)
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;                 // num_q_heads / num_kv_heads
  int32_t q_groups;              // ceil(group / 8)
  int32_t k_row_bytes;
  int32_t v_row_bytes;
  int32_t max_blocks_per_seq;
  int32_t kv_per_wg;             // KV heads of one workgroup
  int32_t head_groups;           // num_kv_heads / kv_per_wg
  int32_t streams;               // pages per stage
  int32_t waves;                 // kv_per_wg * q_groups * streams (<= 16)
  int32_t pages_per_split;       // pages per workgroup
  int32_t num_splits;            // S
  int32_t q_dtype;               // tq_dtype of q
  // staging (per component): whole pages when kv_per_wg == num_kv_heads
  // (each row in a 16-byte aligned slice, token rows of an odd number of
  // chunks), else a token's slice of the workgroup's heads as C 16-byte chunks
  int32_t k_tok_chunks, v_tok_chunks;  // 16-byte chunks per token row: C (slices) or tc (whole pages)
  int32_t k_slice_chunks, v_slice_chunks;  // whole pages: chunks per (token, head) slice, ceil(RB / 16)
  int32_t k_chunks, v_chunks;    // 16-byte chunks per page
  int32_t k_loads, v_loads;      // 1 KB loads per page: ceil(chunks / 64)
  int32_t k_region;              // LDS bytes of a page's K part: 16 k_chunks
  int32_t page_slot_bytes;       // 16 (k_chunks + v_chunks)
  int32_t stage_bytes;           // streams * page_slot_bytes
  int32_t bt_base;               // LDS byte offset of the split's block ids
  float q_scale;                 // softmax scale * log2(e) / (sqrt(128) * k_scale)
  uint32_t sign_bits[kHeadDim / 32];
  float k_cent[32];              // fp32 centroids of K times k_scale
  float v_cent[32];              // fp32 centroids of V times v_scale
  AppendArgs app;
};

// Arguments of the wave-private decode kernel (tq_decode_wave.hip).  The
// pages of every sequence are concatenated in sequence order (sequence b
// holds ceil(min(seq_lens[b], max_len) / 16) of them) and workgroup i of
// num_wg takes pages [i T / num_wg, (i + 1) T / num_wg) of the T in total,
// one sequence segment after the other.  Every wave of a workgroup owns all
// KV heads (1, 2 or 4), loads whole pages with its own 16-byte loads into a
// private LDS slot and computes every head's query group (group <= 8 query
// heads per KV head); the waves of a workgroup (streams) walk alternate
// pages of a segment and merge at its end.  Partial results of sequence b
// from workgroup i go to workspace slot b + i; a sequence whose pages all
// fall in one workgroup's share is finished by that workgroup (out).
struct WaveArgs {
  const void* q;                 // [B, Hq, 128]
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const int32_t* block_table;    // [B, max_blocks_per_seq]
  const int32_t* seq_lens;       // [B]
  float* part_acc;               // [B + num_wg - 1, Hq, 128] rotated, normalised, x v_scale
  float* part_lse;               // [B + num_wg - 1, Hq]      log2-sum-exp2 of the segment
  float* out;                    // [B, Hq, 128]: written here for every sequence whose pages one workgroup holds
  float* lse_out;                // [B, Hq] or null: log2-sum-exp2 of the scores wherever out is written (-inf: empty)
  int64_t k_page_bytes;
  int64_t v_page_bytes;
  int64_t num_blocks;            // block ids outside [0, num_blocks) read as zero rows
  int32_t max_len;               // lengths are clamped to this (the block table's reach)
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;                 // num_q_heads / num_kv_heads (<= 8)
  int32_t max_blocks_per_seq;
  int32_t num_wg;                // workgroups of the launch
  int32_t q_dtype;               // tq_dtype of q
  int32_t direct;                // 1: no merge kernel follows (one workgroup): empty sequences are zeroed here too
  float q_scale;                 // softmax scale * log2(e) / (sqrt(128) * k_scale)
  float out_scale;               // 1 / (v_scale * sqrt(128)): value scale and the rotation's normalisation
  uint32_t sign_bits[kHeadDim / 32];
  float k_cent[32];              // fp32 centroids of K times k_scale
  float v_cent[32];              // fp32 centroids of V times v_scale
};

// Arguments of the merge kernel of the wave-private decode: sequence b's
// partials are the slots b + i of the workgroups i that took its pages; a
// sequence whose pages one workgroup took was finished by the decode kernel.
struct WaveMergeArgs {
  const float* part_acc;
  const float* part_lse;
  const int32_t* seq_lens;
  float* out;                    // [B, Hq, 128]
  float* lse_out;                // [B, Hq] or null: log2-sum-exp2 of the sequence's scores (-inf: empty)
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_wg;
  int32_t max_len;
  float inv_v_scale_over_sqrt_d;
  uint32_t sign_bits[kHeadDim / 32];
};

// Arguments of the recent-window kernel of the hybrid decode
// (tq_hybrid.hip): one workgroup per (sequence, KV head, group of up to 8
// query heads) attends over the sequence's dense window rows and merges the
// result with the packed part's finished output by the two log2-sum-exp2s.
struct HybridArgs {
  const void* q;                 // [B, Hq, 128] of q_dtype
  const void* recent_k;          // [B, cap, Hkv, 128] of r_dtype
  const void* recent_v;
  const int32_t* recent_lens;    // [B], clamped to 0..cap
  const float* lse;              // [B, Hq] packed part's log2-sum-exp2 (-inf: no packed token)
  float* out;                    // [B, Hq, 128]: the packed part's output in, the merged output out
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t cap;
  int32_t q_dtype;
  int32_t r_dtype;
  int32_t causal_group;          // 0, or the query heads per KV head of one query token (causal chunk tail)
  float scale_log2;              // softmax scale * log2(e)
};

// Arguments of the multi-query (prefill / verify chunk) helpers
// (tq_prefill.hip).  The chunk's Lq queries of each sequence become Lq * G
// query heads per KV head of a decode over the prefix every query sees
// (tokens 0 .. P, P = seq_len - q_len), and the rest of the chunk
// (tokens P + 1 .. seq_len - 1, read back densely) is a causal window.
struct PrefillArgs {
  const void* q;                 // [B, Lq, Hq, 128] of q_dtype
  const int32_t* q_lens;         // [B], clamped to 0 .. min(Lq, seq_len)
  const int32_t* seq_lens;       // [B], clamped to 0 .. max_len
  const int32_t* block_table;    // [B, max_blocks_per_seq]
  void* vq;                      // [B, Hkv * Lq * G, 128] of q_dtype: query (j, i) of KV head g at g Lq G + j G + i
  int32_t* prefix_lens;          // [B] P + 1 (0 without queries)
  int32_t* tail_lens;            // [B] q_len - 1 (0 without queries)
  int64_t* tail_slots;           // [B, Lq - 1] flat slots of tokens P + 1 + r (-1 past the tail)
  const float* vout;             // [B, Hkv * Lq * G, 128]
  float* out;                    // [B, Lq, Hq, 128]
  int32_t batch;
  int32_t q_len;                 // Lq
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t block_size;
  int32_t max_len;
  int32_t q_dtype;
};

// Arguments of the split-merge + inverse-rotation kernel.
struct MergeArgs {
  const float* part_acc;
  const float* part_lse;
  const int32_t* seq_lens;
  float* out;                    // [B, Hq, 128]
  float* lse_out;                // [B, Hq] or null: log2-sum-exp2 of the sequence's scores (-inf: empty)
  int32_t batch;
  int32_t num_q_heads;
  int32_t pages_per_split;
  int32_t num_splits;
  int32_t max_len;               // as DecodeArgs::max_len
  float inv_v_scale_over_sqrt_d; // 1 / (v_scale * sqrt(128))
  uint32_t sign_bits[kHeadDim / 32];
};

hipError_t launch_write(const WriteArgs& a, int raw_dtype, int bits, hipStream_t stream);
// prod key rows of `bits` bits (2..5): indices at bits - 1, sketch signs, gamma
hipError_t launch_write_prod(const ProdWriteArgs& a, int raw_dtype, int bits, int num_cus, hipStream_t stream);
hipError_t launch_prod_scores(const ProdScoreArgs& a, int bits, hipStream_t stream);
// the new row of every sequence at its last token (AppendWriteArgs)
hipError_t launch_write_append(const AppendWriteArgs& a, int k_bits, int v_bits, hipStream_t stream);
// K and V rows of the same tokens (same num_rows) in one launch
hipError_t launch_write_pair(const WriteArgs& k, const WriteArgs& v, int raw_dtype, int k_bits, int v_bits,
                             hipStream_t stream);
hipError_t launch_decompress(const ReadArgs& a, int bits, int out_dtype, int num_cus, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int k_bits, int v_bits, hipStream_t stream);
int decode_table_bytes(int k_bits, int v_bits);  // LDS bytes of the decode lookup tables
int decode_merge_lds_bytes();                     // LDS bytes of the stream merge
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
// wave-private decode: nh = KV heads per wave (1, 2 or 4); wave_fits is
// false for any other nh and when the layout does not fit the CU's LDS
bool wave_fits(int k_bits, int v_bits, int nh, int num_kv_heads);
int wave_waves(int nh);                           // waves per workgroup (0: not built)
hipError_t launch_decode_wave(const WaveArgs& a, int k_bits, int v_bits, int nh, hipStream_t stream);
hipError_t launch_merge_wave(const WaveMergeArgs& a, hipStream_t stream);
hipError_t launch_hybrid(const HybridArgs& a, hipStream_t stream);
hipError_t launch_prefill_prep(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_out(const PrefillArgs& a, hipStream_t stream);

// the static scratch of tq_paged_decode_noalloc (tq_scratch.hip): its size, and
// its device address on the current device (looked up once per device; nullptr
// and *err set when the lookup fails)
size_t scratch_bytes();
void* scratch_device_ptr(hipError_t* err);

}  // namespace tq
