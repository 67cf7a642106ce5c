/*
 * tq.h -- C ABI of the TurboQuant packed-page KV library for AMD Instinct
 * MI355X (gfx950).
 *
 * The library writes K/V rows into uint8 pages in the TQ row format, reads
 * them back as dense rows, and runs single-query paged decode attention over
 * those pages, alone or together with an exact window of recent rows, and
 * multi-query (prefill / verify) attention over them.  Everything below is
 * plain C: device buffers are raw device pointers, streams are hipStream_t
 * passed as void*.  The library never allocates device memory inside
 * tq_write_kv / tq_paged_decode and never synchronises the stream; the caller
 * owns every buffer.
 *
 * Definitions this ABI implements (TurboQuant documentation pages):
 *
 *  - Row format ("vLLM Usage", section "TQ Byte Layout"): for one component
 *    (K or V), one token and one KV head, a row is
 *    index_bytes = ceil(head_dim * bits / 8) bytes of bit-packed codebook
 *    indices followed by the 4-byte fp32 norm of the raw row
 *    (row_bytes = index_bytes + 4; 36/52/68/84 bytes for 2/3/4/5 bits at
 *    head_dim 128).  K and V are stored independently with their own bits.
 *    Indices form one LSB-first bit stream: index i occupies stream bits
 *    [i*bits, (i+1)*bits), stream bit 8j+k is bit k of byte j.  The norm is
 *    little-endian.  No row or page padding.
 *  - Page tensor ("Architecture", section "Cache Storage Objects"):
 *    uint8 [num_blocks, block_size, num_kv_heads, row_bytes], one tensor per
 *    component, contiguous.
 *  - Flat slots ("vLLM Usage", section "Slot Mapping"): token n goes to page
 *    slot / block_size at offset slot % block_size; negative slots are
 *    ignored; a slot beyond the allocated pages is an error.
 *  - Codec ("vLLM Usage", "TQ Packed Page Contract"; "vLLM Reference Audit",
 *    Feature Checklist): a row x is encoded as n = ||x||_2 (float64 sum of
 *    squares, rounded once to fp32), u = x / n, r = H (s * u) / sqrt(d)
 *    (randomized Hadamard transform: seeded +-1 signs s, then the orthonormal
 *    Sylvester Hadamard matrix), and each r_i is replaced by the index of its
 *    nearest centroid of the 2^bits-level Lloyd-Max codebook of the exact
 *    coordinate law of a uniform unit vector in R^d.  The signs come from
 *    SplitMix64 seeded with the rotation seed (s_i = -1 when bit 63 of the
 *    i-th output is set).
 *  - Decode ("Architecture", section "Diagnostic vs Serving Paths"; "vLLM
 *    Usage", "Live Backend Gap"): one query token per sequence; query head h
 *    attends to KV head h / (num_q_heads / num_kv_heads) over tokens
 *    0..seq_lens[b]-1 found through block_table[b, t / block_size];
 *    out = softmax(scale * q . k_t) . v_t with k_t, v_t the reconstructed rows
 *    n * R^T c[idx].  A sequence of length 0 yields zeros.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tq_status {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = 1,  /* null pointer, bad size, inconsistent shapes */
  TQ_ERR_UNSUPPORTED = 2,  /* a valid request this build does not implement */
  TQ_ERR_ALIGNMENT = 3,    /* a pointer is not aligned as documented */
  TQ_ERR_WORKSPACE = 4,    /* workspace smaller than tq_decode_workspace_bytes */
  TQ_ERR_HIP = 5,          /* a HIP runtime call failed (see tq_last_hip_error) */
  TQ_ERR_NO_DEVICE = 6     /* no gfx950 device is current */
} tq_status;

typedef enum tq_dtype {
  TQ_F32 = 0,
  TQ_F16 = 1,
  TQ_BF16 = 2
} tq_dtype;

/* Opaque, immutable after creation; host memory only (no device state), so
 * one context may serve every device and concurrent calls. */
typedef struct tq_ctx tq_ctx;

/* Human-readable name of a status code (static string). */
const char* tq_status_string(tq_status status);

/* Last HIP error code seen by this thread (0 if none). */
int tq_last_hip_error(void);

/* Row size in bytes: ceil(head_dim * bits / 8) + 4.  Returns 0 when
 * head_dim <= 0 or bits is outside 1..8 ("vLLM Usage", "TQ Byte Layout"). */
size_t tq_row_bytes(int head_dim, int bits);

/* Host-only: the 2^bits fp32 centroids (increasing) and 2^bits - 1 fp32
 * boundaries (midpoints of neighbouring centroids, rounded to fp32) of the
 * Lloyd-Max codebook of the coordinate law f(x) ~ (1 - x^2)^((d-3)/2) on
 * [-1, 1] ("vLLM Reference Audit", File Map row "Lloyd-Max codebooks":
 * centroids and boundaries; Feature Checklist: exact Beta law).
 * centroids: 2^bits floats; boundaries: 2^bits - 1 floats or NULL.
 * head_dim in 3..4096, bits in 1..5.  Deterministic. */
tq_status tq_codebook(int head_dim, int bits, float* centroids, float* boundaries);

/* Host-only: the head_dim rotation signs (+1/-1) for a seed ("vLLM Usage",
 * "TQ Packed Page Contract": RHT rotation built from a seed). */
tq_status tq_rht_signs(uint64_t seed, int head_dim, int8_t* signs);

/* Create a context for one head dimension and rotation seed: computes the
 * signs and the codebooks for bits 1..5 on the host.  head_dim must be 128
 * (the only width the kernels are built for).  Does not touch the GPU. */
tq_status tq_ctx_create(int head_dim, uint64_t rht_seed, tq_ctx** out);
tq_status tq_ctx_destroy(tq_ctx* ctx);

/* Write rows into pages ("vLLM Usage", "Slot Mapping" and "TQ Packed Page
 * Contract", write_tq4_kv).  Arguments are validated first (no device needed);
 * TQ_ERR_NO_DEVICE when the current device is not a gfx950 (checked once per
 * device).
 *   raw       device, [num_tokens, num_kv_heads, head_dim] of raw_dtype,
 *             contiguous, 4-byte aligned (16-byte aligned for best speed).
 *   pages     device, uint8 [num_blocks, block_size, num_kv_heads,
 *             tq_row_bytes(head_dim, bits)], contiguous, 4-byte aligned.
 *   slots     device, int64 [num_tokens].  slot < 0: token skipped, pages
 *             untouched.  slot >= num_blocks * block_size: token skipped and
 *             counted in *err_count.
 *   bits      2..5.
 *   err_count device int32 or NULL; the kernel atomically ADDS the number of
 *             out-of-range slots (the caller zeroes it beforehand).
 *   stream    hipStream_t (NULL = default stream).
 * Asynchronous; the caller keeps every buffer alive until the stream has
 * executed the call.  Two tokens mapping to the same slot race (undefined
 * which one lands). */
tq_status tq_write_kv(const tq_ctx* ctx, const void* raw, tq_dtype raw_dtype,
                      int64_t num_tokens, int num_kv_heads, uint8_t* pages,
                      int64_t num_blocks, int block_size, const int64_t* slots,
                      int bits, int32_t* err_count, void* stream);

/* K and V rows of the same tokens in one launch (the same write as
 * tq_write_kv for K, then for V, with the same slots; "vLLM Usage", "Slot
 * Mapping" and "TQ Packed Page Contract").  raw_k / raw_v, k_pages / v_pages
 * and bits as in tq_write_kv per component; both page tensors have
 * num_blocks pages of block_size tokens.  An out-of-range slot is skipped by
 * both components and counted once in *err_count.  Asynchronous, allocates
 * nothing. */
tq_status tq_write_kv_pair(const tq_ctx* ctx, const void* raw_k, const void* raw_v,
                           tq_dtype raw_dtype, int64_t num_tokens, int num_kv_heads,
                           uint8_t* k_pages, int k_bits, uint8_t* v_pages, int v_bits,
                           int64_t num_blocks, int block_size, const int64_t* slots,
                           int32_t* err_count, void* stream);

/* Dense readback of stored rows: the diagnostic reconstruction of packed
 * bytes ("Architecture", section "Data Flow"; "vLLM Reference Audit", File
 * Map row "TQ4 unpack kernel": packed index bytes and norms in, rows out,
 * into a caller-given buffer).  The row of token n and KV head h is the TQ
 * row at flat slot slots[n] ("vLLM Usage", "Slot Mapping"), reconstructed
 * as x = n * s * (H c[idx]) / sqrt(head_dim): the fp32 centroids of its
 * indices, the inverse rotation, the stored norm.
 *   pages      device, uint8 [num_blocks, block_size, num_kv_heads,
 *              tq_row_bytes(head_dim, bits)], contiguous, 4-byte aligned.
 *   bits       2..5.
 *   slots      device, int64 [num_tokens], 8-byte aligned.  slot < 0: the
 *              token's rows are written as zeros.  slot >= num_blocks *
 *              block_size: zeros too, and counted in *err_count.
 *   out        device, [num_tokens, num_kv_heads, head_dim] of out_dtype
 *              (fp32, fp16 or bf16, rounded to nearest even), contiguous,
 *              16-byte aligned; every element is written.
 *   err_count  device int32 or NULL; the kernel atomically ADDS the number of
 *              out-of-range slots (the caller zeroes it beforehand).
 * num_tokens * num_kv_heads must stay below 2^31 (TQ_ERR_UNSUPPORTED).
 * Asynchronous, allocates nothing; TQ_ERR_NO_DEVICE when the current device
 * is not a gfx950. */
tq_status tq_decompress_kv(const tq_ctx* ctx, const uint8_t* pages, int64_t num_blocks, int block_size,
                           int num_kv_heads, int bits, const int64_t* slots, int64_t num_tokens,
                           void* out, tq_dtype out_dtype, int32_t* err_count, void* stream);

/* Inner-product ("prod") key rows: the published TurboQuant inner-product
 * quantiser, which the pages name ("vLLM Reference Audit", File Map row "MSE
 * and QJL codecs": TurboQuantProd, indices, norms, signs; Feature Checklist
 * row "QJL residual") without its arithmetic or layout.  A b-bit row encodes
 * the rotated unit vector r with the (b-1)-bit codec of the MSE rows, then
 * sketches its residual e = r - c[idx] with a d x d matrix S of N(0, 1)
 * entries: z_i = +1 when (S e)_i >= 0, and gamma = ||e||.  Layout (this
 * library's): ceil(d (b-1) / 8) index bytes, fp32 norm, d / 8 sign bytes
 * (bit i = z_i > 0, LSB-first), fp32 gamma; 40/56/72/88 bytes at d = 128
 * for b = 2..5.  Returns 0 for a head_dim not a multiple of 8 or bits
 * outside 2..8. */
size_t tq_prod_row_bytes(int head_dim, int bits);

/* Write prod key rows (as tq_write_kv: same raw rows, slots, page shape with
 * tq_prod_row_bytes rows, errors and err_count).  sketch: device fp32
 * [head_dim, head_dim] row-major, 16-byte aligned: the matrix S, an input
 * (the method's random draw).  gamma is computed in fp32 from the fp32
 * residual; the projection S e is formed from fp16 hi + lo parts of e and S
 * with fp32 accumulation (error about 2^-22 of sum_j |S_ij e_j|), so the sign
 * of a projection that close to zero may differ from an exact computation.
 * bits 2..5.  Asynchronous, allocates nothing. */
tq_status tq_write_kv_prod(const tq_ctx* ctx, const void* raw, tq_dtype raw_dtype,
                           int64_t num_tokens, int num_kv_heads, uint8_t* pages,
                           int64_t num_blocks, int block_size, const int64_t* slots,
                           int bits, const float* sketch, int32_t* err_count, void* stream);

/* Bytes of device workspace tq_prod_scores needs: two rows of 128 floats per
 * query head.  0 for a non-positive batch or head count. */
size_t tq_prod_scores_workspace_bytes(int batch, int num_q_heads);

/* Estimated inner products of every query head with every key of its
 * sequence over prod key pages (the score-only diagnostic the pages list as
 * the packed score kernel, "vLLM Reference Audit", File Map): for token t of
 * sequence b and query head h (KV head h / (num_q_heads / num_kv_heads)),
 * scores[b, h, t] = n (<q~, c[idx]> + gamma sqrt(pi / 2) / d <S q~, z>) with
 * q~ = rht(q): unbiased for <q, k> over the draw of S.
 *   q, block_table, seq_lens, max_seq_len: as tq_paged_decode.
 *   pages       device, prod rows [num_blocks, 16, num_kv_heads,
 *               tq_prod_row_bytes(head_dim, bits)], 4-byte aligned.
 *   sketch      the writer's S.
 *   scores      device, fp32 [batch, num_q_heads, max_seq_len]; entries past a
 *               sequence's length are written as 0.
 *   workspace   device, >= tq_prod_scores_workspace_bytes(...), 16-byte aligned.
 * Products of fp16 hi + lo parts with fp32 accumulation (about fp32
 * accuracy).  max_seq_len must stay below 2^26 (TQ_ERR_UNSUPPORTED).
 * Asynchronous, allocates nothing; errors as tq_paged_decode. */
tq_status tq_prod_scores(const tq_ctx* ctx, const void* q, tq_dtype q_dtype, int batch,
                         int num_q_heads, int num_kv_heads, const uint8_t* pages, int bits,
                         int64_t num_blocks, int block_size, const int32_t* block_table,
                         int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len,
                         const float* sketch, float* scores, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Bytes of device workspace tq_paged_decode needs for these sizes (the
 * split partials: a normalised rotated sum and a log-sum-exp per query head
 * and split).  The count of splits follows the current device's compute
 * units, so the value holds for the device current at this call; a workspace
 * sized on a device with fewer compute units can be too small on another, and
 * tq_paged_decode then returns TQ_ERR_WORKSPACE without launching anything.
 * ctx and block_size are not used (the size covers every bit width).
 * Returns 0 for a non-positive batch or head count or a negative length. */
size_t tq_decode_workspace_bytes(const tq_ctx* ctx, int batch, int num_q_heads,
                                 int num_kv_heads, int max_seq_len, int block_size);

/* Which decode kernel tq_paged_decode runs for these sizes on the current
 * device: "wave" (every wave owns all KV heads and walks its own pages;
 * 1, 2 or 4 KV heads with at most 8 query heads each), "wave1" (the same
 * kernel as one workgroup that finishes every sequence itself, with no merge
 * kernel: at most 32 pages in all and 64 sequences), "staged" (a workgroup
 * stages whole pages for all its waves), or NULL when the sizes are not
 * supported.  The environment variable TQ_DECODE_KERNEL=staged|wave
 * overrides the choice where the sizes allow it.  Host-only; static string. */
const char* tq_decode_kernel(int batch, int num_q_heads, int num_kv_heads,
                             int max_seq_len, int k_bits, int v_bits);

/* Single-query paged decode attention over TQ pages ("Architecture",
 * "Diagnostic vs Serving Paths": the paged decode reads packed pages and
 * reconstructs rows inside the loop; "vLLM Usage", decode_tq4_paged).
 *   q            device, [batch, num_q_heads, head_dim] of q_dtype, contiguous.
 *   k_pages      device, uint8 [num_blocks, block_size, num_kv_heads,
 *                tq_row_bytes(head_dim, k_bits)], 16-byte aligned.
 *   v_pages      same with v_bits.
 *   block_table  device, int32 [batch, max_blocks_per_seq]; entries for pages
 *                beyond a sequence's length are never read.
 *   seq_lens     device, int32 [batch], each in 0..max_seq_len (<= 0: zeros).
 *   max_seq_len  host upper bound of seq_lens (sizes the work split).
 *   scale        softmax scale; <= 0 selects 1/sqrt(head_dim).
 *   out          device, fp32 [batch, num_q_heads, head_dim].
 *   workspace    device, >= tq_decode_workspace_bytes(...) bytes, 16-byte
 *                aligned; contents are scratch.
 * Supported: head_dim 128, block_size 16, k_bits/v_bits 2..5,
 * num_q_heads / num_kv_heads in 1..64 (TQ_ERR_UNSUPPORTED otherwise, or when
 * a sequence is so long that its block ids do not fit the on-chip plan).
 * Asynchronous.  TQ_ERR_NO_DEVICE when the current device is not a gfx950
 * (checked after the arguments and the workspace size).  Device-side values
 * are bounded, never trusted: a block id
 * outside [0, num_blocks) reads as a page of zero rows (norm 0: score 0,
 * value 0), and a seq_lens entry above max_blocks_per_seq * block_size (or
 * above the pages the work split planned for max_seq_len) is clamped to it,
 * so no memory outside the given buffers is read. */
tq_status tq_paged_decode(const tq_ctx* ctx, const void* q, tq_dtype q_dtype,
                          int batch, int num_q_heads, int num_kv_heads,
                          const uint8_t* k_pages, int k_bits,
                          const uint8_t* v_pages, int v_bits,
                          int64_t num_blocks, int block_size,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int32_t* seq_lens, int max_seq_len, float scale,
                          float* out, void* workspace, size_t workspace_bytes,
                          void* stream);

/* One decode step in one call: the new token's K and V rows are written into
 * the pages and the decode attends over every token including it
 * ("Architecture", "Cache Lifecycle": a decoded token's KV joins the cache
 * before the next step attends; rows as in "vLLM Usage", "TQ Byte Layout").
 * For each sequence b with L_b = min(seq_lens[b], the decode's clamp) > 0,
 * k_new[b] and v_new[b] are encoded exactly as tq_write_kv encodes them and
 * stored at token L_b - 1, i.e. row (L_b - 1) % block_size of page
 * block_table[b, (L_b - 1) / block_size]; then the result is tq_paged_decode's
 * over tokens 0 .. L_b - 1.  Output and pages are bit for bit those of
 * tq_write_kv_pair at those slots followed by tq_paged_decode.  Where
 * tq_decode_kernel() names "staged", the decode kernel writes the rows itself
 * (the workgroup that reads the page stores them first), so a step is one
 * decode launch (plus the split merge) instead of a write launch and a decode
 * launch; for the wave kernels a writer launch that finds the slots on the
 * device from seq_lens and block_table runs first.
 *   q ... k_bits, v_pages ... workspace, workspace_bytes: as tq_paged_decode
 *     (k_pages and v_pages are written, at those rows only).
 *   k_new, v_new  device, [batch, num_kv_heads, head_dim] of new_dtype (fp32,
 *                 fp16 or bf16), contiguous, 4-byte aligned.
 *   err_count     device int32 or NULL: incremented once per sequence whose
 *                 last page's block id lies outside [0, num_blocks); that
 *                 sequence's rows are not written (and the page reads as
 *                 zero rows, as in tq_paged_decode).
 * Same support, errors and asynchrony as tq_paged_decode; the pages must not
 * be read or written by other work while the call runs. */
tq_status tq_paged_decode_append(const tq_ctx* ctx, const void* q, tq_dtype q_dtype,
                                 int batch, int num_q_heads, int num_kv_heads,
                                 const void* k_new, const void* v_new, tq_dtype new_dtype,
                                 uint8_t* k_pages, int k_bits,
                                 uint8_t* v_pages, int v_bits,
                                 int64_t num_blocks, int block_size,
                                 const int32_t* block_table, int max_blocks_per_seq,
                                 const int32_t* seq_lens, int max_seq_len, float scale,
                                 float* out, void* workspace, size_t workspace_bytes,
                                 int32_t* err_count, void* stream);

/* Bytes of device workspace tq_paged_decode_hybrid needs: the decode's
 * workspace (rounded up to 256 bytes) plus one float per query head for the
 * packed part's log-sum-exp.  Same arguments, rules and device dependence as
 * tq_decode_workspace_bytes; 0 where that returns 0. */
size_t tq_hybrid_workspace_bytes(const tq_ctx* ctx, int batch, int num_q_heads,
                                 int num_kv_heads, int max_seq_len, int block_size);

/* Decode over packed history plus an exact recent window ("Integration API",
 * vLLM hooks, hybrid mode: compressed history plus exact recent tokens for
 * decode; "Architecture", "Cache Lifecycle": decoded tokens are appended to a
 * recent window before they are flushed to packed pages).  Sequence b attends
 * with one softmax over its seq_lens[b] packed tokens (exactly as
 * tq_paged_decode) and the first recent_lens[b] rows of its window, which
 * hold tokens the pages do not; the order of the window rows does not
 * matter.  A sequence with no token at all yields zeros.
 *   q ... max_seq_len, scale, out: as tq_paged_decode.
 *   recent_k, recent_v  device, [batch, recent_cap, num_kv_heads, head_dim]
 *                       of recent_dtype (fp32, fp16 or bf16, used exactly as
 *                       given), contiguous, 16-byte aligned; rows past a
 *                       sequence's recent length are never read.  May be NULL
 *                       when recent_cap is 0 (then this is tq_paged_decode).
 *   recent_lens         device, int32 [batch]; each entry is clamped to
 *                       0..recent_cap.
 *   workspace           device, >= tq_hybrid_workspace_bytes(...) bytes,
 *                       16-byte aligned; contents are scratch.
 * Runs the decode (which also leaves each query head's log-sum-exp in the
 * workspace) and then one small kernel that attends over the window and
 * merges both parts into out.  Asynchronous, allocates nothing; errors as
 * tq_paged_decode (TQ_ERR_WORKSPACE, before any launch, for a workspace
 * below tq_hybrid_workspace_bytes). */
tq_status tq_paged_decode_hybrid(const tq_ctx* ctx, const void* q, tq_dtype q_dtype,
                                 int batch, int num_q_heads, int num_kv_heads,
                                 const uint8_t* k_pages, int k_bits,
                                 const uint8_t* v_pages, int v_bits,
                                 int64_t num_blocks, int block_size,
                                 const int32_t* block_table, int max_blocks_per_seq,
                                 const int32_t* seq_lens, int max_seq_len,
                                 const void* recent_k, const void* recent_v, tq_dtype recent_dtype,
                                 int recent_cap, const int32_t* recent_lens, float scale,
                                 float* out, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Bytes of device workspace tq_paged_prefill needs for these sizes (sized
 * for fp32 queries, enough for every query dtype).  The count of splits of
 * its decode follows the current device's compute units, as in
 * tq_decode_workspace_bytes.  0 for a non-positive batch, q_len or head
 * count or a negative length. */
size_t tq_prefill_workspace_bytes(const tq_ctx* ctx, int batch, int q_len, int num_q_heads,
                                  int num_kv_heads, int max_seq_len, int block_size);

/* Several query tokens per sequence over the packed pages, causal within the
 * chunk ("vLLM Usage", "Runtime Dispatch": with a cache present, mixed
 * prefill / decode batches attend through the packed cache): chunked
 * prefill, speculative verification, mixed batches.  The queries of
 * sequence b are those of its last q_lens[b] tokens, whose K/V rows are
 * already written to the pages; query j sits at position
 * P + j, P = seq_lens[b] - q_lens[b], and attends tokens 0 .. P + j.
 *   q           device, [batch, q_len, num_q_heads, head_dim] of q_dtype,
 *               contiguous, 16-byte aligned; rows j >= q_lens[b] are ignored.
 *   q_lens      device, int32 [batch], each clamped to 0 .. min(q_len,
 *               seq_lens[b]).
 *   out         device, fp32 [batch, q_len, num_q_heads, head_dim],
 *               16-byte aligned; rows j >= q_lens[b] are written as zeros.
 *   workspace   device, >= tq_prefill_workspace_bytes(...) bytes, 256-byte
 *               aligned; contents are scratch.
 *   the rest    as tq_paged_decode.
 * (num_q_heads / num_kv_heads) * q_len must be at most 64
 * (TQ_ERR_UNSUPPORTED otherwise).  The prefix 0 .. P is read once for all of
 * a sequence's queries: they are decoded together as q_len times as many
 * query heads; the chunk's other tokens are read back densely and attended
 * causally, and the two parts are merged by their log-sum-exps.
 * Asynchronous, allocates nothing; errors as tq_paged_decode. */
tq_status tq_paged_prefill(const tq_ctx* ctx, const void* q, tq_dtype q_dtype, int batch, int q_len,
                           const int32_t* q_lens, int num_q_heads, int num_kv_heads,
                           const uint8_t* k_pages, int k_bits, const uint8_t* v_pages, int v_bits,
                           int64_t num_blocks, int block_size,
                           const int32_t* block_table, int max_blocks_per_seq,
                           const int32_t* seq_lens, int max_seq_len, float scale,
                           float* out, void* workspace, size_t workspace_bytes, void* stream);

/* tq_paged_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same decode, arguments and results, with the split partials kept in a
 * static scratch array of the library instead of a caller workspace.  Every
 * GPU the library runs on holds its own 32 MiB copy of that array from module
 * load until the process ends; the first call on a device looks its address
 * up.  TQ_ERR_WORKSPACE, before any launch, when the sizes need more than
 * 32 MiB (tq_decode_workspace_bytes > 32 MiB).  Calls that overlap on one GPU
 * share the array and race; the caller orders them on one stream.  Nothing is
 * allocated; asynchronous. */
tq_status tq_paged_decode_noalloc(const tq_ctx* ctx, const void* q, tq_dtype q_dtype,
                                  int batch, int num_q_heads, int num_kv_heads,
                                  const uint8_t* k_pages, int k_bits,
                                  const uint8_t* v_pages, int v_bits,
                                  int64_t num_blocks, int block_size,
                                  const int32_t* block_table, int max_blocks_per_seq,
                                  const int32_t* seq_lens, int max_seq_len, float scale,
                                  float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
