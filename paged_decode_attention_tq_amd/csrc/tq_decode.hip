// Single-query paged decode over TQ pages for gfx950: the split kernel and
// the merge + inverse-rotation kernel.
//
// The decode reads packed pages through the block table and rebuilds rows
// inside its loop (TurboQuant docs, "Architecture", section "Diagnostic vs
// Serving Paths"; pages as in "Cache Storage Objects"; rows as in "vLLM
// Usage", section "TQ Byte Layout").  It never materialises a row: R is
// orthogonal, so q . (n R^T c) = n (R q) . c and
// sum_t p_t n_t R^T c_t = R^T sum_t p_t n_t c_t; scores and the value sum are
// formed on the rotated codes and rotated back once per head by the merge.
//
// Split kernel, per 16-token page and KV head (one wave):
//  scores  S[t][h] = q~_h . c_K[idx_K[t]] with v_mfma_f32_16x16x32_f16:
//          A = dequantised keys (16 tokens x 32 dims), B = rotated queries
//          (32 dims x 16 columns).  Keys are split into fp16 hi + lo and so
//          are queries; with G <= 8 the B columns hold [q_hi | q_lo] and one
//          pair of MFMAs (K_hi, K_lo) gives (K_hi + K_lo) . (q_hi + q_lo) as
//          column h plus column h + 8.
//  softmax log2 domain; the running reference is the maximum over tokens of
//          score + e_t, e_t the binary exponent of the value norm, so the
//          weights w = p * n_v stay below 2^9 and fit fp16; the reference is
//          raised lazily, only when the page maximum exceeds it by 8.
//  values  acc[dim][h] += sum_t V^[t][dim] w[t][h] with
//          v_mfma_f32_16x16x32_f16: A = dequantised value pairs (16 dim
//          pairs x (16 tokens x 2 parities)), B = the weights w_hi, then in a
//          second MFMA w_lo, each placed in the column half of its dim parity
//          (columns h: even dims, h + 8: odd dims).
// Lane layout (l = lane, n = l & 15, c = l >> 4):
//  K reads  token n, dims 32c..32c+31 (4*KB contiguous bytes of its row);
//  V reads  tokens 4c..4c+3, dims 8n..8n+7 (VB bits per dim of each row);
//  scores   tokens 4c+r (r = 0..3), column n;
//  acc      column n, dims 32c + 8r + 2 blk + (n >> 3) (blk = 0..3).
// Dequantisation reads LDS pair tables: row p = i0 | i1 << b holds the fp16
// pair (c[i0], c[i1]) and the fp16 pair of its rounding residuals (8 bytes),
// replicated once per lane of a half-wave (bank-conflict free); keys read
// both halves, values only the pair (the upper half of the replicas stores
// the two dwords swapped, so that a half-wave's value reads also hit
// distinct banks).

#include "tq_decode_common.h"
#include "tq_encode.h"

#include <type_traits>
#include <utility>

namespace tq {

#ifndef TQ_WG_WAVES
#define TQ_WG_WAVES 16
#endif
constexpr int kMaxWaves = TQ_WG_WAVES;   // waves per workgroup (one workgroup per CU)
constexpr int kWgThreads = 64 * kMaxWaves;

// CONTIG: the workgroup holds every KV head, so a page is staged as the
// contiguous bytes it is; else per-token chunk windows over the slice of the
// workgroup's heads.  MAXLD: 1 KB loads per wave per stage.

template <int KB, int VB, bool CONTIG, int MAXLD, bool APP>
__global__ __launch_bounds__(kWgThreads) void decode_split_kernel(DecodeArgs a) {
  // all of the CU's LDS, statically: addresses are then known constants
  __shared__ __attribute__((aligned(16))) uint8_t lds[kDecodeLdsBytes];
  using KT = PairTable<KB>;
  using VT = PairTable<VB>;
  constexpr bool kShareV = (KB == VB);
  // run a page's value part one iteration after its key part (registers allow
  // it with whole-page staging and at most three copies per wave and stage)
  constexpr bool kSplit = CONTIG && MAXLD == 3;
  // LDS: lookup tables at 0 (so their addresses need no base), then two
  // stage slots, then the split's block ids
  constexpr int kVTab = 0;
  constexpr int kKTab = kShareV ? 0 : VT::kBytes;
  constexpr int kStages = kKTab + KT::kBytes;

  const int S = a.num_splits;
  const int unit = __builtin_amdgcn_workgroup_id_x();
  const int tid = __builtin_amdgcn_workitem_id_x();
  // split-major order: every sequence's first split is dispatched before any
  // second split, so in a ragged batch the short tails of long sequences come
  // last and the CUs finish close together
  const int bh = unit % (a.batch * a.head_groups);
  const int s = unit / (a.batch * a.head_groups);
  const int hg = bh % a.head_groups;
  const int b = bh / a.head_groups;
  const int L = __builtin_amdgcn_readfirstlane(min(a.seq_lens[b], a.max_len));
  const int npages = (L + kBlockSize - 1) / kBlockSize;
  const int p0 = s * a.pages_per_split;
  if (p0 >= npages) return;  // the whole workgroup leaves together
  const int span = min(a.pages_per_split, npages - p0);

  // ---- appending decode: the new row of the sequence ------------------------------
  // The workgroup holding the sequence's last page (the last split; one per
  // group of KV heads) encodes its heads' K and V rows of the last token as
  // the row writer does and stores them into that page, first thing, while
  // few registers are live.  The prologue barrier orders the stores before
  // every page copy of the workgroup, and no other workgroup reads the page.
  // Quad r < 2 kv_per_wg (kv_per_wg <= waves, 16 quads each) takes component
  // r / kv_per_wg of head kv_per_wg hg + r % kv_per_wg.
  if (APP && s == (npages - 1) / a.pages_per_split) {
    const int tid0 = __builtin_amdgcn_workitem_id_x();
    const int blk = __builtin_amdgcn_readfirstlane(a.block_table[(int64_t)b * a.max_blocks_per_seq + (L - 1) / kBlockSize]);
    const bool ok = blk >= 0 && (int64_t)blk < a.num_blocks;
    const int r = tid0 >> 2;
    if (ok && r < 2 * a.kv_per_wg) {
      const int comp = r / a.kv_per_wg;
      const int head = a.kv_per_wg * hg + (r - comp * a.kv_per_wg);
      const int64_t elem = ((int64_t)b * a.num_kv_heads + head) * kHeadDim;
      const int64_t tok_row = (int64_t)((L - 1) % kBlockSize) * a.num_kv_heads + head;
      if (comp == 0)
        load_encode_store_row<KB>(a.app.k_new, a.app.new_dtype, elem, tid0 & 3, a.sign_bits, a.app.k_bounds,
                                  const_cast<uint8_t*>(a.k_pages) + (int64_t)blk * a.k_page_bytes + tok_row * a.k_row_bytes,
                                  a.k_row_bytes);
      else
        load_encode_store_row<VB>(a.app.v_new, a.app.new_dtype, elem, tid0 & 3, a.sign_bits, a.app.v_bounds,
                                  const_cast<uint8_t*>(a.v_pages) + (int64_t)blk * a.v_page_bytes + tok_row * a.v_row_bytes,
                                  a.v_row_bytes);
    }
    if (!ok && tid0 == 0 && hg == 0 && a.app.err_count) atomicAdd(a.app.err_count, 1);
  }

  // the wave index is uniform; say so, so that everything derived from it
  // (head, page stream, load assignment) lives in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int W = a.waves;
  const int hpw = a.kv_per_wg * a.q_groups;    // waves per page
  const int st = wave / hpw;                   // page stream
  const int hs = wave - st * hpw;
  const int kvl = hs / a.q_groups;
  const int qgi = hs - kvl * a.q_groups;
  const int g0 = hg * a.kv_per_wg;
  const int g = g0 + kvl;                      // KV head
  const int qh0 = g * a.group + qgi * 8;
  const int gsz = min(8, a.group - qgi * 8);   // query heads of this wave
  const int n = lane & 15;
  const int c = lane >> 4;
  const int hq = n & 7;                        // query head (within the wave's group) of column n
  const int par = n >> 3;                      // column half: q_lo / odd value dims
  const int strm = a.streams;
  const int32_t* bt_lds = reinterpret_cast<const int32_t*>(lds + a.bt_base);

  // ---- staging geometry --------------------------------------------------------
  // A stage is strm consecutive pages (one per stream) of the workgroup's
  // heads; two stage slots alternate.  A page slot holds the K part, then the
  // V part.  CONTIG: each row (token t, head g) gets a slice of H = 16 hs
  // bytes at t * 16 tc + g * H, where hs = ceil(RB / 16) and tc (odd) is
  // the 16-byte chunks per token: slices start 16-byte aligned and token
  // rows start on different bank groups, so the lanes of a wave (one token
  // each) read their rows without bank conflicts.  A slice holds the row's
  // bytes 0 .. H - 17 in place and its last 16 bytes (ending with the norm)
  // in its last chunk, so the norm sits at H - 4.  Else the slice of the workgroup's heads
  // for token t (kv_per_wg * RB bytes) is staged as the C 16-byte chunks of a
  // window that covers it and starts delta_t (at most 31) bytes before it:
  // token t at t * 16C + delta_t.
  const int k_rows = (int)a.k_page_bytes, v_rows = (int)a.v_page_bytes;
  const int kC = a.k_tok_chunks, vC = a.v_tok_chunks;
  auto window = [&](int t, int RB, int C, int page_bytes, int& delta) {
    const int row = (t * a.num_kv_heads + g0) * RB;
    int w = row & ~15;
    if (w + 16 * C > page_bytes) w = page_bytes - 16 * C;
    delta = row - w;
    return w;
  };
  // Load x of a stage (0 <= x < strm * (nk + nv)) is 64 chunks of page
  // x / (nk + nv): K chunks 64 r .. 64 r + 63 for r = x % (nk + nv) < nk,
  // else V.  Wave w issues loads w, w + W, ... (at most MAXLD).
  const int nk = a.k_loads, nkv = a.k_loads + a.v_loads;
  const int n_ld = strm * nkv > wave ? (strm * nkv - wave + W - 1) / W : 0;
  auto load_src = [&](int d) -> uint32_t {  // lane's source offset inside the page
    const int x = wave + d * W;
    const int r = x % nkv;
    const bool isv = r >= nk;
    const int ri = isv ? r - nk : r;
    if constexpr (CONTIG) {
      const int tc = isv ? vC : kC, hs = isv ? a.v_slice_chunks : a.k_slice_chunks;
      const int RB = isv ? a.v_row_bytes : a.k_row_bytes;
      const int q = ri * 64 + lane;  // the LDS chunk this lane fills
      const int t = q / tc;
      const int rem = q - t * tc;
      const int gg = min(rem / hs, a.num_kv_heads - 1);  // (padding chunks: any row, not stored)
      const int j = rem - (rem / hs) * hs;
      return (uint32_t)((t * a.num_kv_heads + gg) * RB + (j == hs - 1 ? RB - 16 : 16 * j));
    } else {
      const int C = isv ? vC : kC;
      const int ch = min(ri * 64 + lane, kBlockSize * C - 1);
      const int t = ch / C;
      int dl;
      return (uint32_t)(window(t, isv ? a.v_row_bytes : a.k_row_bytes, C, isv ? v_rows : k_rows, dl) + 16 * (ch - t * C));
    }
  };
  auto lane_loads = [&](int d) {  // this lane carries a chunk of load d
    const int x = wave + d * W;
    const int r = x % nkv;
    const bool isv = r >= nk;
    const int ri = isv ? r - nk : r;
    const int q = ri * 64 + lane;
    if (q >= (isv ? a.v_chunks : a.k_chunks)) return false;
    if constexpr (CONTIG) {  // not a token row's padding chunk
      const int tc = isv ? vC : kC;
      return q - (q / tc) * tc < a.num_kv_heads * (isv ? a.v_slice_chunks : a.k_slice_chunks);
    }
    return true;
  };
  // Everything about a wave's loads but the block id is fixed for the whole
  // walk: work it out once, in scalar registers that the compiler cannot
  // re-derive from the kernel arguments inside the loop.
  auto opaque = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  int ld_j[MAXLD], ld_pb[MAXLD], ld_soff[MAXLD], ld_dst[MAXLD];
  uint32_t ld_lo[MAXLD], ld_hi[MAXLD];  // page pool base, as two scalar halves
  uint32_t ld_voff[MAXLD];              // per-lane part of the source offset
  bool ld_ok[MAXLD];                    // this lane carries a chunk
#pragma unroll
  for (int d = 0; d < MAXLD; ++d) {
    const int x = wave + d * W;
    const int r = x % nkv;
    const bool isv = r >= nk;
    const int ri = isv ? r - nk : r;
    const uint8_t* pool = isv ? a.v_pages : a.k_pages;
    ld_j[d] = opaque(x / nkv);
    ld_pb[d] = opaque(isv ? v_rows : k_rows);
    ld_lo[d] = (uint32_t)opaque((int)(uint32_t)(uintptr_t)pool);
    ld_hi[d] = (uint32_t)opaque((int)(uint32_t)((uintptr_t)pool >> 32));
    ld_soff[d] = 0;
    ld_voff[d] = load_src(d);
    ld_dst[d] = opaque(kStages + (x / nkv) * a.page_slot_bytes + (isv ? a.k_region : 0) + ri * 1024);
    ld_ok[d] = d < n_ld && lane_loads(d);
  }
  const int stage_bytes = opaque(a.stage_bytes);
  // stage si straight into LDS slot `slot` (no registers): the destination
  // slot must be free when this is issued, and the data is there once this
  // wave has waited for its vector memory counter and the workgroup has met
  // at a barrier
  auto issue_dma = [&](int si, int slot) {
    // the block ids first: their LDS reads are in flight together, and one
    // wait covers them all (read per copy, each would wait on its own)
    int blk_ids[MAXLD];
#pragma unroll
    for (int d = 0; d < MAXLD; ++d) blk_ids[d] = bt_lds[min(si * strm + ld_j[d], span - 1)];
#pragma unroll
    for (int d = 0; d < MAXLD; ++d) blk_ids[d] = __builtin_amdgcn_readfirstlane(blk_ids[d]);
#pragma unroll
    for (int d = 0; d < MAXLD; ++d) {
      const int P = si * strm + ld_j[d];
      if (d < n_ld && P < span) {
        const int blk = blk_ids[d];  // -1: out of range
        const uint64_t pool = ((uint64_t)ld_hi[d] << 32) | ld_lo[d];
        const uint64_t base = pool + (uint64_t)((int64_t)max(blk, 0) * ld_pb[d]);
        i32x4 rs;
        rs.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)base);
        rs.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(base >> 32) & 0xFFFFu));
        rs.z = blk < 0 ? 0 : ld_pb[d];  // a zero-sized buffer reads zeros
        rs.w = 0x00020000;
        const uint32_t dst = (uint32_t)__builtin_amdgcn_readfirstlane((int)(ld_dst[d] + slot * stage_bytes));
        if (ld_ok[d]) copy_chunk_to_lds(rs, dst, ld_voff[d], ld_soff[d]);
      }
    }
  };


  // ---- rotated, scaled query as the B operand of the score MFMAs ----------
  // Lane (n, c) covers dims 32c..32c+31 (16 pairs); column n < 8 holds the
  // fp16 hi part of head n, column n + 8 its lo part.  MFMA m takes pairs
  // 2m and 2m+1, each twice (the A operand interleaves K hi and K lo).
  uint32_t qd[16];   // dword = fp16 pair (dims 2p, 2p+1) of this lane's column
  float q_unscale;   // scores come out multiplied by 1 / q_unscale (one power of two per wave)
  {
    const bool has = hq < gsz;
    const int64_t qoff = ((int64_t)b * a.num_q_heads + qh0 + (has ? hq : 0)) * kHeadDim + 32 * c;
    float x[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) x[j] = load_q(a.q, qoff + j, a.q_dtype);
#pragma unroll
    for (int j = 0; j < 32; ++j) x[j] = has ? x[j] : 0.0f;
    const uint32_t sw = pick4(a.sign_bits, c);
#pragma unroll
    for (int j = 0; j < 32; ++j) x[j] = __uint_as_float(__float_as_uint(x[j]) ^ (((sw >> j) & 1u) << 31));
#pragma unroll
    for (int h = 1; h < 32; h <<= 1)
#pragma unroll
      for (int j = 0; j < 32; ++j)
        if ((j & h) == 0) {
          const float u = x[j], v = x[j + h];
          x[j] = u + v;
          x[j + h] = u - v;
        }
#pragma unroll
    for (int j = 0; j < 32; ++j) x[j] = lane_bfly<16>(x[j], lane);
#pragma unroll
    for (int j = 0; j < 32; ++j) x[j] = lane_bfly<32>(x[j], lane);
    // power-of-two scale that puts the wave's largest coordinate near 2^10,
    // so the fp16 hi/lo halves keep their precision for any query magnitude
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, __builtin_fabsf(x[j] * a.q_scale));
    // one power of two for the whole wave (all its heads), so that it can
    // be folded into the key norms
    amax = max_across_rows(amax);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    amax = __builtin_amdgcn_readfirstlane(__float_as_int(amax)) == 0 ? 0.0f
                                                                  : __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(amax)));
    int qe = 0;
    (void)__builtin_frexpf(amax, &qe);
    if (!(amax > 0.0f) || !(amax < __builtin_inff())) qe = 11;
    const float up = __builtin_ldexpf(a.q_scale, 11 - qe);
    q_unscale = __builtin_ldexpf(1.0f, qe - 11);
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      _Float16 h2[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float v = x[2 * p + e] * up;
        const _Float16 hi = (_Float16)v;
        h2[e] = par ? (_Float16)(v - (float)hi) : hi;
      }
      qd[p] = pack_half2(h2[0], h2[1]);
    }
  }

  // the score MFMAs' B operands (each dword of qd twice), built once so
  // that the page loop spends no register copies on them
  half8 Bqs[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) Bqs[m] = __builtin_bit_cast(half8, u32x4{qd[2 * m], qd[2 * m], qd[2 * m + 1], qd[2 * m + 1]});

  // ---- lookup tables and block ids -------------------------------------------
  fill_pair_table<KB>(lds + kKTab, a.k_cent, tid, 64 * W);
  if constexpr (!kShareV) fill_pair_table<VB>(lds + kVTab, a.v_cent, tid, 64 * W);
  {
    const int32_t* bt = a.block_table + (int64_t)b * a.max_blocks_per_seq + p0;
    int32_t* dst = reinterpret_cast<int32_t*>(lds + a.bt_base);
    for (int i = tid; i < span; i += 64 * W) {
      const int v = bt[i];
      dst[i] = (v >= 0 && (int64_t)v < a.num_blocks) ? v : -1;
    }
  }
  __syncthreads();

  // ---- per-lane LDS offsets inside a page slot ------------------------------------
  auto tok_k = [&](int t) {
    if constexpr (CONTIG) {
      return 16 * (t * kC + g * a.k_slice_chunks);
    } else {
      int d;
      (void)window(t, a.k_row_bytes, kC, k_rows, d);
      return t * 16 * kC + d + kvl * a.k_row_bytes;
    }
  };
  auto tok_v = [&](int t) {
    if constexpr (CONTIG) {
      return a.k_region + 16 * (t * vC + g * a.v_slice_chunks);
    } else {
      int d;
      (void)window(t, a.v_row_bytes, vC, v_rows, d);
      return a.k_region + t * 16 * vC + d + kvl * a.v_row_bytes;
    }
  };
  const int v_byte = n * VB;
  const int v_dat = (VB == 3 || VB == 5) ? (v_byte & ~3) : (v_byte & ~1);
  const uint32_t k_idx_off = (uint32_t)(kStages + tok_k(n) + 4 * KB * c);
  // each lane reads the norms of token 4c + (n & 3); quad broadcasts hand
  // every lane those of tokens 4c .. 4c + 3
  const int k_norm_at = CONTIG ? 16 * a.k_slice_chunks - 4 : a.k_row_bytes - 4;
  const int v_norm_at = CONTIG ? 16 * a.v_slice_chunks - 4 : a.v_row_bytes - 4;
  const uint32_t k_norm_off = (uint32_t)(kStages + tok_k(4 * c + (n & 3)) + k_norm_at);
  const uint32_t v_norm_off = (uint32_t)(kStages + tok_v(4 * c + (n & 3)) + v_norm_at);
  // value bytes of token 4c + r: CONTIG: base + r * token stride
  const int v_tstride = 16 * vC;
  uint32_t v_dat_off[CONTIG ? 1 : 4];
#pragma unroll
  for (int r = 0; r < (CONTIG ? 1 : 4); ++r) v_dat_off[r] = (uint32_t)(kStages + tok_v(4 * c + r) + v_dat);
  auto v_dat_at = [&](int r) -> uint32_t {
    if constexpr (CONTIG) return v_dat_off[0] + (uint32_t)(r * v_tstride);
    else return v_dat_off[r];
  };
  const uint32_t v_shift = 8u * (uint32_t)(v_byte & 3);
  const uint32_t k_lane = (uint32_t)(lane & (KT::kRep - 1)) * 8u;
  // the hi dword of this lane's replica
  const uint32_t v_lane = (uint32_t)(lane & (VT::kRep - 1)) * 8u + (((lane & (VT::kRep - 1)) >= VT::kRep / 2) ? 4u : 0u);
  const uint8_t* k_tab = lds + kKTab;
  const uint8_t* v_tab = lds + kVTab;
  const uint32_t w_shift = 16u * (uint32_t)par;  // weight half: even dims in columns < 8

  // acc[blk][r]: column n (head hq), dim 32c + 8r + 2blk + par
  floatx4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -__builtin_inff();
  float l_part = 0.0f;

  // ---- one wave's page, in two parts ---------------------------------------------
  // Key part: the key indices and table lookups (LDS), the score MFMAs, and
  // the page's value index words and norms, all left in registers.  Value
  // part: value table lookups, softmax, value MFMAs.  The stage loop runs a
  // page's value part one iteration after its key part (when registers allow
  // it), which frees the page's stage slot a whole iteration early.
  constexpr int kVW = (VB == 3 || VB == 5) ? 2 : 1;  // value index words per token row slice
  struct PagePart {
    floatx4 sc;          // raw scores (fp16 hi and lo columns not yet summed)
    uint32_t vw[kVW][4]; // value index words of tokens 4c .. 4c + 3
    float nk, nv;        // the norms of token 4c + (n & 3)
  };
  auto key_part = [&](uint32_t pg, PagePart& o) {
    // pg: byte offset of the page slot inside the stage area
    uint32_t kw[KB];
    if constexpr (CONTIG && KB == 4) {  // 16-byte aligned: one read
      const u32x4 w4 = *reinterpret_cast<const u32x4*>(lds + pg + k_idx_off);
#pragma unroll
      for (int i = 0; i < 4; ++i) kw[i] = w4[i];
    } else {
#pragma unroll
      for (int i = 0; i < KB; ++i) kw[i] = lds_u32(lds, pg + k_idx_off + 4 * i);
    }
    o.nk = __uint_as_float(lds_u32(lds, pg + k_norm_off));
    uint32_t kh[16], kl[16];
    auto klook = [&](int k) {
      const u32x2 e = *reinterpret_cast<const u32x2*>(k_tab + pair_addr<KB>(kw, k, k_lane));
      kh[k] = e[0];
      kl[k] = e[1];
    };
    // A = [K_hi(p), K_lo(p), K_hi(p'), K_lo(p')], B = [q(p), q(p), q(p'), q(p')]
    floatx4 sc = floatx4{0.f, 0.f, 0.f, 0.f};
    auto kmfma = [&](int m) {
      const half8 A = __builtin_bit_cast(half8, u32x4{kh[2 * m], kl[2 * m], kh[2 * m + 1], kl[2 * m + 1]});
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bqs[m], sc, 0, 0, 0);
    };
    // rolling window: the lookups of the next two MFMAs are in flight while
    // one runs, which keeps few lookup results live at a time
    constexpr int kWin = 2;
#pragma unroll
    for (int k = 0; k < 2 * kWin; ++k) klook(k);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (m + kWin < 8) {
        klook(2 * (m + kWin));
        klook(2 * (m + kWin) + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      kmfma(m);
    }
    o.sc = sc;
    // value norms and index words: the slot is rewritten before the value part runs
    o.nv = __uint_as_float(lds_u32(lds, pg + v_norm_off));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t vo = pg + v_dat_at(r);
      if constexpr (VB == 2) {
        o.vw[0][r] = *reinterpret_cast<const uint16_t*>(lds + vo);
      } else {
        o.vw[0][r] = lds_u32(lds, vo);
        if constexpr (kVW == 2) o.vw[kVW - 1][r] = lds_u32(lds, vo + 4);
      }
    }
  };
  auto value_part = [&](const PagePart& o, int tok0, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    // -- value lookups: dword (V[t][2p], V[t][2p+1]) for pair p = 4n + blk of
    // token 4c + j is exactly A[row n][k = 2j, 2j+1] of value block blk
    uint32_t va[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t words[2];
      if constexpr (kVW == 2) {
        const uint64_t all = ((((uint64_t)o.vw[kVW - 1][j]) << 32) | o.vw[0][j]) >> v_shift;
        words[0] = (uint32_t)all;
        words[1] = (uint32_t)(all >> 32);
      } else {
        words[0] = o.vw[0][j];
        words[1] = 0;
      }
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) va[blk][j] = lds_u32(v_tab, pair_addr<VB>(words, blk, v_lane));
    }
    // -- softmax bookkeeping (log2 domain).  e = an upper bound of log2(n_v)
    // from the exponent bits (clamped so empty rows cannot blow up p).  The
    // per-token factors are formed on the lane that read the norm and
    // broadcast inside each quad (lane (n, c) needs tokens 4c .. 4c + 3).
    const float nkq_mine = o.nk * q_unscale;
    const float e_mine = fmaxf(__builtin_fmaf((float)(__float_as_uint(o.nv) >> 24), 2.0f, -126.0f), -64.0f);
    float full[4], xv[4];
    {
      // (no contraction here: a plain multiply and add each take their
      // broadcast operand straight from the neighbouring lane)
#pragma clang fp contract(off)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        full[r] = (o.sc[r] + row_ror8(o.sc[r])) * quad_bcast_r(nkq_mine, r);
        xv[r] = full[r] + quad_bcast_r(e_mine, r);
        if constexpr (!FULL) xv[r] = (tok0 + r < L) ? xv[r] : -__builtin_inff();
      }
    }
    float pmax = fmaxf(fmaxf(xv[0], xv[1]), fmaxf(xv[2], xv[3]));
    pmax = max_across_rows(pmax);
    if (__builtin_amdgcn_ballot_w64(pmax > m_ref + 8.0f) != 0) {
      const float m_new = fmaxf(m_ref, pmax);
      const float alpha = (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] *= alpha;
      m_ref = m_new;
    }
    // -- weights w = p * n_v as fp16 hi + lo, placed in this column's half
    uint32_t whi[4], wlo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float pr = __builtin_amdgcn_exp2f(full[r] - m_ref);
      if constexpr (!FULL) pr = (tok0 + r < L) ? pr : 0.0f;
      l_part += pr;
      float wv = pr * quad_bcast_r(o.nv, r);
      if constexpr (!FULL) wv = (tok0 + r < L) ? wv : 0.0f;  // rows past the end may hold anything
      const _Float16 hi = (_Float16)wv;
      const _Float16 lo = (_Float16)(wv - (float)hi);
      whi[r] = (uint32_t)__builtin_bit_cast(uint16_t, hi) << w_shift;
      wlo[r] = (uint32_t)__builtin_bit_cast(uint16_t, lo) << w_shift;
    }
    const half8 Whi = __builtin_bit_cast(half8, u32x4{whi[0], whi[1], whi[2], whi[3]});
    const half8 Wlo = __builtin_bit_cast(half8, u32x4{wlo[0], wlo[1], wlo[2], wlo[3]});
    // -- values: acc[pair][col] += sum_(t, parity) V[t][2 pair + parity] * w[t][head] [parity == col half]
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const half8 A = __builtin_bit_cast(half8, u32x4{va[blk][0], va[blk][1], va[blk][2], va[blk][3]});
      acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Whi, acc[blk], 0, 0, 0);
      acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Wlo, acc[blk], 0, 0, 0);
    }
  };

  // ---- stage loop ------------------------------------------------------------------
  // Stage i lives in LDS slot i & 1.  Iteration i: wait for this wave's
  // copies of stage i, barrier (now every wave's copies are in, and every
  // wave is done with stage i - 1), start the copies of stage i + 1 into the
  // other slot, then compute.  The copies of one stage are in flight while
  // the previous one is computed.
  const int nit = (span + strm - 1) / strm;
  auto advance = [&](int i) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    issue_dma(i + 1, (i + 1) & 1);
  };
  auto slot_of = [&](int i) { return (uint32_t)((i & 1) * stage_bytes + st * a.page_slot_bytes); };
  issue_dma(0, 0);
  if constexpr (kSplit) {
    // Iteration i runs the value part of this wave's page of stage i - 1,
    // then the key part of its page of stage i.  The value part needs no
    // stage data, so it starts right after the barrier; the key part reads
    // the slot.  Iterations 1 .. nit - 2 have both pages whole, so their
    // bodies have no branches.  (The scheduling barriers keep the compiler
    // from interleaving the two parts, which would hold both parts' lookups
    // in registers at once.)
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    // part[(nit - 1 - i) & 1]: this wave's page of stage i (so that the last
    // iteration always fills part[0] and a single copy of the tail exists)
    PagePart part[2];
    auto iteration = [&](int i, auto cur_tag) {  // cur_tag: (nit - 1 - i) & 1
      constexpr int CUR = decltype(cur_tag)::value;
      advance(i);
      value_part(part[CUR ^ 1], 0, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
      key_part(slot_of(i), part[CUR]);
      __builtin_amdgcn_sched_barrier(0);
    };
    // iteration 0: a key part only
    advance(0);
    if (st < span) {
      if ((nit - 1) & 1)
        key_part(slot_of(0), part[1]);
      else
        key_part(slot_of(0), part[0]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // iterations 1 .. nit - 2 (both pages whole) in pairs that end with
    // iteration nit - 2, whose page is in part 1
    int i = 1;
    if (nit - 2 > 0 && ((nit - 2) & 1)) iteration(i++, C1{});
    for (; i < nit - 1; i += 2) {
      iteration(i, C0{});
      iteration(i + 1, C1{});
    }
    // the last iteration (if it is not iteration 0), then the value part of
    // its page, masked at the sequence's end (only the sequence's last page
    // can be partial)
    const int P = strm * (nit - 1) + st;
    if (nit > 1) {
      advance(nit - 1);
      value_part(part[1], 0, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
      if (P < span) key_part(slot_of(nit - 1), part[0]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (P < span) value_part(part[0], (p0 + P) * kBlockSize + 4 * c, std::false_type{});
  } else {
    // both parts of a page in its own iteration (fewer registers live)
    auto iteration = [&](int i, auto full_tag) {
      advance(i);
      const int P = strm * i + st;
      if (P < span) {
        PagePart part;
        key_part(slot_of(i), part);
        __builtin_amdgcn_sched_barrier(0);
        value_part(part, (p0 + P) * kBlockSize + 4 * c, full_tag);
      }
    };
    for (int i = 0; i + 1 < nit; ++i) iteration(i, std::true_type{});
    iteration(nit - 1, std::false_type{});
  }

  // ---- finish the split ---------------------------------------------------------
  float l_tot = l_part + __shfl_xor(l_part, 16);
  l_tot += __shfl_xor(l_tot, 32);
  // gather the odd dims from column n + 8: o[r][d] = dim 32c + 8r + d of head hq
  float o[4][8];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const float mine = acc[blk][r];
      const float other = row_ror8(mine);
      o[r][2 * blk] = par ? other : mine;
      o[r][2 * blk + 1] = par ? mine : other;
    }
  const bool owner = par == 0 && hq < gsz;

  if (strm == 1) {
    if (owner) {
      const int h = qh0 + hq;
      const int64_t slot = ((int64_t)b * a.num_q_heads + h) * S + s;
      const float inv = 1.0f / l_tot;
      float* dst = a.part_acc + slot * kHeadDim + 32 * c;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<floatx4*>(dst + 8 * r) = floatx4{o[r][0] * inv, o[r][1] * inv, o[r][2] * inv, o[r][3] * inv};
        *reinterpret_cast<floatx4*>(dst + 8 * r + 4) = floatx4{o[r][4] * inv, o[r][5] * inv, o[r][6] * inv, o[r][7] * inv};
      }
      if (c == 0) a.part_lse[slot] = m_ref + __builtin_log2f(l_tot);
    }
    return;
  }

  // several streams per head: merge them through LDS (the stages and the
  // tables are dead after the barrier)
  __syncthreads();
  float* m_buf = reinterpret_cast<float*>(lds);                   // [waves][8]
  float* l_buf = m_buf + kMaxWaves * 8;                           // [waves][8]
  float* a_buf = l_buf + kMaxWaves * 8;                           // [waves][8][128]
  if (c == 0 && par == 0) {
    m_buf[wave * 8 + hq] = m_ref;
    l_buf[wave * 8 + hq] = l_tot;
  }
  if (par == 0) {
    float* dst = a_buf + (wave * 8 + hq) * kHeadDim + 32 * c;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int d = 0; d < 8; ++d) dst[8 * r + d] = o[r][d];
  }
  __syncthreads();
  if (st != 0 || !owner) return;
  float M = -__builtin_inff();
  for (int t = 0; t < strm; ++t) M = fmaxf(M, m_buf[(t * hpw + hs) * 8 + hq]);
  float lsum = 0.0f;
  float out[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) out[j] = 0.0f;
  for (int t = 0; t < strm; ++t) {
    const int wv = t * hpw + hs;
    const float mt = m_buf[wv * 8 + hq];
    const float scl = (mt == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mt - M);
    lsum += scl * l_buf[wv * 8 + hq];
    const float* src = a_buf + (wv * 8 + hq) * kHeadDim + 32 * c;
#pragma unroll
    for (int j = 0; j < 32; ++j) out[j] += scl * src[j];
  }
  const int h = qh0 + hq;
  const int64_t slot = ((int64_t)b * a.num_q_heads + h) * S + s;
  const float inv = 1.0f / lsum;
  float* dst = a.part_acc + slot * kHeadDim + 32 * c;
#pragma unroll
  for (int j = 0; j < 32; j += 4)
    *reinterpret_cast<floatx4*>(dst + j) = floatx4{out[j] * inv, out[j + 1] * inv, out[j + 2] * inv, out[j + 3] * inv};
  if (c == 0) a.part_lse[slot] = M + __builtin_log2f(lsum);
}

int decode_table_bytes(int k_bits, int v_bits) {
  auto bytes = [](int b) {
    switch (b) {
      case 2: return PairTable<2>::kBytes;
      case 3: return PairTable<3>::kBytes;
      case 4: return PairTable<4>::kBytes;
      case 5: return PairTable<5>::kBytes;
    }
    return 0;
  };
  return k_bits == v_bits ? bytes(k_bits) : bytes(k_bits) + bytes(v_bits);
}

int decode_merge_lds_bytes() { return kMaxWaves * 8 * (kHeadDim + 2) * 4; }

template <int KB, int VB, bool CONTIG, int MAXLD>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  const long long units = (long long)a.batch * a.head_groups * a.num_splits;
  // the appending decode is its own instantiation, so that the plain decode
  // compiles without the row encode
  if (a.app.on)
    hipLaunchKernelGGL((decode_split_kernel<KB, VB, CONTIG, MAXLD, true>), dim3((unsigned)units), dim3(64 * a.waves), 0,
                       st, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<KB, VB, CONTIG, MAXLD, false>), dim3((unsigned)units), dim3(64 * a.waves),
                       0, st, a);
  return hipGetLastError();
}

template <int KB, int VB>
static hipError_t launch_decode_kv(const DecodeArgs& a, hipStream_t st) {
  const int per_wave = (a.streams * (a.k_loads + a.v_loads) + a.waves - 1) / a.waves;
  const bool contig = a.kv_per_wg == a.num_kv_heads;
  if (per_wave <= 3) return contig ? launch_decode_t<KB, VB, true, 3>(a, st) : launch_decode_t<KB, VB, false, 3>(a, st);
  if (per_wave <= 4) return contig ? launch_decode_t<KB, VB, true, 4>(a, st) : launch_decode_t<KB, VB, false, 4>(a, st);
  return hipErrorInvalidValue;
}

template <int KB>
static hipError_t launch_decode_k(const DecodeArgs& a, int vb, hipStream_t st) {
  switch (vb) {
    case 2: return launch_decode_kv<KB, 2>(a, st);
    case 3: return launch_decode_kv<KB, 3>(a, st);
    case 4: return launch_decode_kv<KB, 4>(a, st);
    case 5: return launch_decode_kv<KB, 5>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int k_bits, int v_bits, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  switch (k_bits) {
    case 2: return launch_decode_k<2>(a, v_bits, stream);
    case 3: return launch_decode_k<3>(a, v_bits, stream);
    case 4: return launch_decode_k<4>(a, v_bits, stream);
    case 5: return launch_decode_k<5>(a, v_bits, stream);
  }
  return hipErrorInvalidValue;
}

// ===========================================================================
// Merge: one wave per (b, h).  Combines the splits' normalised rotated sums by
// their log2-sum-exp2, divides the value scale out, applies the inverse
// rotation s * H y / sqrt(128) and writes fp32 out (and, when asked, the
// sequence's log2-sum-exp2).  Lane l owns dims l and l + 64; lane s holds the
// weight of split s (at most 64 splits).
// ===========================================================================
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int lane = tid & 63;
  const int unit = __builtin_amdgcn_workgroup_id_x() * 4 + (tid >> 6);
  if (unit >= a.batch * a.num_q_heads) return;
  const int b = unit / a.num_q_heads;
  const int L = min(a.seq_lens[b], a.max_len);
  float* o = a.out + (int64_t)unit * kHeadDim;
  if (L <= 0) {
    o[lane] = 0.0f;
    o[lane + 64] = 0.0f;
    if (a.lse_out && lane == 0) a.lse_out[unit] = -__builtin_inff();
    return;
  }
  const int npages = (L + kBlockSize - 1) / kBlockSize;
  const int ns = (npages + a.pages_per_split - 1) / a.pages_per_split;
  const float* lse = a.part_lse + (int64_t)unit * a.num_splits;
  const float* pa = a.part_acc + (int64_t)unit * a.num_splits * kHeadDim;
  const float my = lane < ns ? lse[lane] : -__builtin_inff();
  float M = my;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float wgt = lane < ns ? __builtin_amdgcn_exp2f(my - M) : 0.0f;
  float den = wgt;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
  float y0 = 0.0f, y1 = 0.0f;
  // rounds of 16 splits with all their loads in flight together; past the
  // end a round reads the last split again (every split below ns wrote its
  // partial) with weight 0, so the loads need no branches
  constexpr int kU = 16;
  for (int sidx = 0; sidx < ns; sidx += kU) {
    float v0[kU], v1[kU], wu[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int si = min(sidx + u, ns - 1);
      wu[u] = sidx + u < ns ? __shfl(wgt, si) : 0.0f;
      v0[u] = pa[(int64_t)si * kHeadDim + lane];
      v1[u] = pa[(int64_t)si * kHeadDim + lane + 64];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      y0 += wu[u] * v0[u];
      y1 += wu[u] * v1[u];
    }
  }
  const float inv = 1.0f / den;
  y0 *= inv;
  y1 *= inv;
  if (a.lse_out && lane == 0) a.lse_out[unit] = M + __builtin_log2f(den);
  // H over 128 points: stage 64 inside the lane, stages 1..32 across lanes
  {
    const float u = y0, v = y1;
    y0 = u + v;
    y1 = u - v;
  }
  static_for<6>([&](auto sc) {
    constexpr int M = 1 << decltype(sc)::value;
    y0 = lane_bfly<M>(y0, lane);
    y1 = lane_bfly<M>(y1, lane);
  });
  const float s0 = ((pick4(a.sign_bits, lane >> 5) >> (lane & 31)) & 1u) ? -1.0f : 1.0f;
  const float s1 = ((pick4(a.sign_bits, 2 + (lane >> 5)) >> (lane & 31)) & 1u) ? -1.0f : 1.0f;
  o[lane] = s0 * y0 * a.inv_v_scale_over_sqrt_d;
  o[lane + 64] = s1 * y1 * a.inv_v_scale_over_sqrt_d;
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int units = a.batch * a.num_q_heads;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3((units + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tq
