// Single-query paged decode over TQ pages for gfx950: the wave-private
// kernel and its merge + inverse-rotation kernel.
//
// Same arithmetic as the staged kernel in tq_decode.hip: scores and value
// sums are formed in the rotated domain (R is orthogonal, so
// q . (n R^T c) = n (R q) . c and sum_t p_t n_t R^T c_t = R^T sum_t p_t n_t c_t),
// keys and values are looked up in replicated LDS pair tables, both
// contractions run on v_mfma_f32_16x16x32_f16 and the softmax is an online
// log2-domain one (TurboQuant docs, "Architecture", "Diagnostic vs Serving
// Paths": the paged decode rebuilds rows from packed pages inside its loop;
// pages as in "Cache Storage Objects"; rows as in "vLLM Usage", "TQ Byte
// Layout").  What differs is how the pages reach the compute, so that no
// wave ever waits for another inside the page walk:
//  * A wave owns every KV head of the page (NH = 1, 2 or 4 heads) and walks
//    its own pages: a whole page (K, then V) arrives through 16-byte
//    non-temporal buffer loads into registers one page ahead, is written into
//    the wave's private LDS slot, and all NH heads' query groups are computed
//    from there.  LDS operations of one wave run in order, so writing page
//    k + 1 over page k right after page k's reads were issued is safe without
//    a wait.
//  * Workgroups take equal shares of the concatenation of all sequences'
//    pages: workgroup i of n takes pages [i T / n, (i + 1) T / n) of the T in
//    total, computed on the device from seq_lens, so a ragged batch balances
//    by pages; a share may cover parts of several sequences (segments).
//  * The waves of a workgroup meet only at the start of a segment (rotated
//    queries and lookup tables, staged through LDS) and at its end (the
//    waves that walked the segment's pages merge through LDS); the segment's
//    partial result of sequence b from workgroup i goes to workspace slot
//    b + i, unique because workgroups take pages in order.  A segment that
//    is the whole sequence is finished on the spot (rotated back and written
//    to out; the merge kernel skips it), and a launch of one workgroup needs
//    no merge kernel at all.

#include "tq_decode_common.h"

#include <type_traits>
#include <utility>

namespace tq {

template <int NH>
struct WaveCount {  // waves per workgroup: two per SIMD (256 registers each)
  static constexpr int value = 8;
};

template <int KB, int VB, int NH>
struct WaveLayout {
  static constexpr int kRBK = 16 * KB + 4;
  static constexpr int kRBV = 16 * VB + 4;
  static constexpr int kKC = NH * kRBK;          // 16-byte chunks of a page (K): 16 tokens x NH rows
  static constexpr int kVC = NH * kRBV;          // (V)
  static constexpr int kMaxK = (kKC + 63) / 64;  // 64-lane loads per page
  static constexpr int kMaxV = (kVC + 63) / 64;
  static constexpr int kSlot = 16 * (kKC + kVC); // bytes of a wave's page slot: K rows, then V rows
  static constexpr int kW = WaveCount<NH>::value;
  static constexpr int kVTab = 0;
  static constexpr int kKTab = KB == VB ? 0 : PairTable<VB>::kBytes;
  static constexpr int kSlots = kKTab + PairTable<KB>::kBytes;
  static constexpr int kBytes = kSlots + kW * kSlot;
  // end-of-segment merge: [wave][head][query head][128 (+4 padding)] sums, then maxima and sums
  static constexpr int kMergeRow = kHeadDim + 4;
  static constexpr int kMergeBytes = (kW * NH * 8 * kMergeRow + 2 * kW * NH * 8) * 4;
};

// rotated queries staged per KV head: 16 dwords per lane, then one scale per head
constexpr int kQStageDwords = 16 * 64;
inline int wave_stage_bytes(int num_kv_heads) { return num_kv_heads * (kQStageDwords * 4 + 4); }

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// floor(T i / n) for 0 <= i <= n (T, i, n wave-uniform): the boundaries of
// the workgroups' shares.  32-bit division when T n fits in 32 bits (the
// 64-bit one is a long software sequence on the critical path of both kernels).
__device__ __forceinline__ long long share_point(long long T, long long i, long long n) {
  if (T * n < (1LL << 32)) return (long long)((uint32_t)(T * i) / (uint32_t)n);
  return T * i / n;
}

// Rotated, scaled query of KV head x's query group as the B operand of the
// score MFMAs.  Lane (n, c) covers dims 32c .. 32c + 31; column n < 8 holds
// the fp16 hi part of query head x * group + n, column n + 8 its lo part;
// qd[p] = the fp16 pair (dims 32c + 2p, 32c + 2p + 1) of the lane's column.
// Scores come out multiplied by 1 / q_unscale, one power of two per group.
// load_query reads the lane's 32 query values (so that the loads can be in
// flight while other work is issued), rotate_query forms qd from them.
__device__ __forceinline__ void load_query(const WaveArgs& a, int b, int x, int lane, float (&v)[32]) {
  const int n = lane & 15, c = lane >> 4;
  const int hq = n & 7;
  const bool has = hq < a.group;
  const int64_t qoff = ((int64_t)b * a.num_q_heads + (int64_t)x * a.group + (has ? hq : 0)) * kHeadDim + 32 * c;
  // (columns past the group read head 0's values; rotate_query zeroes them)
  if (a.q_dtype == 0) {
    const float* p = static_cast<const float*>(a.q) + qoff;
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = p[j];
  } else if (a.q_dtype == 1) {
    const _Float16* p = static_cast<const _Float16*>(a.q) + qoff;
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = (float)p[j];
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(a.q) + qoff;
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = bf16_to_f32(p[j]);
  }
}

__device__ __forceinline__ void rotate_query(const WaveArgs& a, int lane, float (&v)[32], uint32_t (&qd)[16],
                                             float& q_unscale) {
  const int n = lane & 15, c = lane >> 4;
  const int par = n >> 3;
  const bool has = (n & 7) < a.group;
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = has ? v[j] : 0.0f;
  uint32_t sw = pick4(a.sign_bits, c);
  asm volatile("" : "+v"(sw));  // keeps the 32 sign masks below from being hoisted (and held) out of the segment loop
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (((sw >> j) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 32; h <<= 1)
#pragma unroll
    for (int j = 0; j < 32; ++j)
      if ((j & h) == 0) {
        const float u = v[j], w = v[j + h];
        v[j] = u + w;
        v[j + h] = u - w;
      }
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = lane_bfly<16>(v[j], lane);
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = lane_bfly<32>(v[j], lane);
  // one power of two for the group that puts its largest coordinate near 2^10,
  // so the fp16 hi / lo halves keep their precision for any query magnitude
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, __builtin_fabsf(v[j] * a.q_scale));
  amax = max_across_rows(amax);
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  amax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(amax)));
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
      const float s = v[2 * p + e] * up;
      const _Float16 hi = (_Float16)s;
      h2[e] = par ? (_Float16)(s - (float)hi) : hi;
    }
    qd[p] = pack_half2(h2[0], h2[1]);
  }
}

template <int KB, int VB, int NH>
__global__ __launch_bounds__(64 * WaveCount<NH>::value) void decode_wave_kernel(WaveArgs a) {
  using LY = WaveLayout<KB, VB, NH>;
  using KT = PairTable<KB>;
  using VT = PairTable<VB>;
  constexpr int W = LY::kW;
  constexpr int RBK = LY::kRBK, RBV = LY::kRBV;
  constexpr int KC = LY::kKC, VC = LY::kVC;
  constexpr int MAXK = LY::kMaxK, MAXV = LY::kMaxV;
  constexpr int kNT = 2;  // cache policy of the page loads: non-temporal (read once)
  __shared__ __attribute__((aligned(16))) uint8_t lds[kDecodeLdsBytes];

  const int wg = __builtin_amdgcn_workgroup_id_x();
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15, c = lane >> 4;
  const int hq = n & 7, par = n >> 3;
  constexpr int S = W;     // streams: every wave owns every KV head and walks every W-th page
  const int st = wave;
  constexpr int g0 = 0;    // first KV head of this wave
  const int G = a.group;
  const int Hkv = a.num_kv_heads;
  const int B = a.batch;

  // ---- this workgroup's share of the pages ----------------------------------------
  auto seq_len = [&](int b) { return min(max(a.seq_lens[b], 0), a.max_len); };
  auto pages_of = [](int L) { return (L + kBlockSize - 1) / kBlockSize; };
  auto seq_pages = [&](int b) { return pages_of(seq_len(b)); };
  // lengths of sequences base + lane (those of the first 64 are read once)
  const int len_first = lane < B ? seq_len(lane) : 0;
  auto len_at = [&](int base) { return base == 0 ? len_first : (base + lane < B ? seq_len(base + lane) : 0); };
  long long T = 0;
  for (int base = 0; base < B; base += 64) T += __builtin_amdgcn_readfirstlane(wave_sum_i(pages_of(len_at(base))));
  const int Hq = a.num_q_heads;
  if (a.direct) {
    // no merge kernel follows: the one workgroup also writes the zero rows of
    // empty sequences (one wave per sequence)
    for (int bb = wave; bb < B; bb += W) {
      if (seq_pages(bb) > 0) continue;
      float* o = a.out + (int64_t)bb * Hq * kHeadDim;
      for (int i = lane; i < Hq * kHeadDim / 4; i += 64)
        *reinterpret_cast<floatx4*>(o + 4 * i) = floatx4{0.f, 0.f, 0.f, 0.f};
      if (a.lse_out)
        for (int h = lane; h < Hq; h += 64) a.lse_out[(int64_t)bb * Hq + h] = -__builtin_inff();
    }
  }
  const long long r0 = share_point(T, wg, a.num_wg);
  const long long r1 = share_point(T, wg + 1, a.num_wg);
  if (r0 >= r1) return;  // every wave of the workgroup leaves here together
  int b = 0;             // the sequence holding page r0, its first page and its length
  long long sb = 0;
  int L_cur = 0;
  {
    long long off = 0;
    for (int base = 0; base < B; base += 64) {
      const int lv = len_at(base);
      const int p = pages_of(lv);
      const int incl = wave_incl_scan(p, lane);
      const long long s_l = off + incl - p;
      const uint64_t hit = __ballot(p > 0 && s_l <= r0 && r0 < s_l + p);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        b = base + l;
        sb = off + __builtin_amdgcn_readlane(incl - p, l);
        L_cur = __builtin_amdgcn_readlane(lv, l);
        break;
      }
      off += __builtin_amdgcn_readlane(incl, 63);
    }
  }

  // ---- load geometry: load i, lane l moves chunk f = 64 i + l of the page to
  // slot byte 16 f; lanes past the last chunk repeat a chunk of the load
  // before (the same data to the same place) -------------------------------------
  auto fold = [&](int i, int C) {
    const int f = 64 * i + lane;
    return f < C ? f : f - (C >= 64 ? 64 : C);
  };

  // ---- per-lane offsets inside a slot: row (t, u) of K at (t NH + u) RB, of V
  // at 16 KC + (t NH + u) RB ------------------------------------------------------
  const uint32_t slot = (uint32_t)(LY::kSlots + wave * LY::kSlot);
  const uint32_t k_idx_lane = slot + (uint32_t)(n * NH * RBK + 4 * KB * c);
  const uint32_t k_norm_lane = slot + (uint32_t)((4 * c + (n & 3)) * NH * RBK + RBK - 4);
  const int v_byte = n * VB;
  const int v_dat = (VB == 3 || VB == 5) ? (v_byte & ~3) : (v_byte & ~1);
  const uint32_t v_dat_lane = slot + (uint32_t)(16 * KC + 4 * c * NH * RBV + v_dat);
  const uint32_t v_norm_lane = slot + (uint32_t)(16 * KC + (4 * c + (n & 3)) * NH * RBV + RBV - 4);
  const uint32_t v_shift = 8u * (uint32_t)(v_byte & 3);
  // this lane's replica (hi dword; the lo dword is 4 bytes further)
  const uint32_t k_lane = (uint32_t)(lane & (KT::kRep - 1)) * 8u;
  const uint32_t v_lane = (uint32_t)(lane & (VT::kRep - 1)) * 8u;
  const uint8_t* k_tab = lds + LY::kKTab;
  const uint8_t* v_tab = lds + LY::kVTab;
  const uint32_t w_shift = 16u * (uint32_t)par;  // weight half: even dims in columns < 8

  // ---- segments: the pages of one sequence inside this workgroup's share ------------
  bool first = true;
  while (sb < r1) {
    const int L = L_cur;
    const int pb = pages_of(L);
    if (pb > 0) {
      const int ja = (int)((r0 > sb ? r0 : sb) - sb);
      const int je = (int)((r1 < sb + pb ? r1 : sb + pb) - sb);

      // -- loads first, in the order they are needed: this wave's block ids
      // (its pages are segment pages ja + st, ja + st + S, ...), the query of
      // its KV head (one head per wave: num_kv_heads <= 8 waves), then page 0,
      // which is in flight while the query is rotated and the tables filled
      const int nseg = je - ja;
      const int n_my = nseg > st ? (nseg - st + S - 1) / S : 0;
      const int32_t* bt = a.block_table + (int64_t)b * a.max_blocks_per_seq;
      auto bids_at = [&](int k0) {  // block ids of pages k0 .. k0 + 63, one per lane; -1: out of range
        // (the read is unconditional, of an entry inside the sequence's row,
        // so that it does not wait where it is issued)
        const int k = k0 + lane;
        const int e = min(ja + st + min(k, max(n_my - 1, 0)) * S, a.max_blocks_per_seq - 1);
        const int x = bt[e];
        return (k < n_my && x >= 0 && (int64_t)x < a.num_blocks) ? x : -1;
      };
      int bid_cur = bids_at(0);
      int bid_next = bids_at(64);

      // (with four heads per wave the registers do not allow the query and
      // page 0 to be held across the other loads and the barrier: they are
      // loaded where they are used)
      constexpr bool kEarly = NH <= 2;
      float qraw[32];
      const bool has_q = wave < Hkv;
      if (kEarly && has_q) load_query(a, b, wave, lane, qraw);
      u32x4 R[MAXK + MAXV];
      auto issue = [&](int k) {  // page k's span into registers
        if ((k & 63) == 0 && k > 0) {
          bid_cur = bid_next;
          bid_next = bids_at(k + 64);
        }
        const int blk = __builtin_amdgcn_readlane(bid_cur, k & 63);
        const uint8_t* kp = a.k_pages + (blk < 0 ? 0 : (int64_t)blk * a.k_page_bytes);
        const uint8_t* vp = a.v_pages + (blk < 0 ? 0 : (int64_t)blk * a.v_page_bytes);
        // a block id out of range gets a zero-sized buffer, which reads zeros
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void*)kp, 0, blk < 0 ? 0 : (int)a.k_page_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)vp, 0, blk < 0 ? 0 : (int)a.v_page_bytes, 0x00020000);
#pragma unroll
        for (int i = 0; i < MAXK; ++i)
          R[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, 16u * fold(i, KC), 0, kNT));
#pragma unroll
        for (int i = 0; i < MAXV; ++i)
          R[MAXK + i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, 16u * fold(i, VC), 0, kNT));
      };
      if (kEarly && n_my > 0) issue(0);
      if (!first) __syncthreads();  // the previous segment's merge is done with the LDS
      first = false;

      // -- rotated queries staged in LDS past the tables (in the page slots,
      // which are not written before the next barrier), the tables meanwhile
      uint32_t* qst = reinterpret_cast<uint32_t*>(lds + LY::kSlots);
      if (has_q) {
        uint32_t qx[16];
        float qu;
        if (!kEarly) load_query(a, b, wave, lane, qraw);
        rotate_query(a, lane, qraw, qx, qu);
#pragma unroll
        for (int p = 0; p < 16; ++p) qst[wave * kQStageDwords + p * 64 + lane] = qx[p];
        if (lane == 0) reinterpret_cast<float*>(qst)[Hkv * kQStageDwords + wave] = qu;
      }
      fill_pair_table_flat<KB>(lds + LY::kKTab, a.k_cent, tid, 64 * W);
      if constexpr (KB != VB) fill_pair_table_flat<VB>(lds + LY::kVTab, a.v_cent, tid, 64 * W);
      __syncthreads();
      uint32_t qd[NH][16];
      float q_unscale[NH];
#pragma unroll
      for (int u = 0; u < NH; ++u) {
#pragma unroll
        for (int p = 0; p < 16; ++p) qd[u][p] = qst[(g0 + u) * kQStageDwords + p * 64 + lane];
        q_unscale[u] = __int_as_float(
            __builtin_amdgcn_readfirstlane(__float_as_int(reinterpret_cast<float*>(qst)[Hkv * kQStageDwords + g0 + u])));
      }
      __syncthreads();  // the staged queries are read: the slots may be written

      floatx4 acc[NH][4];
      float m_ref[NH], l_part[NH];
#pragma unroll
      for (int u = 0; u < NH; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[u][i] = floatx4{0.f, 0.f, 0.f, 0.f};
        m_ref[u] = -__builtin_inff();
        l_part[u] = 0.0f;
      }

      auto commit = [&]() {  // the registers into the slot (in LDS order after the reads of the last page)
#pragma unroll
        for (int i = 0; i < MAXK; ++i) *reinterpret_cast<u32x4*>(lds + slot + 16 * fold(i, KC)) = R[i];
#pragma unroll
        for (int i = 0; i < MAXV; ++i) *reinterpret_cast<u32x4*>(lds + slot + 16 * KC + 16 * fold(i, VC)) = R[MAXK + i];
      };

      // -- one head's part of a page ------------------------------------------------
      constexpr int kVW = (VB == 3 || VB == 5) ? 2 : 1;
      auto head_page = [&](auto uc, auto full_tag, int tok0) {
        constexpr int u = decltype(uc)::value;
        constexpr bool FULL = decltype(full_tag)::value;
        // key indices (dims 32c .. 32c + 31 of token n) and the key norm of token 4c + (n & 3)
        uint32_t kw[KB];
#pragma unroll
        for (int i = 0; i < KB; ++i) kw[i] = lds_u32(lds, k_idx_lane + u * RBK + 4 * i);
        const float nk = __uint_as_float(lds_u32(lds, k_norm_lane + u * RBK));
        // value index words of tokens 4c .. 4c + 3 and the value norm of token 4c + (n & 3)
        uint32_t vw[kVW][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t vo = v_dat_lane + (uint32_t)(r * NH * RBV + u * RBV);
          if constexpr (VB == 2) {
            vw[0][r] = *reinterpret_cast<const uint16_t*>(lds + vo);
          } else {
            vw[0][r] = lds_u32(lds, vo);
            if constexpr (kVW == 2) vw[kVW - 1][r] = lds_u32(lds, vo + 4);
          }
        }
        const float nv = __uint_as_float(lds_u32(lds, v_norm_lane + u * RBV));

        uint32_t kh[16], kl[16];
        auto klook = [&](int p) {
          const uint32_t ad = pair_addr<KB>(kw, p, k_lane);
          kh[p] = lds_u32(k_tab, ad);
          kl[p] = lds_u32(k_tab, ad + 4);
        };
        floatx4 sc = floatx4{0.f, 0.f, 0.f, 0.f};
        if constexpr (NH == 1) {
          // scores, one head per wave: MFMA m takes pairs p = 2m and p' = 2m + 1,
          // A = [K_hi(p), K_lo(p), K_hi(p'), K_lo(p')] as the lookups return them,
          // B = [q(p), q(p), q(p'), q(p')]; columns h and h + 8 sum to
          // (K_hi + K_lo) . (q_hi + q_lo).  The rolling window keeps the lookups of
          // the next two MFMAs in flight while one runs.
          auto kmfma = [&](int m) {
            const half8 A = __builtin_bit_cast(half8, u32x4{kh[2 * m], kl[2 * m], kh[2 * m + 1], kl[2 * m + 1]});
            const half8 Bq = __builtin_bit_cast(
                half8, u32x4{qd[u][2 * m], qd[u][2 * m], qd[u][2 * m + 1], qd[u][2 * m + 1]});
            sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bq, sc, 0, 0, 0);
          };
#pragma unroll
          for (int p = 0; p < 4; ++p) klook(p);
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            if (m + 2 < 8) {
              klook(2 * (m + 2));
              klook(2 * (m + 2) + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            kmfma(m);
          }
        } else {
          // scores, several heads per wave (registers are tight): MFMA pair m
          // covers dims 32c + 8m .. 32c + 8m + 7 (pairs 4m .. 4m + 3), A = the hi
          // (then lo) fp16 parts of those keys, B = the query pairs qd[4m .. 4m + 3]
          // as they are stored; columns h and h + 8 sum to (K_hi + K_lo) . (q_hi + q_lo)
          auto kmfma = [&](int m) {
            const half8 Bq =
                __builtin_bit_cast(half8, u32x4{qd[u][4 * m], qd[u][4 * m + 1], qd[u][4 * m + 2], qd[u][4 * m + 3]});
            const half8 Ah = __builtin_bit_cast(half8, u32x4{kh[4 * m], kh[4 * m + 1], kh[4 * m + 2], kh[4 * m + 3]});
            const half8 Al = __builtin_bit_cast(half8, u32x4{kl[4 * m], kl[4 * m + 1], kl[4 * m + 2], kl[4 * m + 3]});
            sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Bq, sc, 0, 0, 0);
            sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, Bq, sc, 0, 0, 0);
          };
#pragma unroll
          for (int p = 0; p < 4; ++p) klook(p);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            if (m + 1 < 4) {
#pragma unroll
              for (int p = 0; p < 4; ++p) klook(4 * (m + 1) + p);
            }
            __builtin_amdgcn_sched_barrier(0);
            kmfma(m);
          }
        }

        // value lookups: dword (V[t][2p], V[t][2p+1]) for pair p = 4n + blk of
        // token 4c + j is exactly A[row n][k = 2j, 2j + 1] of value block blk
        uint32_t va[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t words[2];
          if constexpr (kVW == 2) {
            const uint64_t all = ((((uint64_t)vw[kVW - 1][j]) << 32) | vw[0][j]) >> v_shift;
            words[0] = (uint32_t)all;
            words[1] = (uint32_t)(all >> 32);
          } else {
            words[0] = vw[0][j];
            words[1] = 0;
          }
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) va[blk][j] = lds_u32(v_tab, pair_addr<VB>(words, blk, v_lane));
        }

        // softmax bookkeeping (log2 domain).  e = an upper bound of log2(n_v) from
        // the exponent bits (clamped so empty rows cannot blow up p).  Per-token
        // factors are formed on the lane that read the norm and broadcast inside
        // each quad (lane (n, c) needs tokens 4c .. 4c + 3).
        const float nkq_mine = nk * q_unscale[u];
        const float e_mine = fmaxf(__builtin_fmaf((float)(__float_as_uint(nv) >> 24), 2.0f, -126.0f), -64.0f);
        float full[4], xv[4];
        {
#pragma clang fp contract(off)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            full[r] = (sc[r] + row_ror8(sc[r])) * quad_bcast_r(nkq_mine, r);
            xv[r] = full[r] + quad_bcast_r(e_mine, r);
            if constexpr (!FULL) xv[r] = (tok0 + r < L) ? xv[r] : -__builtin_inff();
          }
        }
        float pmax = fmaxf(fmaxf(xv[0], xv[1]), fmaxf(xv[2], xv[3]));
        pmax = max_across_rows(pmax);
        if (__builtin_amdgcn_ballot_w64(pmax > m_ref[u] + 8.0f) != 0) {
          const float m_new = fmaxf(m_ref[u], pmax);
          const float alpha = (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_ref[u] - m_new);
          l_part[u] *= alpha;
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[u][q] *= alpha;
          m_ref[u] = m_new;
        }
        // weights w = p * n_v as fp16 hi + lo, placed in this column's half
        uint32_t whi[4], wlo[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float pr = __builtin_amdgcn_exp2f(full[r] - m_ref[u]);
          if constexpr (!FULL) pr = (tok0 + r < L) ? pr : 0.0f;
          l_part[u] += pr;
          float wv = pr * quad_bcast_r(nv, r);
          if constexpr (!FULL) wv = (tok0 + r < L) ? wv : 0.0f;  // rows past the end may hold anything
          const _Float16 hi = (_Float16)wv;
          const _Float16 lo = (_Float16)(wv - (float)hi);
          whi[r] = (uint32_t)__builtin_bit_cast(uint16_t, hi) << w_shift;
          wlo[r] = (uint32_t)__builtin_bit_cast(uint16_t, lo) << w_shift;
        }
        const half8 Whi = __builtin_bit_cast(half8, u32x4{whi[0], whi[1], whi[2], whi[3]});
        const half8 Wlo = __builtin_bit_cast(half8, u32x4{wlo[0], wlo[1], wlo[2], wlo[3]});
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          const half8 A = __builtin_bit_cast(half8, u32x4{va[blk][0], va[blk][1], va[blk][2], va[blk][3]});
          acc[u][blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Whi, acc[u][blk], 0, 0, 0);
          acc[u][blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Wlo, acc[u][blk], 0, 0, 0);
        }
      };

      // -- the page walk: page k + 1 is in flight while page k is computed.  Only
      // the sequence's last page can be partly filled; it is computed after the
      // loop by the wave that has it.  (The scheduling barriers keep the
      // compiler from interleaving heads, which would hold several heads'
      // lookups in registers at once.)
      const bool tail = n_my > 0 && (ja + st + (n_my - 1) * S + 1) * kBlockSize > L;
      const int n_full = n_my - (tail ? 1 : 0);
      auto compute = [&](auto full_tag, int tok0) {
        static_for<NH>([&](auto uc) {
          head_page(uc, full_tag, tok0);
          __builtin_amdgcn_sched_barrier(0);
        });
      };
      if (n_my > 0) {
        if (!kEarly) issue(0);
        commit();
        if (n_my > 1) issue(1);
      }
      for (int k = 0; k < n_full; ++k) {
        compute(std::true_type{}, 0);
        if (k + 1 < n_my) {
          commit();
          if (k + 2 < n_my) issue(k + 2);
        }
      }
      if (tail) compute(std::false_type{}, (ja + st + (n_my - 1) * S) * kBlockSize + 4 * c);

      // -- finish the segment ------------------------------------------------------
      // per head: l summed over the four token rows; o[r][d] = dim 32c + 8r + d of
      // query head hq, gathered from the two column halves (lanes with par == 0)
      auto finish_head = [&](int u, float (&o)[4][8]) {
        float lt = l_part[u] + __shfl_xor(l_part[u], 16);
        lt += __shfl_xor(lt, 32);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) {
            const float mine = acc[u][blk][r];
            const float other = row_ror8(mine);
            o[r][2 * blk] = par ? other : mine;
            o[r][2 * blk + 1] = par ? mine : other;
          }
        return lt;
      };
      const int64_t out_slot = (int64_t)b + wg;
      // this workgroup holds every page of the sequence: it writes the final
      // output (normalised, rotated back, value scale divided out) and the
      // merge kernel skips the sequence
      const bool whole = ja == 0 && je == pb;
      {
        // the W streams merge through LDS (slots and tables are dead)
        __syncthreads();
        constexpr int kRow = LY::kMergeRow;
        float* mg = reinterpret_cast<float*>(lds);
        float* m_buf = mg + W * NH * 8 * kRow;
        float* l_buf = m_buf + W * NH * 8;
#pragma unroll
        for (int u = 0; u < NH; ++u) {
          float o[4][8];
          const float lt = finish_head(u, o);
          const int e = (wave * NH + u) * 8 + hq;
          if (c == 0 && par == 0) {
            m_buf[e] = m_ref[u];
            l_buf[e] = lt;
          }
          if (par == 0) {
            float* dst = mg + e * kRow + 32 * c;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              *reinterpret_cast<floatx4*>(dst + 8 * r) = floatx4{o[r][0], o[r][1], o[r][2], o[r][3]};
              *reinterpret_cast<floatx4*>(dst + 8 * r + 4) = floatx4{o[r][4], o[r][5], o[r][6], o[r][7]};
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        // KV head x of the workgroup is combined by wave x % W: lane = (query head
        // lane >> 3, dims 16 (lane & 7) .. + 15)
        const int hh = lane >> 3, d0 = 16 * (lane & 7);
        for (int x = wave; x < Hkv; x += W) {
          const int hsx = x / NH, ux = x - hsx * NH;
          if (hh < G) {
            float M = -__builtin_inff();
            for (int t = 0; t < S; ++t) M = fmaxf(M, m_buf[((hsx * S + t) * NH + ux) * 8 + hh]);
            float lsum = 0.0f;
            float ov[16];
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) ov[jj] = 0.0f;
#pragma unroll 2
            for (int t = 0; t < S; ++t) {
              const int e = ((hsx * S + t) * NH + ux) * 8 + hh;
              const float mt = m_buf[e];
              const float scl = (mt == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mt - M);
              lsum += scl * l_buf[e];
              const float* src = mg + e * kRow + d0;
#pragma unroll
              for (int jj = 0; jj < 16; jj += 4) {
                const floatx4 v4 = *reinterpret_cast<const floatx4*>(src + jj);
                ov[jj] += scl * v4[0];
                ov[jj + 1] += scl * v4[1];
                ov[jj + 2] += scl * v4[2];
                ov[jj + 3] += scl * v4[3];
              }
            }
            const float inv = 1.0f / lsum;
            const int h = x * G + hh;
            if (whole) {
              // y = H (ov / l) over the 128 dims d0 + jj = 16 (lane & 7) + jj
              // (the unnormalised Hadamard butterfly: dims i < j = i + step
              // become (y_i + y_j, y_i - y_j)): steps 1 .. 8 inside the lane,
              // 16 .. 64 across the head's eight lanes; then the signs and the
              // value scale with the rotation's 1 / sqrt(128)
              float y[16];
#pragma unroll
              for (int jj = 0; jj < 16; ++jj) y[jj] = ov[jj] * inv;
#pragma unroll
              for (int st2 = 1; st2 < 16; st2 <<= 1)
#pragma unroll
                for (int jj = 0; jj < 16; ++jj)
                  if ((jj & st2) == 0) {
                    const float u0 = y[jj], u1 = y[jj + st2];
                    y[jj] = u0 + u1;
                    y[jj + st2] = u0 - u1;
                  }
              static_for<3>([&](auto sc) {
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) y[jj] = lane_bfly<(1 << decltype(sc)::value)>(y[jj], lane);
              });
              uint32_t sw = pick4(a.sign_bits, d0 >> 5) >> (d0 & 31);  // the 16 signs of dims d0 .. d0 + 15
              asm volatile("" : "+v"(sw));  // (computed here, not hoisted and held across the walk)
              float* dst = a.out + ((int64_t)b * Hq + h) * kHeadDim + d0;
              if (a.lse_out && (lane & 7) == 0) a.lse_out[(int64_t)b * Hq + h] = M + __builtin_log2f(lsum);
#pragma unroll
              for (int jj = 0; jj < 16; jj += 4) {
                floatx4 o4;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  o4[e] = (((sw >> (jj + e)) & 1u) ? -a.out_scale : a.out_scale) * y[jj + e];
                *reinterpret_cast<floatx4*>(dst + jj) = o4;
              }
            } else {
              float* dst = a.part_acc + (out_slot * Hq + h) * kHeadDim + d0;
#pragma unroll
              for (int jj = 0; jj < 16; jj += 4)
                *reinterpret_cast<floatx4*>(dst + jj) =
                    floatx4{ov[jj] * inv, ov[jj + 1] * inv, ov[jj + 2] * inv, ov[jj + 3] * inv};
              if ((lane & 7) == 0) a.part_lse[out_slot * Hq + h] = M + __builtin_log2f(lsum);
            }
          }
        }
      }
    }
    sb += pb;
    ++b;
    if (sb < r1) L_cur = seq_len(b);
  }
}

template <int KB, int VB, int NH>
static constexpr bool wave_layout_fits(int num_kv_heads) {
  using LY = WaveLayout<KB, VB, NH>;
  return LY::kBytes <= kDecodeLdsBytes && LY::kMergeBytes <= kDecodeLdsBytes && num_kv_heads <= LY::kW &&
         num_kv_heads * (kQStageDwords * 4 + 4) <= LY::kW * LY::kSlot;
}

template <int KB, int VB>
static bool wave_fits_kv(int nh, int hkv) {
  switch (nh) {
    case 1: return wave_layout_fits<KB, VB, 1>(hkv);
    case 2: return wave_layout_fits<KB, VB, 2>(hkv);
    case 4: return wave_layout_fits<KB, VB, 4>(hkv);
  }
  return false;
}

template <int KB>
static bool wave_fits_k(int vb, int nh, int hkv) {
  switch (vb) {
    case 2: return wave_fits_kv<KB, 2>(nh, hkv);
    case 3: return wave_fits_kv<KB, 3>(nh, hkv);
    case 4: return wave_fits_kv<KB, 4>(nh, hkv);
    case 5: return wave_fits_kv<KB, 5>(nh, hkv);
  }
  return false;
}

bool wave_fits(int k_bits, int v_bits, int nh, int num_kv_heads) {
  switch (k_bits) {
    case 2: return wave_fits_k<2>(v_bits, nh, num_kv_heads);
    case 3: return wave_fits_k<3>(v_bits, nh, num_kv_heads);
    case 4: return wave_fits_k<4>(v_bits, nh, num_kv_heads);
    case 5: return wave_fits_k<5>(v_bits, nh, num_kv_heads);
  }
  return false;
}

int wave_waves(int nh) { return (nh == 1 || nh == 2 || nh == 4) ? WaveCount<1>::value : 0; }

template <int KB, int VB, int NH>
static hipError_t launch_wave_t(const WaveArgs& a, hipStream_t st) {
  if constexpr (!wave_layout_fits<KB, VB, NH>(NH)) {
    return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((decode_wave_kernel<KB, VB, NH>), dim3((unsigned)a.num_wg), dim3(64 * WaveCount<NH>::value), 0,
                       st, a);
    return hipGetLastError();
  }
}

template <int KB, int VB>
static hipError_t launch_wave_kv(const WaveArgs& a, int nh, hipStream_t st) {
  switch (nh) {
    case 1: return launch_wave_t<KB, VB, 1>(a, st);
    case 2: return launch_wave_t<KB, VB, 2>(a, st);
    case 4: return launch_wave_t<KB, VB, 4>(a, st);
  }
  return hipErrorInvalidValue;
}

template <int KB>
static hipError_t launch_wave_k(const WaveArgs& a, int vb, int nh, hipStream_t st) {
  switch (vb) {
    case 2: return launch_wave_kv<KB, 2>(a, nh, st);
    case 3: return launch_wave_kv<KB, 3>(a, nh, st);
    case 4: return launch_wave_kv<KB, 4>(a, nh, st);
    case 5: return launch_wave_kv<KB, 5>(a, nh, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_wave(const WaveArgs& a, int k_bits, int v_bits, int nh, hipStream_t stream) {
  if (a.batch == 0 || a.num_wg == 0) return hipSuccess;
  switch (k_bits) {
    case 2: return launch_wave_k<2>(a, v_bits, nh, stream);
    case 3: return launch_wave_k<3>(a, v_bits, nh, stream);
    case 4: return launch_wave_k<4>(a, v_bits, nh, stream);
    case 5: return launch_wave_k<5>(a, v_bits, nh, stream);
  }
  return hipErrorInvalidValue;
}

// ===========================================================================
// Merge: one wave per (b, h).  Finds the workgroups that took sequence b's
// pages (the same integer split of the page concatenation as the decode
// kernel); a sequence that one workgroup held was finished there.  Otherwise
// it combines the workgroups' normalised rotated sums by their
// log2-sum-exp2, divides the value scale out, applies the inverse rotation
// s * H y / sqrt(128) and writes fp32 out.  Lane l owns dims l and l + 64.
// ===========================================================================
__global__ __launch_bounds__(256) void merge_wave_kernel(WaveMergeArgs a) {
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int lane = tid & 63;
  const int unit = __builtin_amdgcn_workgroup_id_x() * 4 + (tid >> 6);
  if (unit >= a.batch * a.num_q_heads) return;
  const int b = unit / a.num_q_heads;
  const int h = unit - b * a.num_q_heads;
  const int Hq = a.num_q_heads;
  float* o = a.out + (int64_t)unit * kHeadDim;
  auto seq_pages = [&](int s) {
    const int L = min(max(a.seq_lens[s], 0), a.max_len);
    return (L + kBlockSize - 1) / kBlockSize;
  };
  long long T = 0, sb = 0;
  for (int base = 0; base < a.batch; base += 64) {
    const int s = base + lane;
    const int p = s < a.batch ? seq_pages(s) : 0;
    T += __builtin_amdgcn_readfirstlane(wave_sum_i(p));
    sb += __builtin_amdgcn_readfirstlane(wave_sum_i(s < b ? p : 0));
  }
  const int pb = seq_pages(b);
  if (pb <= 0) {
    o[lane] = 0.0f;
    o[lane + 64] = 0.0f;
    if (a.lse_out && lane == 0) a.lse_out[unit] = -__builtin_inff();
    return;
  }
  const long long NW = a.num_wg;
  auto wg_of = [&](long long page) {  // the workgroup i with i T / NW <= page < (i + 1) T / NW
    long long i = T * NW < (1LL << 32) ? (long long)((uint32_t)(page * NW) / (uint32_t)T) : page * NW / T;
    while (i + 1 < NW && share_point(T, i + 1, NW) <= page) ++i;
    while (i > 0 && share_point(T, i, NW) > page) --i;
    return (int)i;
  };
  const int i0 = wg_of(sb), i1 = wg_of(sb + pb - 1);
  if (i0 == i1) return;  // one workgroup held the whole sequence and wrote its output
  const int ns = i1 - i0 + 1;
  // a workgroup between i0 and i1 whose share is empty (more workgroups than
  // pages) wrote nothing: its slot is skipped
  auto live = [&](int i) { return share_point(T, i, NW) < share_point(T, i + 1, NW); };
  const int64_t slot0 = (int64_t)b + i0;
  const float* lse = a.part_lse + slot0 * Hq + h;                      // stride Hq per slot
  const float* pa = a.part_acc + (slot0 * Hq + h) * kHeadDim;          // stride Hq * 128 per slot
  const int64_t pstride = (int64_t)Hq * kHeadDim;
  // lane s holds slot s's log2-sum-exp2 (the first 64 slots are read once)
  auto lse_at = [&](int s) { return (s < ns && live(i0 + s)) ? lse[(int64_t)s * Hq] : -__builtin_inff(); };
  const float lse_first = lse_at(lane);
  float M = lse_first;
  for (int s = lane + 64; s < ns; s += 64) M = fmaxf(M, lse_at(s));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float den = 0.0f, y0 = 0.0f, y1 = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const int cnt = min(64, ns - s0);
    const float my = s0 == 0 ? lse_first : lse_at(s0 + lane);
    const float wgt = (my == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(my - M);
    float ws = wgt;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ws += __shfl_xor(ws, off);
    den += ws;
    // rounds of 8 slots with all their loads in flight together; a slot past
    // the end or of weight 0 is not read (it may be an empty workgroup's)
    constexpr int kU = 8;
    for (int u = 0; u < cnt; u += kU) {
      float v0[kU], v1[kU], wu[kU];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const float wq = __shfl(wgt, min(u + q, 63));
        wu[q] = u + q < cnt ? wq : 0.0f;
        const int64_t at = (int64_t)(s0 + u + q) * pstride;
        v0[q] = wu[q] != 0.0f ? pa[at + lane] : 0.0f;
        v1[q] = wu[q] != 0.0f ? pa[at + lane + 64] : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        y0 += wu[q] * v0[q];
        y1 += wu[q] * v1[q];
      }
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

hipError_t launch_merge_wave(const WaveMergeArgs& a, hipStream_t stream) {
  const int units = a.batch * a.num_q_heads;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_wave_kernel, dim3((units + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tq
