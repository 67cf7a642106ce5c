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
//          v_mfma_f32_16x16x16_f16: A = dequantised values (16 dims x 16
//          tokens), B = weights, again [w_hi | w_lo] in the columns for G <= 8.
// Lane layout (l = lane, n = l & 15, c = l >> 4):
//  K loads  token n, dims 32c..32c+31 (4*KB contiguous bytes of its row);
//  V loads  tokens 4c..4c+3, dims 8n..8n+7 (VB bytes of each row);
//  scores   tokens 4c+r (r = 0..3), column n;
//  acc      column n, dims 32c + 8r + blk (blk = 0..7).
// Dequantisation reads LDS pair tables: row p = i0 | i1 << b holds the fp16
// pair (c[i0], c[i1]) replicated once per lane of a half-wave (bank-conflict
// free), hi part then lo part.

#include "tq_internal.h"
#include "tq_device.h"

namespace tq {

// ---------------------------------------------------------------------------
// Replicated pair tables.  Row r of a b-bit table is at r << kShift; replica
// k (k = lane & (kRep - 1)) of the hi pair at +4k, of the lo pair at
// +kLoOff + 4k.
template <int B>
struct PairTable {
  static constexpr int kRows = 1 << (2 * B);
  static constexpr int kRep = (B == 5) ? 4 : 32;
  static constexpr int kShift = (B == 5) ? 5 : 8;
  static constexpr int kStride = 1 << kShift;  // = 8 * kRep
  static constexpr int kBytes = kRows * kStride;
  static constexpr int kLoOff = 4 * kRep;
};

template <int B>
__device__ __forceinline__ void fill_pair_table(uint8_t* base, const float* cent) {
  using T = PairTable<B>;
  constexpr int kQuads = T::kBytes / 16;  // 4 replicas per 16-byte store
  for (int i = threadIdx.x; i < kQuads; i += blockDim.x) {
    const int word = 4 * i;
    const int row = word / (2 * T::kRep);
    const bool lo = (word % (2 * T::kRep)) >= T::kRep;
    const float c0 = cent[row & ((1 << B) - 1)], c1 = cent[row >> B];
    const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
    const uint32_t v = lo ? pack_half2((_Float16)(c0 - (float)h0), (_Float16)(c1 - (float)h1)) : pack_half2(h0, h1);
    *reinterpret_cast<u32x4*>(base + 4 * word) = u32x4{v, v, v, v};
  }
}

// 2B-bit field k of a little-endian bit stream held in words w[]
template <int B>
__device__ __forceinline__ uint32_t pair_field(const uint32_t* w, int k) {
  constexpr int W = 2 * B;
  const int pos = W * k;
  const int wi = pos >> 5, sh = pos & 31;
  uint32_t v = w[wi] >> sh;
  if (sh + W > 32) v |= w[wi + 1] << (32 - sh);
  return v & ((1u << W) - 1u);
}

// LDS byte address (within the table) of the hi pair for pair k
template <int B>
__device__ __forceinline__ uint32_t pair_addr(const uint32_t* w, int k, uint32_t lane_off) {
  if constexpr (B == 4) {
    // byte k of the stream, moved to bits 8..15 next to the lane offset
    return __builtin_amdgcn_perm(w[k >> 2], lane_off, 0x0c0c0000u | ((4u + (uint32_t)(k & 3)) << 8));
  } else {
    return (pair_field<B>(w, k) << PairTable<B>::kShift) | lane_off;
  }
}

__device__ __forceinline__ uint32_t lds_u32(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const uint32_t*>(base + off);
}

template <int QT>
__device__ __forceinline__ float load_q(const void* q, int64_t i) {
  if constexpr (QT == 0) return static_cast<const float*>(q)[i];
  else if constexpr (QT == 1) return (float)static_cast<const _Float16*>(q)[i];
  else return bf16_to_f32(static_cast<const uint16_t*>(q)[i]);
}

__device__ __forceinline__ float row_ror8(float v) {  // lane n <-> n ^ 8 inside a 16-lane row
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t ld_u32(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ float ld_f32(const uint8_t* p) { return *reinterpret_cast<const float*>(p); }

// one page of one KV head, as loaded by one lane
template <int KB, int VB>
struct PageRegs {
  uint32_t kw[KB];
  float nk[4];
  uint32_t vw[4];
  uint32_t vw2[4];  // second word for 3- and 5-bit values
  float nv[4];
};

constexpr int kMaxWaves = 8;

template <int KB, int VB, int QT, bool PACK>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 8))) void decode_split_kernel(DecodeArgs a) {
  using KT = PairTable<KB>;
  using VT = PairTable<VB>;
  constexpr bool kShareV = (KB == VB);
  constexpr int kVBase = 0;
  constexpr int kKBase = kShareV ? 0 : VT::kBytes;
  constexpr int kTabBytes = kKBase + KT::kBytes;
  constexpr int kMergeBytes = kMaxWaves * 16 * (kHeadDim + 2) * 4;
  constexpr int kLds = kTabBytes > kMergeBytes ? kTabBytes : kMergeBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];

  const int S = a.num_splits;
  const int unit = blockIdx.x;
  const int s = unit % S;
  const int hg = (unit / S) % a.head_groups;
  const int b = unit / (S * a.head_groups);
  const int L = a.seq_lens[b];
  const int npages = (L + kBlockSize - 1) / kBlockSize;
  const int p0 = s * a.pages_per_split;
  if (p0 >= npages) return;  // the whole workgroup leaves together
  const int p1 = min(p0 + a.pages_per_split, npages);

  fill_pair_table<KB>(lds + kKBase, a.k_cent);
  if constexpr (!kShareV) fill_pair_table<VB>(lds + kVBase, a.v_cent);
  __syncthreads();

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int gl = wave % a.heads_per_wg;
  const int st = wave / a.heads_per_wg;
  const int g = hg * a.heads_per_wg + gl;
  const int n = lane & 15;
  const int c = lane >> 4;
  const int G = a.group;
  const int span = p1 - p0;
  const int nw = span > st ? (span - st + a.streams - 1) / a.streams : 0;

  // ---- rotated, scaled query in the B-operand layout --------------------
  // lane (n, c) holds dims 32c..32c+31 of column n; PACK: columns 0..7 hold
  // q_hi of heads 0..7 of the group, columns 8..15 their q_lo.
  half8 qb[4];
  half8 qb_lo[PACK ? 1 : 4];
  float q_unscale;  // scores come out multiplied by 1 / q_unscale
  {
    const int hq = PACK ? (n & 7) : n;
    const bool has = hq < G;
    // columns past the group read head 0 of the group and are zeroed
    const int64_t qoff = ((int64_t)b * a.num_q_heads + (int64_t)g * G + (has ? hq : 0)) * kHeadDim + 32 * c;
    float x[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) x[j] = load_q<QT>(a.q, qoff + j);
#pragma unroll
    for (int j = 0; j < 32; ++j) x[j] = has ? x[j] : 0.0f;
    const uint32_t sw = a.sign_bits[c];
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
    for (int j = 0; j < 32; ++j) {
      const float p = __shfl_xor(x[j], 16);
      x[j] = (c & 1) ? p - x[j] : x[j] + p;
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float p = __shfl_xor(x[j], 32);
      x[j] = (c & 2) ? p - x[j] : x[j] + p;
    }
    // power-of-two scale that puts the head's largest coordinate near 2^10,
    // so the fp16 hi/lo halves keep their precision for any query magnitude
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, __builtin_fabsf(x[j] * a.q_scale));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    int qe = 0;
    (void)__builtin_frexpf(amax, &qe);
    if (!(amax > 0.0f) || !(amax < __builtin_inff())) qe = 11;
    const float up = __builtin_ldexpf(a.q_scale, 11 - qe);
    q_unscale = __builtin_ldexpf(1.0f, qe - 11);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = x[8 * m + j] * up;
        const _Float16 hi = (_Float16)v;
        const _Float16 lo = (_Float16)(v - (float)hi);
        if constexpr (PACK) {
          qb[m][j] = (n < 8) ? hi : lo;
        } else {
          qb[m][j] = hi;
          qb_lo[m][j] = lo;
        }
      }
  }

  // ---- per-lane byte offsets inside a page --------------------------------
  const int k_tok = a.num_kv_heads * a.k_row_bytes;  // bytes between tokens
  const int v_tok = a.num_kv_heads * a.v_row_bytes;
  const int k_idx_off = n * k_tok + g * a.k_row_bytes + 4 * KB * c;
  const int k_norm_off = 4 * c * k_tok + g * a.k_row_bytes + a.k_row_bytes - 4;  // + r * k_tok
  const int v_byte = n * VB;
  const int v_row = 4 * c * v_tok + g * a.v_row_bytes;                            // + j * v_tok
  const int v_dat_off = v_row + ((VB == 3 || VB == 5) ? (v_byte & ~3) : v_byte);
  const int v_norm_off = v_row + a.v_row_bytes - 4;
  const uint32_t v_shift = 8u * (uint32_t)(v_byte & 3);
  const uint32_t k_lane = (uint32_t)(lane & (KT::kRep - 1)) * 4u;
  const uint32_t v_lane = (uint32_t)(lane & (VT::kRep - 1)) * 4u;
  const uint8_t* k_tab = lds + kKBase;
  const uint8_t* v_tab = kShareV ? (lds + kKBase) : (lds + kVBase);

  // ---- block ids: lane j holds the id of this wave's page 64*chunk + j ----
  const int32_t* bt = a.block_table + (int64_t)b * a.max_blocks_per_seq + p0 + st;
  const int stride_p = a.streams;
  auto load_ids = [&](int chunk) -> int {
    const int i = 64 * chunk + lane;
    return i < nw ? bt[(int64_t)i * stride_p] : 0;
  };
  int ids0 = load_ids(0);
  int ids1 = nw > 64 ? load_ids(1) : 0;
  int id_chunk = 0;
  auto block_of = [&](int i) -> int {
    if ((i >> 6) != id_chunk) {  // once every 64 pages, uniform
      ids0 = ids1;
      ++id_chunk;
      ids1 = (nw > 64 * (id_chunk + 1)) ? load_ids(id_chunk + 1) : 0;
    }
    return __builtin_amdgcn_readlane(ids0, i & 63);
  };

  auto load_page = [&](PageRegs<KB, VB>& P, int blk) {
    const uint8_t* kp = a.k_pages + (int64_t)blk * a.k_page_bytes;
    const uint8_t* vp = a.v_pages + (int64_t)blk * a.v_page_bytes;
#pragma unroll
    for (int i = 0; i < KB; ++i) P.kw[i] = ld_u32(kp + k_idx_off + 4 * i);
#pragma unroll
    for (int r = 0; r < 4; ++r) P.nk[r] = ld_f32(kp + r * k_tok + k_norm_off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint8_t* vr = vp + j * v_tok;
      if constexpr (VB == 2) {
        P.vw[j] = *reinterpret_cast<const uint16_t*>(vr + v_dat_off);
      } else {
        P.vw[j] = ld_u32(vr + v_dat_off);
        if constexpr (VB == 3 || VB == 5) P.vw2[j] = ld_u32(vr + v_dat_off + 4);
      }
      P.nv[j] = ld_f32(vr + v_norm_off);
    }
  };

  floatx4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -__builtin_inff();
  float l_part = 0.0f;

  auto compute_page = [&](const PageRegs<KB, VB>& P, int i) {
    const int tok0 = (p0 + st + stride_p * i) * kBlockSize + 4 * c;
    // -- scores
    floatx4 sc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t ah[4], al[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t ad = pair_addr<KB>(P.kw, 4 * m + k, k_lane);
        ah[k] = lds_u32(k_tab, ad);
        al[k] = lds_u32(k_tab + KT::kLoOff, ad);
      }
      const half8 Ahi = __builtin_bit_cast(half8, u32x4{ah[0], ah[1], ah[2], ah[3]});
      const half8 Alo = __builtin_bit_cast(half8, u32x4{al[0], al[1], al[2], al[3]});
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, qb[m], sc, 0, 0, 0);
      if constexpr (!PACK) sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, qb_lo[m], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, qb[m], sc, 0, 0, 0);
    }
    // -- softmax bookkeeping (log2 domain)
    float sv[4];
    float pmax = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float full = PACK ? sc[r] + row_ror8(sc[r]) : sc[r];
      const bool valid = tok0 + r < L;
      sv[r] = valid ? full * (P.nk[r] * q_unscale) : -__builtin_inff();
      int e = 0;
      (void)__builtin_frexpf(P.nv[r], &e);
      const float ev = (P.nv[r] > 0.0f) ? (float)max(e, -64) : -64.0f;
      pmax = fmaxf(pmax, sv[r] + ev);
    }
    pmax = fmaxf(pmax, __shfl_xor(pmax, 16));
    pmax = fmaxf(pmax, __shfl_xor(pmax, 32));
    if (__builtin_amdgcn_ballot_w64(pmax > m_ref + 8.0f) != 0) {
      const float m_new = fmaxf(m_ref, pmax);
      const float alpha = (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] *= alpha;
      m_ref = m_new;
    }
    half4 W, Wlo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool valid = tok0 + r < L;
      const float pr = valid ? __builtin_amdgcn_exp2f(sv[r] - m_ref) : 0.0f;
      l_part += pr;
      const float wv = valid ? pr * P.nv[r] : 0.0f;
      const _Float16 hi = (_Float16)wv;
      const _Float16 lo = (_Float16)(wv - (float)hi);
      if constexpr (PACK) {
        W[r] = (n < 8) ? hi : lo;
      } else {
        W[r] = hi;
        Wlo[r] = lo;
      }
    }
    // -- values
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t L4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t words[2];
        if constexpr (VB == 3 || VB == 5) {
          const uint64_t all = ((((uint64_t)P.vw2[j]) << 32) | P.vw[j]) >> v_shift;
          words[0] = (uint32_t)all;
          words[1] = (uint32_t)(all >> 32);
        } else {
          words[0] = P.vw[j];
          words[1] = 0;
        }
        L4[j] = lds_u32(v_tab, pair_addr<VB>(words, k, v_lane));
      }
      // block 2k takes the low halves (dim 8n+2k), block 2k+1 the high halves
      const uint32_t lo01 = __builtin_amdgcn_perm(L4[1], L4[0], 0x05040100u);
      const uint32_t lo23 = __builtin_amdgcn_perm(L4[3], L4[2], 0x05040100u);
      const uint32_t hi01 = __builtin_amdgcn_perm(L4[1], L4[0], 0x07060302u);
      const uint32_t hi23 = __builtin_amdgcn_perm(L4[3], L4[2], 0x07060302u);
      const half4 Ae = __builtin_bit_cast(half4, (uint64_t)lo01 | ((uint64_t)lo23 << 32));
      const half4 Ao = __builtin_bit_cast(half4, (uint64_t)hi01 | ((uint64_t)hi23 << 32));
      acc[2 * k] = __builtin_amdgcn_mfma_f32_16x16x16f16(Ae, W, acc[2 * k], 0, 0, 0);
      acc[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(Ao, W, acc[2 * k + 1], 0, 0, 0);
      if constexpr (!PACK) {
        acc[2 * k] = __builtin_amdgcn_mfma_f32_16x16x16f16(Ae, Wlo, acc[2 * k], 0, 0, 0);
        acc[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(Ao, Wlo, acc[2 * k + 1], 0, 0, 0);
      }
    }
  };

  // ---- page loop, one page of prefetch ------------------------------------
  if (nw > 0) {
    PageRegs<KB, VB> A, Bq;
    load_page(A, block_of(0));
    for (int i = 0; i < nw; i += 2) {
      load_page(Bq, block_of(min(i + 1, nw - 1)));
      compute_page(A, i);
      if (i + 1 >= nw) break;
      load_page(A, block_of(min(i + 2, nw - 1)));
      compute_page(Bq, i + 1);
    }
  }

  // ---- fold the lo columns, finish the split --------------------------------
  if constexpr (PACK) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[q][r] += row_ror8(acc[q][r]);
    }
  }
  float l_tot = l_part + __shfl_xor(l_part, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const int hq = PACK ? (n & 7) : n;
  const bool owner = (PACK ? n < 8 : true) && hq < G;

  if (a.streams == 1) {
    if (owner) {
      const int h = g * G + hq;
      const int64_t slot = ((int64_t)b * a.num_q_heads + h) * S + s;
      const float inv = 1.0f / l_tot;
      float* dst = a.part_acc + slot * kHeadDim + 32 * c;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        floatx4 v0, v1;
        v0.x = acc[0][r] * inv; v0.y = acc[1][r] * inv; v0.z = acc[2][r] * inv; v0.w = acc[3][r] * inv;
        v1.x = acc[4][r] * inv; v1.y = acc[5][r] * inv; v1.z = acc[6][r] * inv; v1.w = acc[7][r] * inv;
        *reinterpret_cast<floatx4*>(dst + 8 * r) = v0;
        *reinterpret_cast<floatx4*>(dst + 8 * r + 4) = v1;
      }
      if (c == 0) a.part_lse[slot] = m_ref + __builtin_log2f(l_tot);
    }
    return;
  }

  // several streams per head: merge them through LDS (the tables are dead)
  __syncthreads();
  float* m_buf = reinterpret_cast<float*>(lds);                   // [waves][16]
  float* l_buf = m_buf + kMaxWaves * 16;                          // [waves][16]
  float* a_buf = l_buf + kMaxWaves * 16;                          // [waves][16][128]
  if (c == 0) {
    m_buf[wave * 16 + n] = m_ref;
    l_buf[wave * 16 + n] = l_tot;
  }
  {
    float* dst = a_buf + (wave * 16 + n) * kHeadDim + 32 * c;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < 8; ++q) dst[8 * r + q] = acc[q][r];
  }
  __syncthreads();
  if (st != 0 || !owner) return;
  float M = -__builtin_inff();
  for (int t = 0; t < a.streams; ++t) M = fmaxf(M, m_buf[(t * a.heads_per_wg + gl) * 16 + n]);
  float lsum = 0.0f;
  float out[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) out[j] = 0.0f;
  for (int t = 0; t < a.streams; ++t) {
    const int wv = t * a.heads_per_wg + gl;
    const float mt = m_buf[wv * 16 + n];
    const float sc = (mt == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mt - M);
    lsum += sc * l_buf[wv * 16 + n];
    const float* src = a_buf + (wv * 16 + n) * kHeadDim + 32 * c;
#pragma unroll
    for (int j = 0; j < 32; ++j) out[j] += sc * src[j];
  }
  const int h = g * G + hq;
  const int64_t slot = ((int64_t)b * a.num_q_heads + h) * S + s;
  const float inv = 1.0f / lsum;
  float* dst = a.part_acc + slot * kHeadDim + 32 * c;
#pragma unroll
  for (int j = 0; j < 32; j += 4) {
    floatx4 v;
    v.x = out[j] * inv; v.y = out[j + 1] * inv; v.z = out[j + 2] * inv; v.w = out[j + 3] * inv;
    *reinterpret_cast<floatx4*>(dst + j) = v;
  }
  if (c == 0) a.part_lse[slot] = M + __builtin_log2f(lsum);
}

template <int KB, int VB, bool PACK>
static hipError_t launch_decode_kvp(const DecodeArgs& a, int qt, hipStream_t st) {
  const long long units = (long long)a.batch * a.head_groups * a.num_splits;
  const dim3 grid((unsigned)units), block(64 * a.heads_per_wg * a.streams);
  if (qt == 0)
    hipLaunchKernelGGL((decode_split_kernel<KB, VB, 0, PACK>), grid, block, 0, st, a);
  else if (qt == 1)
    hipLaunchKernelGGL((decode_split_kernel<KB, VB, 1, PACK>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<KB, VB, 2, PACK>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <int KB, int VB>
static hipError_t launch_decode_kv(const DecodeArgs& a, int qt, hipStream_t st) {
  return a.group <= 8 ? launch_decode_kvp<KB, VB, true>(a, qt, st) : launch_decode_kvp<KB, VB, false>(a, qt, st);
}

template <int KB>
static hipError_t launch_decode_k(const DecodeArgs& a, int qt, int vb, hipStream_t st) {
  switch (vb) {
    case 2: return launch_decode_kv<KB, 2>(a, qt, st);
    case 3: return launch_decode_kv<KB, 3>(a, qt, st);
    case 4: return launch_decode_kv<KB, 4>(a, qt, st);
    case 5: return launch_decode_kv<KB, 5>(a, qt, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int q_dtype, int k_bits, int v_bits, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  switch (k_bits) {
    case 2: return launch_decode_k<2>(a, q_dtype, v_bits, stream);
    case 3: return launch_decode_k<3>(a, q_dtype, v_bits, stream);
    case 4: return launch_decode_k<4>(a, q_dtype, v_bits, stream);
    case 5: return launch_decode_k<5>(a, q_dtype, v_bits, stream);
  }
  return hipErrorInvalidValue;
}

// ===========================================================================
// Merge: one wave per (b, h).  Combines the splits' normalised rotated sums by
// their log2-sum-exp2, divides the value scale out, applies the inverse
// rotation s * H y / sqrt(128) and writes fp32 out.  Lane l owns dims l and
// l + 64; lane s holds the weight of split s (at most 64 splits).
// ===========================================================================
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= a.batch * a.num_q_heads) return;
  const int b = unit / a.num_q_heads;
  const int L = a.seq_lens[b];
  float* o = a.out + (int64_t)unit * kHeadDim;
  if (L <= 0) {
    o[lane] = 0.0f;
    o[lane + 64] = 0.0f;
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
  int sidx = 0;
  for (; sidx + 4 <= ns; sidx += 4) {
    float v0[4], v1[4], w4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v0[u] = pa[(int64_t)(sidx + u) * kHeadDim + lane];
      v1[u] = pa[(int64_t)(sidx + u) * kHeadDim + lane + 64];
      w4[u] = __shfl(wgt, sidx + u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      y0 += w4[u] * v0[u];
      y1 += w4[u] * v1[u];
    }
  }
  for (; sidx < ns; ++sidx) {
    const float wv = __shfl(wgt, sidx);
    y0 += wv * pa[(int64_t)sidx * kHeadDim + lane];
    y1 += wv * pa[(int64_t)sidx * kHeadDim + lane + 64];
  }
  const float inv = 1.0f / den;
  y0 *= inv;
  y1 *= inv;
  // H over 128 points: stage 64 inside the lane, stages 1..32 across lanes
  {
    const float u = y0, v = y1;
    y0 = u + v;
    y1 = u - v;
  }
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    const float q0 = __shfl_xor(y0, h), q1 = __shfl_xor(y1, h);
    y0 = (lane & h) ? q0 - y0 : y0 + q0;
    y1 = (lane & h) ? q1 - y1 : y1 + q1;
  }
  const float s0 = ((a.sign_bits[lane >> 5] >> (lane & 31)) & 1u) ? -1.0f : 1.0f;
  const float s1 = ((a.sign_bits[2 + (lane >> 5)] >> (lane & 31)) & 1u) ? -1.0f : 1.0f;
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
