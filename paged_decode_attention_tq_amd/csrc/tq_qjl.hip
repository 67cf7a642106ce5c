// Inner-product scores over prod key rows for gfx950: for every query head
// and every key of its sequence, n (<q~, c[idx]> + gamma sqrt(pi / 2) / d
// <S q~, z>), q~ = rht(q).
//
// Sources: TurboQuant docs, "vLLM Reference Audit", File Map rows "MSE and
// QJL codecs" (TurboQuantProd: indices, norms, signs) and "packed score
// kernel" (score-only diagnostic over packed key rows); Feature Checklist row
// "QJL residual".  The estimator is the published inner-product quantiser's:
// the (b-1)-bit MSE part plus the residual's 1-bit sketch, unbiased over the
// draw of the Gaussian matrix S.

#include "tq_internal.h"
#include "tq_device.h"
#include "tq_decode_common.h"

namespace tq {

namespace {

__device__ __forceinline__ float load_q1(const void* base, int64_t elem, int dt) {
  if (dt == 0) return static_cast<const float*>(base)[elem];
  const uint16_t u = static_cast<const uint16_t*>(base)[elem];
  return dt == 1 ? (float)__builtin_bit_cast(_Float16, u) : bf16_to_f32(u);
}

template <int XOR>
__device__ __forceinline__ float lane_xor(float v) {
  return __shfl_xor(v, XOR);
}

}  // namespace

// One wave per (b, h): q~ = H (s * q) / sqrt(128) (lane l holds dims l and
// l + 64), then S q~ (lane l forms outputs l and l + 64 from q~ in LDS).
__global__ __launch_bounds__(256) void prod_query_kernel(ProdScoreArgs a) {
  __shared__ float qs[4][kHeadDim];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t unit = (int64_t)blockIdx.x * 4 + wave;
  const bool live = unit < (int64_t)a.batch * a.num_q_heads;
  const int64_t u = live ? unit : 0;
  float y0 = load_q1(a.q, u * kHeadDim + lane, a.q_dtype);
  float y1 = load_q1(a.q, u * kHeadDim + lane + 64, a.q_dtype);
  const uint32_t s0 = (pick4(a.sign_bits, lane >> 5) >> (lane & 31)) & 1u;
  const uint32_t s1 = (pick4(a.sign_bits, 2 + (lane >> 5)) >> (lane & 31)) & 1u;
  y0 = s0 ? -y0 : y0;
  y1 = s1 ? -y1 : y1;
  {
    const float p = y0, r = y1;
    y0 = p + r;
    y1 = p - r;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const float o0 = __shfl_xor(y0, m), o1 = __shfl_xor(y1, m);
    y0 = (lane & m) ? o0 - y0 : y0 + o0;
    y1 = (lane & m) ? o1 - y1 : y1 + o1;
  }
  y0 *= 0.08838834764831845f;  // 1 / sqrt(128)
  y1 *= 0.08838834764831845f;
  qs[wave][lane] = y0;
  qs[wave][lane + 64] = y1;
  __syncthreads();
  float a0 = 0.0f, a1 = 0.0f;
  const float* r0 = a.sketch + (int64_t)lane * kHeadDim;
  const float* r1 = a.sketch + (int64_t)(lane + 64) * kHeadDim;
  for (int j = 0; j < kHeadDim; j += 4) {
    const floatx4 v = *reinterpret_cast<const floatx4*>(&qs[wave][j]);
    const floatx4 w0 = *reinterpret_cast<const floatx4*>(r0 + j);
    const floatx4 w1 = *reinterpret_cast<const floatx4*>(r1 + j);
    a0 = fmaf(w0[0], v[0], fmaf(w0[1], v[1], fmaf(w0[2], v[2], fmaf(w0[3], v[3], a0))));
    a1 = fmaf(w1[0], v[0], fmaf(w1[1], v[1], fmaf(w1[2], v[2], fmaf(w1[3], v[3], a1))));
  }
  if (!live) return;
  a.qr[u * kHeadDim + lane] = y0;
  a.qr[u * kHeadDim + lane + 64] = y1;
  a.sq[u * kHeadDim + lane] = a0;
  a.sq[u * kHeadDim + lane + 64] = a1;
}

// Scores on MFMA.  For the 16 tokens t of one page and one KV head, with up
// to 8 query heads h of its group,
//   S[t, h] = n_t (<c_t, q~_h> + gamma_t sqrt(pi / 2) / 128 <z_t, (S q~)_h>)
// is two dense contractions over the 128 coordinates: A = the tokens'
// centroid rows c_t (fp16 hi and lo from a pair table, side by side in the
// k-slots, each against the same query value) or sign rows z_t (exact +-1),
// B = the heads' q~ or S q~, split into fp16 hi (columns 0..7) and lo
// (columns 8..15) after a power-of-two scaling per head.  Columns h and
// h + 8 of the product sum to the fp32-accurate inner product.
//
// MFMA layout (v_mfma_f32_16x16x32_f16): lane l = 16 c + n holds A row n
// (token n) and B column n at k-slots 8 c .. 8 c + 7, so lane (n, c) reads
// row n's index words and sign word for coordinates 32 c .. 32 c + 31 and
// supplies those coordinates' A and B values.  The result sits in lane
// (n, c) as tokens 4 c .. 4 c + 3 of column n.
//
// Grid: one workgroup of 4 waves per (slab = sequence and chunk of pages,
// group of H KV heads, chunk of 8 query heads).  Wave w takes KV head w % H
// of the group and every P-th page of the chunk from page w / H (P = 4 / H
// phases), so with H > 1 the waves read the neighbouring rows of a page's KV
// heads together and use whole cache lines; with H = 1 each wave takes every
// fourth page of one head.  Workgroups of one slab have blockIdx congruent
// mod 8, i.e. run on one XCD and share its L2 for the page lines that hold
// several KV heads' rows.  A wave walks its pages in batches of four whose
// row fields are loaded while the previous batch is computed.

constexpr float kCentScale = 16.0f;  // the host passes centroids times 16 (exact)

// Sign nibble table: entry e (4 coordinates, bit j for coordinate j) holds
// fp16 (z0, z1), (z2, z3), z = +1 for a set bit, else -1; 32 replicas of 8
// bytes at (e << 8) + 8 (lane & 31), so a half-wave's reads hit distinct banks.
constexpr int kNibBytes = 16 * 256;
constexpr int kMaxChunkPages = 128;  // pages per workgroup at most (the host's choice)

// fp16 part (hi, or the rounding residual lo) of the 32 scaled values of v
// as 16 pairs
__device__ __forceinline__ void split_pairs(const float (&v)[32], float s, bool lo, uint32_t (&out)[16]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float x0 = v[2 * j] * s, x1 = v[2 * j + 1] * s;
    const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
    out[j] = lo ? pack_half2((_Float16)(x0 - (float)h0), (_Float16)(x1 - (float)h1)) : pack_half2(h0, h1);
  }
}

template <int BITS>
__global__ __launch_bounds__(256) void prod_scores_kernel(ProdScoreArgs a) {
  constexpr int MB = BITS - 1;
  using T = PairTable<MB>;
  __shared__ __align__(16) uint8_t lds[T::kBytes + kNibBytes];
  __shared__ int32_t bids[kMaxChunkPages];  // the chunk's block ids (-1 past the sequence)
  uint8_t* const ptab = lds;
  uint8_t* const ntab = lds + T::kBytes;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: page loop and block ids in scalar registers
  const int n = lane & 15, c = lane >> 4;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int nhc = (G + 7) / 8;
  const int ngroups = a.num_kv_heads / a.head_group;
  const int inner = ngroups * nhc;
  const int r8 = (int)(blockIdx.x >> 3);
  const int64_t slab = (int64_t)(r8 / inner) * 8 + (blockIdx.x & 7);
  if (slab >= (int64_t)a.batch * a.chunks) return;  // uniform per workgroup
  const int hc = (r8 % inner) / ngroups;
  // wave: KV head g of the workgroup's group, page phase ph (pages ph, ph + P, ...)
  const int ph = wave / a.head_group;
  const bool active = ph < a.phases;
  const int g = ((r8 % inner) % ngroups) * a.head_group + wave % a.head_group;
  const int b = (int)(slab / a.chunks), ck = (int)(slab % a.chunks);

  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  const int pg_first = ck * a.chunk_pages;
  if (tid < a.chunk_pages) {
    const int pg = pg_first + tid;
    bids[tid] = pg * kBlockSize < L ? a.block_table[(int64_t)b * a.max_blocks_per_seq + pg] : -1;
  }
  fill_pair_table_flat<MB>(ptab, a.cent, tid, 256);
  {
    const int e = tid >> 4;
    auto z = [&](int j) { return ((e >> j) & 1) ? 0x3C00u : 0xBC00u; };
    const uint32_t w0 = z(0) | z(1) << 16, w1 = z(2) | z(3) << 16;
    *reinterpret_cast<u32x4*>(ntab + 16 * tid) = u32x4{w0, w1, w0, w1};
  }

  // B fragments: this lane's head (column n & 7 of the chunk), coordinates
  // 32 c .. 32 c + 31, hi (n < 8) or lo (n >= 8) parts
  const int hl = hc * 8 + (n & 7);
  const bool hv = hl < G;
  const int64_t hq = (int64_t)b * a.num_q_heads + g * G + (hv ? hl : 0);
  uint32_t bq[16], bs[16];
  float inv_q, inv_s;
  {
    float v[32];
    float mx = 0.0f;
    const float* src = a.qr + hq * kHeadDim + 32 * c;
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
      const floatx4 t = hv ? *reinterpret_cast<const floatx4*>(src + j) : floatx4{0.f, 0.f, 0.f, 0.f};
      v[j] = t[0], v[j + 1] = t[1], v[j + 2] = t[2], v[j + 3] = t[3];
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) mx = fmaxf(mx, __builtin_fabsf(v[j]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float sc = pow2_scale(mx);
    split_pairs(v, sc, n >= 8, bq);
    inv_q = 1.0f / (sc * kCentScale);
    src = a.sq + hq * kHeadDim + 32 * c;
    mx = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
      const floatx4 t = hv ? *reinterpret_cast<const floatx4*>(src + j) : floatx4{0.f, 0.f, 0.f, 0.f};
      v[j] = t[0], v[j + 1] = t[1], v[j + 2] = t[2], v[j + 3] = t[3];
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) mx = fmaxf(mx, __builtin_fabsf(v[j]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    sc = pow2_scale(mx);
    split_pairs(v, sc, n >= 8, bs);
    inv_s = 1.0f / sc;
  }
  // the MFMA operands: centroid MFMA j repeats query pairs 2j and 2j + 1 (one
  // for the hi, one for the lo part of each centroid pair); sign MFMA m takes
  // pairs 4m .. 4m + 3
  half8 Bq[8], Bs[4];
#pragma unroll
  for (int j = 0; j < 8; ++j) Bq[j] = __builtin_bit_cast(half8, u32x4{bq[2 * j], bq[2 * j], bq[2 * j + 1], bq[2 * j + 1]});
#pragma unroll
  for (int m = 0; m < 4; ++m) Bs[m] = __builtin_bit_cast(half8, u32x4{bs[4 * m], bs[4 * m + 1], bs[4 * m + 2], bs[4 * m + 3]});
  const float zq = inv_s * 0.009791516697777346f;  // sqrt(pi / 2) / 128 over the S q~ scale
  __syncthreads();
  if (!active) return;  // uniform per wave; no barrier follows

  const uint32_t lane_off = 8u * (uint32_t)(lane & 31);
  // scores of the chunk's heads through one buffer descriptor (the host
  // keeps 8 rows under 2^31 bytes); lanes that store nothing address past it
  const int nh = min(8, G - hc * 8);
  const __amdgpu_buffer_rsrc_t rso = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.scores + ((int64_t)b * a.num_q_heads + g * G + hc * 8) * a.max_seq_len), 0,
      (int)(nh * a.max_seq_len * 4), 0x00020000);
  const bool store = hv && n < 8;
  const uint32_t so_lane = store ? (uint32_t)(n * a.max_seq_len + 4 * c) * 4u : 0x80000000u;
  const bool vec4 = a.vec_store != 0;
  const int pg_end = min((ck + 1) * a.chunk_pages, (a.max_seq_len + kBlockSize - 1) / kBlockSize);
  // a page's row fields for this lane, through a buffer descriptor of the
  // page: a token past the sequence lies past the buffer's end and a block
  // id outside the pages (or a page past the sequence or the chunk) gets a
  // zero-sized buffer, both of which read zeros (norm 0: score 0).  The
  // loads are unconditional, so no register is cleared while the other
  // batch's loads are in flight.
  struct Rows {
    uint32_t w[MB];
    uint32_t zw;
    float nrm, gam;
  };
  const uint32_t row_off = (uint32_t)((n * a.num_kv_heads + g) * a.row_bytes);  // inside a page (< 2^30)
  auto fetch = [&](int pg, Rows& d) {
    const int blk = __builtin_amdgcn_readfirstlane(pg < pg_end ? bids[pg - pg_first] : -1);
    // the buffer ends after the sequence's last token of the page: the rows
    // of later tokens lie past it
    const int live = min(kBlockSize, L - pg * kBlockSize);
    const bool page_ok = blk >= 0 && blk < a.num_blocks && live > 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.pages + (page_ok ? (int64_t)blk * a.page_bytes : 0)), 0,
        page_ok ? live * a.num_kv_heads * a.row_bytes : 0, 0x00020000);
    const uint32_t off = row_off;
    const uint32_t wo = off + 4u * (uint32_t)(MB * c);
    if constexpr (MB == 1) {
      d.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, wo, 0, 0);
    } else if constexpr (MB == 2) {
      const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, wo, 0, 0));
      d.w[0] = v.x, d.w[1] = v.y;
    } else if constexpr (MB == 3) {
      typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
      const u32x3 v = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(rs, wo, 0, 0));
      d.w[0] = v.x, d.w[1] = v.y, d.w[2] = v.z;
    } else {
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, wo, 0, 0));
      d.w[0] = v.x, d.w[1] = v.y, d.w[2] = v.z, d.w[3] = v.w;
    }
    d.zw = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4u * (uint32_t)(4 * MB + 1 + c), 0, 0);
    d.nrm = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off + 16u * MB, 0, 0));
    d.gam = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off + 16u * MB + 20u, 0, 0));
  };
  auto tile = [&](int pg, const Rows& d) {
    const int t0 = pg * kBlockSize;
    float res[4] = {0.f, 0.f, 0.f, 0.f};
    if (t0 < L) {  // uniform per wave
      // centroids: MFMA j takes pairs 2j, 2j + 1 of the lane's 16, A = the two
      // table entries as read, (hi, lo) of each, against the query pairs
      // repeated; sign rows: MFMA m takes coordinates 8m .. 8m + 7
      floatx4 am = {0.f, 0.f, 0.f, 0.f}, az = am;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = 2 * m + h;
          const u32x2 e0 = *reinterpret_cast<const u32x2*>(ptab + pair_addr<MB>(d.w, 2 * j, lane_off));
          const u32x2 e1 = *reinterpret_cast<const u32x2*>(ptab + pair_addr<MB>(d.w, 2 * j + 1, lane_off));
          const half8 A = __builtin_bit_cast(half8, u32x4{e0.x, e0.y, e1.x, e1.y});
          am = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bq[j], am, 0, 0, 0);
        }
        const u32x2 z0 = *reinterpret_cast<const u32x2*>(ntab + ((((d.zw >> (8 * m)) & 15u) << 8) | lane_off));
        const u32x2 z1 = *reinterpret_cast<const u32x2*>(ntab + ((((d.zw >> (8 * m + 4)) & 15u) << 8) | lane_off));
        az = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, u32x4{z0.x, z0.y, z1.x, z1.y}), Bs[m],
                                                    az, 0, 0, 0);
      }
      // tokens past the sequence read norm 0 and score 0
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float tn = __shfl(d.nrm, 4 * c + r), tg = __shfl(d.gam, 4 * c + r);
        const float mse = am[r], zz = az[r];
        const float msum = mse + row_ror8(mse), zsum = zz + row_ror8(zz);
        res[r] = tn * fmaf(tg * zq, zsum, msum * inv_q);
      }
    }
    const int t = t0 + 4 * c;
    if (vec4) {  // uniform; 4 columns at once, none past the row (max_seq_len % 4 == 0)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, floatx4{res[0], res[1], res[2], res[3]}), rso,
                                             t < a.max_seq_len ? so_lane + 4u * (uint32_t)t0 : 0x80000000u, 0, 0);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(res[r]), rso,
                                              t + r < a.max_seq_len ? so_lane + 4u * (uint32_t)(t0 + r) : 0x80000000u,
                                              0, 0);
    }
  };
  // pages pg, pg + P, ... of this wave in batches of four, two batch
  // buffers in turn: a batch's rows are requested while the previous batch
  // is computed
  const int P = a.phases;
  Rows da[4], db[4];
  const int pg0 = pg_first + ph;
#pragma unroll
  for (int u = 0; u < 4; ++u) fetch(pg0 + P * u, da[u]);
  for (int pg = pg0; pg < pg_end; pg += 8 * P) {
#pragma unroll
    for (int u = 0; u < 4; ++u) fetch(pg + P * (4 + u), db[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (pg + P * u < pg_end) tile(pg + P * u, da[u]);  // uniform per wave
    if (pg + 4 * P >= pg_end) break;
#pragma unroll
    for (int u = 0; u < 4; ++u) fetch(pg + P * (8 + u), da[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (pg + P * (4 + u) < pg_end) tile(pg + P * (4 + u), db[u]);
  }
}

hipError_t launch_prod_scores(const ProdScoreArgs& a, int bits, hipStream_t stream) {
  const int64_t heads = (int64_t)a.batch * a.num_q_heads;
  if (heads == 0) return hipSuccess;
  hipLaunchKernelGGL(prod_query_kernel, dim3((unsigned)((heads + 3) / 4)), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_seq_len == 0) return e;
  const int G = a.num_q_heads / a.num_kv_heads, nhc = (G + 7) / 8;
  const int64_t inner = (int64_t)(a.num_kv_heads / a.head_group) * nhc;
  const int64_t slabs = (int64_t)a.batch * a.chunks;
  const int64_t wgs = (slabs + 7) / 8 * 8 * inner;
  if (wgs > 0x7fffffffLL || a.head_group * a.phases > 4 || a.num_kv_heads % a.head_group) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs), block(256);
  switch (bits) {
    case 2: hipLaunchKernelGGL(prod_scores_kernel<2>, grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL(prod_scores_kernel<3>, grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(prod_scores_kernel<4>, grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL(prod_scores_kernel<5>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tq
