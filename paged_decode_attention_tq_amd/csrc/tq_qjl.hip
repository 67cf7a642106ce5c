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

// One workgroup per (sequence, KV head, up to 8 of its query heads, chunk of
// 32 pages): the heads' q~ and S q~ are staged in LDS once, then each wave
// walks 8 of the chunk's pages, a quad per token, lane q holding coordinates
// 32 q .. 32 q + 31 (its index words, its sign word).  A token's centroids
// and signs are decoded once and used for every head.  Every lane runs the
// centroid shuffles; tokens past the sequence give score 0.
constexpr int kScoreHeads = 8;
constexpr int kChunkPages = 32;

template <int BITS>
__global__ __launch_bounds__(256) void prod_scores_kernel(ProdScoreArgs a, int chunks) {
  constexpr int MB = BITS - 1;
  constexpr uint32_t kMask = (1u << MB) - 1;
  __shared__ float qs[kScoreHeads][2][kHeadDim];  // q~ and S q~ per head
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, q = lane & 3;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int nhc = (G + kScoreHeads - 1) / kScoreHeads;
  int64_t unit = blockIdx.x;
  const int ck = (int)(unit % chunks);
  unit /= chunks;
  const int hc = (int)(unit % nhc);
  unit /= nhc;
  const int g = (int)(unit % a.num_kv_heads), b = (int)(unit / a.num_kv_heads);
  const int h0 = g * G + kScoreHeads * hc, nh = min(kScoreHeads, G - kScoreHeads * hc);
  for (int e = threadIdx.x; e < kScoreHeads * kHeadDim; e += 256) {
    const int i = e >> 7, d = e & 127;
    const int64_t at = ((int64_t)b * a.num_q_heads + h0 + min(i, nh - 1)) * kHeadDim + d;
    qs[i][0][d] = a.qr[at];
    qs[i][1][d] = a.sq[at];
  }
  __syncthreads();
  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  const float cl = cent_of_lane<MB>(a.cent, lane & ((1 << MB) - 1));
  for (int pi = wave; pi < kChunkPages; pi += 4) {
    const int page = ck * kChunkPages + pi;
    const int t = page * kBlockSize + (lane >> 2);
    if (page * kBlockSize >= a.max_seq_len) break;  // uniform per wave
    const bool valid = t < L;
    uint32_t w[MB], zw = 0;
    float n = 0.0f, gamma = 0.0f;
#pragma unroll
    for (int k = 0; k < MB; ++k) w[k] = 0;
    if (valid) {
      const int64_t blk = a.block_table[(int64_t)b * a.max_blocks_per_seq + page];
      if (blk >= 0 && blk < a.num_blocks) {
        const uint32_t* row = reinterpret_cast<const uint32_t*>(
            a.pages + blk * a.page_bytes + ((int64_t)(t % kBlockSize) * a.num_kv_heads + g) * a.row_bytes);
#pragma unroll
        for (int k = 0; k < MB; ++k) w[k] = row[MB * q + k];
        zw = row[4 * MB + 1 + q];
        n = __uint_as_float(row[4 * MB]);
        gamma = __uint_as_float(row[4 * MB + 5]);
      }
    }
    float c[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int pos = MB * j;
      uint32_t idx = w[pos >> 5] >> (pos & 31);
      if ((pos & 31) + MB > 32) idx |= w[(pos >> 5) + 1] << (32 - (pos & 31));
      c[j] = __shfl(cl, (int)(idx & kMask));
    }
    const float kq = gamma * 0.009791516697777346f;  // gamma sqrt(pi / 2) / 128
    for (int i = 0; i < nh; ++i) {
      const float* qr = &qs[i][0][32 * q];
      const float* sq = &qs[i][1][32 * q];
      float m0 = 0.0f, m1 = 0.0f, z0 = 0.0f, z1 = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; j += 4) {
        const floatx4 qv = *reinterpret_cast<const floatx4*>(qr + j);
        const floatx4 sv = *reinterpret_cast<const floatx4*>(sq + j);
        m0 = fmaf(c[j], qv[0], fmaf(c[j + 1], qv[1], m0));
        m1 = fmaf(c[j + 2], qv[2], fmaf(c[j + 3], qv[3], m1));
        z0 += __uint_as_float(__float_as_uint(sv[0]) ^ ((~zw >> j) & 1u) << 31) +
              __uint_as_float(__float_as_uint(sv[1]) ^ ((~zw >> (j + 1)) & 1u) << 31);
        z1 += __uint_as_float(__float_as_uint(sv[2]) ^ ((~zw >> (j + 2)) & 1u) << 31) +
              __uint_as_float(__float_as_uint(sv[3]) ^ ((~zw >> (j + 3)) & 1u) << 31);
      }
      float s = n * (m0 + m1) + n * kq * (z0 + z1);
      s += quad_xor<1>(s);
      s += quad_xor<2>(s);
      if (q == 0 && t < a.max_seq_len)
        a.scores[((int64_t)b * a.num_q_heads + h0 + i) * a.max_seq_len + t] = valid ? s : 0.0f;
    }
  }
}

hipError_t launch_prod_scores(const ProdScoreArgs& a, int bits, hipStream_t stream) {
  const int64_t heads = (int64_t)a.batch * a.num_q_heads;
  if (heads == 0) return hipSuccess;
  hipLaunchKernelGGL(prod_query_kernel, dim3((unsigned)((heads + 3) / 4)), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_seq_len == 0) return e;
  const int pages = (a.max_seq_len + kBlockSize - 1) / kBlockSize;
  const int chunks = (pages + kChunkPages - 1) / kChunkPages;
  const int G = a.num_q_heads / a.num_kv_heads, nhc = (G + kScoreHeads - 1) / kScoreHeads;
  const dim3 grid((unsigned)((int64_t)a.batch * a.num_kv_heads * nhc * chunks)), block(256);
  switch (bits) {
    case 2: hipLaunchKernelGGL(prod_scores_kernel<2>, grid, block, 0, stream, a, chunks); break;
    case 3: hipLaunchKernelGGL(prod_scores_kernel<3>, grid, block, 0, stream, a, chunks); break;
    case 4: hipLaunchKernelGGL(prod_scores_kernel<4>, grid, block, 0, stream, a, chunks); break;
    case 5: hipLaunchKernelGGL(prod_scores_kernel<5>, grid, block, 0, stream, a, chunks); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tq
