// Recent-window part of the hybrid decode for gfx950: attention of each
// query head over its sequence's dense recent K/V rows, merged with the
// packed part's finished output.
//
// Sources: TurboQuant docs, "Integration API" (vLLM hooks, hybrid mode:
// compressed history plus the exact recent tokens for decode) and
// "Architecture", "Cache Lifecycle" (decoded tokens go to a recent window
// before they are flushed to packed pages).  One softmax spans both parts:
// with Z_p, o_p the packed part's normaliser and normalised output and
// Z_w, a_w the window's, out = (Z_p o_p + a_w) / (Z_p + Z_w), evaluated from
// the two log2-sum-exp2s.

#include "tq_internal.h"
#include "tq_device.h"

namespace tq {

namespace {

constexpr int kChunk = 64;   // window tokens staged per round
constexpr int kRow = 132;    // floats per staged row: 16-byte aligned, neighbouring rows on other banks
constexpr int kHeads = 8;    // query heads per workgroup

// Four consecutive elements of a row of fp32 / fp16 / bf16 values, widened to fp32.
__device__ __forceinline__ floatx4 load4(const void* base, int64_t elem, int dt) {
  if (dt == 0) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const float*>(base) + elem);
    return floatx4{__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
  }
  const u32x2 v = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(base) + elem);
  if (dt == 1) {
    const half4 h = __builtin_bit_cast(half4, v);
    return floatx4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
  }
  return floatx4{bf16_to_f32((uint16_t)v.x), bf16_to_f32((uint16_t)(v.x >> 16)), bf16_to_f32((uint16_t)v.y),
                 bf16_to_f32((uint16_t)(v.y >> 16))};
}

__device__ __forceinline__ float load1(const void* base, int64_t elem, int dt) {
  if (dt == 0) return static_cast<const float*>(base)[elem];
  const uint16_t u = static_cast<const uint16_t*>(base)[elem];
  return dt == 1 ? (float)__builtin_bit_cast(_Float16, u) : bf16_to_f32(u);
}

}  // namespace

// One workgroup of 256 threads per (sequence b, KV head g, group of up to 8
// query heads).  Per round of up to 64 window tokens: the K and V rows are
// staged in LDS as fp32; thread pairs (head, token) form the scores; the 32
// threads of each head (thread = head * 32 + dim quad) update its running
// maximum, normaliser and 4 output dims (online softmax in the log2 domain).
// Finally the window's part is merged with the packed part's output.
__global__ __launch_bounds__(256) void hybrid_window_kernel(HybridArgs a) {
  __shared__ float ks[kChunk * kRow];
  __shared__ float vs[kChunk * kRow];
  __shared__ float qs[kHeads * 128];
  __shared__ float ps[kHeads * kChunk];
  const int tid = threadIdx.x;
  const int G = a.group, Hkv = a.num_kv_heads;
  const int nhc = (G + kHeads - 1) / kHeads;
  int wg = blockIdx.x;
  const int hc = wg % nhc;
  wg /= nhc;
  const int g = wg % Hkv, b = wg / Hkv;
  const int h0 = g * G + kHeads * hc, nh = min(kHeads, G - kHeads * hc);
  const int R = min(max(a.recent_lens[b], 0), a.cap);
  if (R == 0) return;  // the packed part's output stands (uniform per workgroup)

  for (int e = tid; e < nh * 128; e += 256)
    qs[e] = load1(a.q, ((int64_t)b * a.num_q_heads + h0) * 128 + e, a.q_dtype);

  const int hi = tid >> 5, dq = tid & 31;  // this thread's head and dims 4 dq .. 4 dq + 3
  float m = -__builtin_inff(), l = 0.0f;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  const int64_t row_stride = (int64_t)Hkv * 128;  // elements between tokens of one head
  const int64_t base = ((int64_t)b * a.cap * Hkv + g) * 128;
  for (int c0 = 0; c0 < R; c0 += kChunk) {
    const int n = min(kChunk, R - c0);
    __syncthreads();  // the previous round's reads of ks / vs / ps are done (and qs is written)
    for (int e = tid; e < n * 32; e += 256) {
      const int t = e >> 5, d4 = 4 * (e & 31);
      const int64_t at = base + (int64_t)(c0 + t) * row_stride + d4;
      *reinterpret_cast<floatx4*>(ks + t * kRow + d4) = load4(a.recent_k, at, a.r_dtype);
      *reinterpret_cast<floatx4*>(vs + t * kRow + d4) = load4(a.recent_v, at, a.r_dtype);
    }
    __syncthreads();
    // scores, in log2 units: pair p = tid + 256 k -> (head p / 64, token p % 64)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int p = tid + 256 * k, i = p >> 6, t = p & 63;
      float s = -__builtin_inff();
      if (i < nh && t < n) {
        const float* qr = qs + i * 128;
        const float* kr = ks + t * kRow;
        float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll 8
        for (int d = 0; d < 128; d += 4) {
          const floatx4 qv = *reinterpret_cast<const floatx4*>(qr + d);
          const floatx4 kv = *reinterpret_cast<const floatx4*>(kr + d);
          d0 = fmaf(qv[0], kv[0], d0);
          d1 = fmaf(qv[1], kv[1], d1);
          d2 = fmaf(qv[2], kv[2], d2);
          d3 = fmaf(qv[3], kv[3], d3);
        }
        s = ((d0 + d1) + (d2 + d3)) * a.scale_log2;
      }
      ps[p] = s;
    }
    __syncthreads();
    if (hi < nh) {
      // the 32 threads of head hi: running maximum and normaliser
      const float s0 = ps[hi * kChunk + dq], s1 = ps[hi * kChunk + dq + 32];
      float cm = fmaxf(s0, s1);
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off, 32));
      const float mn = fmaxf(m, cm);  // finite: the round has at least one token
      const float alpha = __builtin_amdgcn_exp2f(m - mn);  // 0 while m = -inf
      const float p0 = __builtin_amdgcn_exp2f(s0 - mn), p1 = __builtin_amdgcn_exp2f(s1 - mn);
      float ls = p0 + p1;
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) ls += __shfl_xor(ls, off, 32);
      l = l * alpha + ls;
      m = mn;
      acc *= alpha;
      // weights go back to the staging row; only this head's 32 threads (half
      // a wave) read them below
      ps[hi * kChunk + dq] = p0;
      ps[hi * kChunk + dq + 32] = p1;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const float* pr = ps + hi * kChunk;
      for (int t = 0; t < n; ++t) {
        const float w = pr[t];
        const floatx4 v = *reinterpret_cast<const floatx4*>(vs + t * kRow + 4 * dq);
        acc += w * v;
      }
    }
  }
  if (hi >= nh) return;
  // merge with the packed part
  const int h = h0 + hi;
  const float lp = a.lse[(int64_t)b * a.num_q_heads + h];
  const float M = fmaxf(lp, m);
  const float wp = lp == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(lp - M);
  const float ww = __builtin_amdgcn_exp2f(m - M);
  float* o = a.out + ((int64_t)b * a.num_q_heads + h) * 128 + 4 * dq;
  const floatx4 op = *reinterpret_cast<const floatx4*>(o);
  const float inv = 1.0f / (wp + ww * l);
  *reinterpret_cast<floatx4*>(o) = (wp * op + ww * acc) * inv;
}

hipError_t launch_hybrid(const HybridArgs& a, hipStream_t stream) {
  const int nhc = (a.group + kHeads - 1) / kHeads;
  const long long wgs = (long long)a.batch * a.num_kv_heads * nhc;
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL(hybrid_window_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tq
