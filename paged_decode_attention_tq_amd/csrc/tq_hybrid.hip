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

constexpr int kChunk = 64;   // window tokens per round
constexpr int kRow = 132;    // floats per staged row: 16-byte aligned, neighbouring rows on other banks
constexpr int kHeads = 8;    // query heads per workgroup
constexpr int kPer = kChunk * 32 / 256;  // (token, dim quad) slots per thread per round

// Raw words of four consecutive elements (fp32: 4 words; fp16 / bf16: 2).
template <int RDT>
struct Quad {
  uint32_t w[RDT == 0 ? 4 : 2];
};

template <int RDT>
__device__ __forceinline__ Quad<RDT> load_quad(const void* base, int64_t elem) {
  Quad<RDT> r;
  if constexpr (RDT == 0) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const float*>(base) + elem);
    r.w[0] = v.x, r.w[1] = v.y, r.w[2] = v.z, r.w[3] = v.w;
  } else {
    const u32x2 v = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(base) + elem);
    r.w[0] = v.x, r.w[1] = v.y;
  }
  return r;
}

template <int RDT>
__device__ __forceinline__ floatx4 widen(const Quad<RDT>& r) {
  if constexpr (RDT == 0) {
    return floatx4{__uint_as_float(r.w[0]), __uint_as_float(r.w[1]), __uint_as_float(r.w[2]), __uint_as_float(r.w[3])};
  } else if constexpr (RDT == 1) {
    const half4 h = __builtin_bit_cast(half4, u32x2{r.w[0], r.w[1]});
    return floatx4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
  } else {
    return floatx4{bf16_to_f32((uint16_t)r.w[0]), bf16_to_f32((uint16_t)(r.w[0] >> 16)), bf16_to_f32((uint16_t)r.w[1]),
                   bf16_to_f32((uint16_t)(r.w[1] >> 16))};
  }
}

__device__ __forceinline__ float load1(const void* base, int64_t elem, int dt) {
  if (dt == 0) return static_cast<const float*>(base)[elem];
  const uint16_t u = static_cast<const uint16_t*>(base)[elem];
  return dt == 1 ? (float)__builtin_bit_cast(_Float16, u) : bf16_to_f32(u);
}

}  // namespace

// One workgroup of 256 threads per (sequence b, KV head g, group of up to 8
// query heads).  Rounds of 64 window tokens: each thread holds 8 (token, dim
// quad) pieces of the round's K and V rows in registers (the next round's
// are loaded while the current one is computed), writes them to LDS as
// fp32 (zeros past the window), and then
//   * scores: lane t of wave w forms token t's scores for heads w and w + 4;
//   * softmax and values: the 32 threads of head i (thread = 32 i + dim quad)
//     update its running maximum and normaliser and 4 output dims over the
//     64 tokens (online softmax in the log2 domain).
// Finally the window's part is merged with the packed part's output.  With
// causal_group set (the chunk tail of a multi-query call), query head h of
// KV head g is query j = (h - g G) / causal_group of the chunk and sees
// window rows r < j only.
template <int RDT>
__global__ __launch_bounds__(256) void hybrid_window_kernel(HybridArgs a) {
  __shared__ float ks[kChunk * kRow];
  __shared__ float vs[kChunk * kRow];
  __shared__ float qs[kHeads * 128];
  __shared__ float ps[kHeads * kChunk];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.group, Hkv = a.num_kv_heads;
  const int nhc = (G + kHeads - 1) / kHeads;
  int wg = blockIdx.x;
  const int hc = wg % nhc;
  wg /= nhc;
  const int g = wg % Hkv, b = wg / Hkv;
  const int h0 = g * G + kHeads * hc, nh = min(kHeads, G - kHeads * hc);
  const int R = min(max(a.recent_lens[b], 0), a.cap);
  if (R == 0) return;  // the packed part's output stands (uniform per workgroup)

  const int hi = tid >> 5, dq = tid & 31;  // head and dim quad (values); also the first staged token
  const int64_t row_stride = (int64_t)Hkv * 128;  // elements between tokens of one head
  const int64_t base = ((int64_t)b * a.cap * Hkv + g) * 128 + 4 * dq;
  Quad<RDT> kq[kPer], vq[kPer];
  auto fetch = [&](int c0) {  // tokens c0 + hi + 8 j, dims 4 dq .. 4 dq + 3
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int t = c0 + hi + 8 * j;
      if (t < R) {
        kq[j] = load_quad<RDT>(a.recent_k, base + t * row_stride);
        vq[j] = load_quad<RDT>(a.recent_v, base + t * row_stride);
      } else {
#pragma unroll
        for (int u = 0; u < (RDT == 0 ? 4 : 2); ++u) kq[j].w[u] = vq[j].w[u] = 0u;
      }
    }
  };
  fetch(0);
  for (int e = tid; e < kHeads * 128; e += 256)
    qs[e] = e < nh * 128 ? load1(a.q, ((int64_t)b * a.num_q_heads + h0) * 128 + e, a.q_dtype) : 0.0f;

  float m = -__builtin_inff(), l = 0.0f;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < R; c0 += kChunk) {
    __syncthreads();  // the previous round's reads of ks / vs / ps are done (and qs is written)
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int t = hi + 8 * j;
      *reinterpret_cast<floatx4*>(ks + t * kRow + 4 * dq) = widen<RDT>(kq[j]);
      *reinterpret_cast<floatx4*>(vs + t * kRow + 4 * dq) = widen<RDT>(vq[j]);
    }
    if (c0 + kChunk < R) fetch(c0 + kChunk);  // in flight during this round's work
    __syncthreads();
    {
      // scores in log2 units; past the window -inf
      const int i0 = wave, i1 = wave + 4, t = lane;
      const float* kr = ks + t * kRow;
      float s0a = 0.f, s0b = 0.f, s1a = 0.f, s1b = 0.f;
#pragma unroll
      for (int d = 0; d < 128; d += 4) {
        const floatx4 kv = *reinterpret_cast<const floatx4*>(kr + d);
        const floatx4 q0 = *reinterpret_cast<const floatx4*>(qs + i0 * 128 + d);
        const floatx4 q1 = *reinterpret_cast<const floatx4*>(qs + i1 * 128 + d);
        s0a = fmaf(q0[0], kv[0], fmaf(q0[1], kv[1], s0a));
        s0b = fmaf(q0[2], kv[2], fmaf(q0[3], kv[3], s0b));
        s1a = fmaf(q1[0], kv[0], fmaf(q1[1], kv[1], s1a));
        s1b = fmaf(q1[2], kv[2], fmaf(q1[3], kv[3], s1b));
      }
      const bool in = c0 + t < R;
      // causal: query j of the chunk (virtual head (j, i)) sees window rows r < j
      const int lim0 = a.causal_group ? ((h0 - g * G + i0) / a.causal_group) : R;
      const int lim1 = a.causal_group ? ((h0 - g * G + i1) / a.causal_group) : R;
      ps[i0 * kChunk + t] = in && c0 + t < lim0 ? (s0a + s0b) * a.scale_log2 : -__builtin_inff();
      ps[i1 * kChunk + t] = in && c0 + t < lim1 ? (s1a + s1b) * a.scale_log2 : -__builtin_inff();
    }
    __syncthreads();
    if (hi < nh) {
      // the 32 threads of head hi: running maximum and normaliser
      const float s0 = ps[hi * kChunk + dq], s1 = ps[hi * kChunk + dq + 32];
      float cm = fmaxf(s0, s1);
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off, 32));
      const float mn = fmaxf(m, cm);
      const bool none = mn == -__builtin_inff();  // every token so far masked (causal)
      const float alpha = none ? 1.0f : __builtin_amdgcn_exp2f(m - mn);  // 0 while m = -inf
      const float p0 = none ? 0.0f : __builtin_amdgcn_exp2f(s0 - mn);
      const float p1 = none ? 0.0f : __builtin_amdgcn_exp2f(s1 - mn);
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
#pragma unroll
      for (int t = 0; t < kChunk; ++t) {  // rows past the window are zero, with weight 0
        const floatx4 v = *reinterpret_cast<const floatx4*>(vs + t * kRow + 4 * dq);
        acc += pr[t] * v;
      }
    }
  }
  if (hi >= nh) return;
  // merge with the packed part
  const int h = h0 + hi;
  const float lp = a.lse[(int64_t)b * a.num_q_heads + h];
  const float M = fmaxf(lp, m);
  float* o = a.out + ((int64_t)b * a.num_q_heads + h) * 128 + 4 * dq;
  if (M == -__builtin_inff()) {  // no token in either part
    *reinterpret_cast<floatx4*>(o) = floatx4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  const float wp = lp == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(lp - M);
  const float ww = m == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m - M);
  const floatx4 op = *reinterpret_cast<const floatx4*>(o);
  const float inv = 1.0f / (wp + ww * l);
  *reinterpret_cast<floatx4*>(o) = (wp * op + ww * acc) * inv;
}

hipError_t launch_hybrid(const HybridArgs& a, hipStream_t stream) {
  const int nhc = (a.group + kHeads - 1) / kHeads;
  const long long wgs = (long long)a.batch * a.num_kv_heads * nhc;
  if (wgs == 0) return hipSuccess;
  const dim3 grid((unsigned)wgs), block(256);
  if (a.r_dtype == 0)
    hipLaunchKernelGGL(hybrid_window_kernel<0>, grid, block, 0, stream, a);
  else if (a.r_dtype == 1)
    hipLaunchKernelGGL(hybrid_window_kernel<1>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(hybrid_window_kernel<2>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace tq
