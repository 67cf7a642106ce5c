// HIP kernels for gfx950 (CDNA4): the TQ row writer, the split-K paged decode
// over TQ pages, and the split merge with the inverse rotation.
//
// Row format and page shape: TurboQuant docs, "vLLM Usage" section "TQ Byte
// Layout" (ceil(128*bits/8) bytes of LSB-first packed indices + fp32 norm)
// and "Architecture" section "Cache Storage Objects" (uint8
// [num_blocks, block_size, num_kv_heads, row_bytes]).  Flat slots: "vLLM
// Usage" section "Slot Mapping".  The decode reads packed pages and rebuilds
// rows inside its loop ("Architecture", "Diagnostic vs Serving Paths"), but
// never materialises them: since R is orthogonal, q . (n R^T c) = n (R q) . c
// and sum_t p_t n_t R^T c_t = R^T sum_t p_t n_t c_t, so scores and the value
// sum are formed on the rotated codes and rotated back once per head.

#include "tq_internal.h"

#include <stdint.h>

namespace tq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// --------------------------------------------------------------------------
// small helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// value of the partner lane inside a quad (xor 1 or xor 2), via DPP
template <int XOR>
__device__ __forceinline__ float quad_xor(float v) {
  constexpr int ctrl = XOR == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
}

template <int XOR>
__device__ __forceinline__ double quad_xor(double v) {
  constexpr int ctrl = XOR == 1 ? 0xB1 : 0x4E;
  uint64_t b = __double_as_longlong(v);
  uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
  lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, ctrl, 0xF, 0xF, false);
  hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, ctrl, 0xF, 0xF, false);
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// Correctly rounded double square root: the hardware sequence is refined by
// one exact Tuckerman test (the residual S - r * r' is exact under FMA).
__device__ __forceinline__ double sqrt_rn(double S) {
  if (!(S > 0.0)) return 0.0;
  double r = __builtin_sqrt(S);
  const long long rb = __double_as_longlong(r);
  double up = __longlong_as_double(rb + 1);  // r > 0 and finite
  double dn = __longlong_as_double(rb - 1);
  double ulp_up = up - r, ulp_dn = r - dn;
  if (__builtin_fma(-r, up, S) > 0.25 * ulp_up * ulp_up) return up;          // S > (r + u/2)^2
  if (__builtin_fma(-r, dn, S) <= 0.25 * ulp_dn * ulp_dn) return dn;         // S <= (r - u/2)^2
  return r;
}

// ==========================================================================
// Row writer: one row (token, head) per 4-lane quad, 32 elements per lane.
//
// Per row: n = fp32(sqrt(sum x^2)) with the sum exact-rounded in float64
// (fast path: plain float64 accumulation; when the error bound does not
// decide the fp32 rounding, the row is re-summed with double-double
// arithmetic); r = H (s * x) / (n sqrt(128)); idx = nearest centroid via the
// symmetric boundary count; LSB-first pack; store at the slot.
// ==========================================================================

template <int DT>
__device__ __forceinline__ void load_row32(const void* raw, int64_t elem_off, float (&x)[32]) {
  if constexpr (DT == 0) {  // fp32: 8 x 16 bytes
    const float* p = static_cast<const float*>(raw) + elem_off;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4 v = *reinterpret_cast<const u32x4*>(p + 4 * i);
      x[4 * i + 0] = __uint_as_float(v.x);
      x[4 * i + 1] = __uint_as_float(v.y);
      x[4 * i + 2] = __uint_as_float(v.z);
      x[4 * i + 3] = __uint_as_float(v.w);
    }
  } else {  // fp16 / bf16: 4 x 16 bytes
    const uint16_t* p = static_cast<const uint16_t*>(raw) + elem_off;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 v = *reinterpret_cast<const u32x4*>(p + 8 * i);
      uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint16_t lo = (uint16_t)(w[k] & 0xFFFF), hi = (uint16_t)(w[k] >> 16);
        if constexpr (DT == 1) {
          x[8 * i + 2 * k] = (float)__builtin_bit_cast(_Float16, lo);
          x[8 * i + 2 * k + 1] = (float)__builtin_bit_cast(_Float16, hi);
        } else {
          x[8 * i + 2 * k] = bf16_to_f32(lo);
          x[8 * i + 2 * k + 1] = bf16_to_f32(hi);
        }
      }
    }
  }
}

template <int BITS, int DT>
__global__ __launch_bounds__(256) void write_rows_kernel(WriteArgs a) {
  constexpr int N = 1 << BITS;
  constexpr int HALF = N / 2;
  const int q = threadIdx.x & 3;
  const int64_t row = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
  if (row >= a.num_rows) return;  // uniform per quad
  const int64_t tok = row / a.num_kv_heads;
  const int head = (int)(row - tok * a.num_kv_heads);
  const int64_t slot = a.slots[tok];
  if (slot < 0) return;
  if (slot >= a.num_slots) {
    if (q == 0 && head == 0 && a.err_count) atomicAdd(a.err_count, 1);
    return;
  }

  float x[32];
  load_row32<DT>(a.raw, row * kHeadDim + 32 * q, x);

  // ---- norm: float64 sum of squares, exact-rounded ------------------------
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < 32; ++j) s = __builtin_fma((double)x[j], (double)x[j], s);
  s += quad_xor<1>(s);
  s += quad_xor<2>(s);
  double n64 = sqrt_rn(s);
  {
    // the fast sum has relative error below 40 * 2^-53; the sqrt halves it
    const double lo = n64 * (1.0 - 0x1p-47), hi = n64 * (1.0 + 0x1p-47);
    if ((float)lo != (float)hi) {
      double sh = 0.0, sl = 0.0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        double sq = (double)x[j] * (double)x[j];  // exact
        double t, e;
        two_sum(sh, sq, t, e);
        sh = t;
        sl += e;
      }
      {
        double oh = quad_xor<1>(sh), ol = quad_xor<1>(sl), t, e;
        two_sum(sh, oh, t, e);
        sh = t;
        sl = sl + ol + e;
      }
      {
        double oh = quad_xor<2>(sh), ol = quad_xor<2>(sl), t, e;
        two_sum(sh, oh, t, e);
        sh = t;
        sl = sl + ol + e;
      }
      n64 = sqrt_rn(sh + sl);
    }
  }
  const float n32 = (float)n64;
  const float c = n64 > 0.0 ? (float)(1.0 / (n64 * 11.313708498984761)) : 0.0f;  // 1/(n sqrt(128))

  // ---- randomized Hadamard transform ------------------------------------
  const uint32_t sw = a.sign_bits[q];
#pragma unroll
  for (int j = 0; j < 32; ++j) x[j] = __uint_as_float(__float_as_uint(x[j]) ^ (((sw >> j) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if ((j & h) == 0) {
        const float u = x[j], v = x[j + h];
        x[j] = u + v;
        x[j + h] = u - v;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float p = quad_xor<1>(x[j]);
    x[j] = (q & 1) ? p - x[j] : x[j] + p;
  }
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float p = quad_xor<2>(x[j]);
    x[j] = (q & 2) ? p - x[j] : x[j] + p;
  }

  // ---- nearest centroid and LSB-first packing ----------------------------
  uint32_t w[BITS];
#pragma unroll
  for (int k = 0; k < BITS; ++k) w[k] = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float r = x[j] * c;
    const float ar = __builtin_fabsf(r);
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < HALF - 1; ++k) cnt += (ar > a.pos_bounds[k]) ? 1 : 0;
    const uint32_t idx = (uint32_t)(r > 0.0f ? HALF + cnt : HALF - 1 - cnt);
    const int pos = BITS * j;
    w[pos >> 5] |= idx << (pos & 31);
    if ((pos & 31) + BITS > 32) w[(pos >> 5) + 1] |= idx >> (32 - (pos & 31));
  }

  uint8_t* dst = a.pages + (slot / a.block_size) * a.page_bytes +
                 ((slot % a.block_size) * a.num_kv_heads + head) * (int64_t)a.row_bytes;
  uint32_t* d32 = reinterpret_cast<uint32_t*>(dst) + BITS * q;
#pragma unroll
  for (int k = 0; k < BITS; ++k) d32[k] = w[k];
  if (q == 3) *reinterpret_cast<float*>(dst + a.row_bytes - 4) = n32;
}

template <int BITS>
static hipError_t launch_write_bits(const WriteArgs& a, int dt, hipStream_t st) {
  const dim3 grid((unsigned)((a.num_rows + 63) / 64)), block(256);
  if (dt == 0)
    hipLaunchKernelGGL((write_rows_kernel<BITS, 0>), grid, block, 0, st, a);
  else if (dt == 1)
    hipLaunchKernelGGL((write_rows_kernel<BITS, 1>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((write_rows_kernel<BITS, 2>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_write(const WriteArgs& a, int raw_dtype, int bits, hipStream_t stream) {
  if (a.num_rows == 0) return hipSuccess;
  switch (bits) {
    case 2: return launch_write_bits<2>(a, raw_dtype, stream);
    case 3: return launch_write_bits<3>(a, raw_dtype, stream);
    case 4: return launch_write_bits<4>(a, raw_dtype, stream);
    case 5: return launch_write_bits<5>(a, raw_dtype, stream);
  }
  return hipErrorInvalidValue;
}

// ==========================================================================
// Decode, split phase.  One wave per (sequence b, KV head g, split s); the
// split covers pages [s*P, min((s+1)*P, npages_b)).  Per 16-token page:
//
//  scores   S[t][h] = q~_h . c_K[idx_K[t]]  on the matrix cores:
//           v_mfma_f32_16x16x32_f16, A = dequantised keys (16 tokens x 32
//           dims), B = rotated queries (32 dims x 16 heads, G used).  Keys
//           and queries are split hi+lo fp16 (K_hi q_hi + K_hi q_lo +
//           K_lo q_hi), giving ~fp32 accuracy.
//  softmax  running maximum over t of (S*n_k + e_t), e_t the binary
//           exponent of the value norm, so the weights w = p * n_v stay in
//           (0, 2^9] and fit fp16; rescale lazily when the maximum grows
//           by more than 8.
//  values   acc[dim][h] += sum_t V^[t][dim] w[t][h]: v_mfma_f32_16x16x16_f16,
//           A = dequantised values (16 dims x 16 tokens), B = w hi / lo.
//
// Lane layout (l = lane, n = l & 15, c = l >> 4):
//  K loads   token n, dims 32c..32c+31 (4*KB contiguous bytes of the row);
//  V loads   tokens 4c..4c+3, dims 8n..8n+7 (VB bytes of each row);
//  scores    tokens 4c+r (r = 0..3) for head n;
//  acc       head n, dims 32c..32c+31 (8 blocks x 4 rows).
// Dequantisation goes through LDS pair tables: entry p = i0 | i1 << b holds
// the fp16 pair (c[i0], c[i1]).
// ==========================================================================

constexpr int kWavesPerBlock = 4;

template <int B>
__device__ __forceinline__ uint32_t pair_field(const uint32_t* w, int k) {
  constexpr int W = 2 * B;
  const int pos = W * k;
  const int wi = pos >> 5, sh = pos & 31;
  uint32_t v = w[wi] >> sh;
  if (sh + W > 32) v |= w[wi + 1] << (32 - sh);
  return v & ((1u << W) - 1u);
}

__device__ __forceinline__ uint32_t pack_half2(_Float16 lo, _Float16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

template <int QT>
__device__ __forceinline__ float load_q(const void* q, int64_t i) {
  if constexpr (QT == 0) return static_cast<const float*>(q)[i];
  else if constexpr (QT == 1) return (float)static_cast<const _Float16*>(q)[i];
  else return bf16_to_f32(static_cast<const uint16_t*>(q)[i]);
}

template <int KB, int VB, int QT>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int KT = 1 << (2 * KB);  // K pair-table entries
  constexpr int VT = 1 << (2 * VB);
  __shared__ uint32_t s_khi[KT];
  __shared__ uint32_t s_klo[KT];
  __shared__ uint32_t s_vhi[VT];

  // ---- pair tables ---------------------------------------------------------
  for (int e = threadIdx.x; e < KT; e += blockDim.x) {
    const float c0 = a.k_cent[e & ((1 << KB) - 1)], c1 = a.k_cent[e >> KB];
    const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
    s_khi[e] = pack_half2(h0, h1);
    s_klo[e] = pack_half2((_Float16)(c0 - (float)h0), (_Float16)(c1 - (float)h1));
  }
  for (int e = threadIdx.x; e < VT; e += blockDim.x)
    s_vhi[e] = pack_half2((_Float16)a.v_cent[e & ((1 << VB) - 1)], (_Float16)a.v_cent[e >> VB]);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int S = a.num_splits;
  const int total_units = a.batch * a.num_kv_heads * S;
  if (unit >= total_units) return;
  const int s = unit % S;
  const int g = (unit / S) % a.num_kv_heads;
  const int b = unit / (S * a.num_kv_heads);
  const int L = a.seq_lens[b];
  const int npages = (L + kBlockSize - 1) / kBlockSize;
  const int p0 = s * a.pages_per_split;
  if (p0 >= npages) return;
  const int p1 = min(p0 + a.pages_per_split, npages);

  const int n = lane & 15;
  const int c = lane >> 4;
  const int G = a.group;

  // ---- rotated, scaled query: q~ = H (s * q) * scale*log2e/sqrt(d) -------
  half8 qhi[4], qlo[4];
  {
    float x[32];
    const bool has = n < G;
    const int64_t qoff = ((int64_t)b * a.num_q_heads + (int64_t)g * G + n) * kHeadDim + 32 * c;
#pragma unroll
    for (int j = 0; j < 32; ++j) x[j] = has ? load_q<QT>(a.q, qoff + j) : 0.0f;
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
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = x[8 * m + j] * a.q_scale;
        const _Float16 hi = (_Float16)v;
        qhi[m][j] = hi;
        qlo[m][j] = (_Float16)(v - (float)hi);
      }
  }

  // ---- per-lane row offsets within a page --------------------------------
  const int kro = (n * a.num_kv_heads + g) * a.k_row_bytes;  // token n
  const int k_idx_off = kro + 4 * KB * c;
  const int k_norm_off = kro + a.k_row_bytes - 4;
  int v_row[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v_row[j] = ((4 * c + j) * a.num_kv_heads + g) * a.v_row_bytes;
  // value bytes [n*VB, n*VB + VB): load the aligned dword(s) that hold them
  const int v_byte = n * VB;
  const int v_dw = v_byte & ~3;
  const int v_sh = 8 * (v_byte & 3);

  floatx4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -__builtin_inff();
  float l_part = 0.0f;

  const int32_t* bt = a.block_table + (int64_t)b * a.max_blocks_per_seq;

  for (int p = p0; p < p1; ++p) {
    const int blk = __builtin_amdgcn_readfirstlane(bt[p]);
    const uint8_t* kp = a.k_pages + (int64_t)blk * a.k_page_bytes;
    const uint8_t* vp = a.v_pages + (int64_t)blk * a.v_page_bytes;

    // -- loads
    uint32_t kw[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) kw[i] = *reinterpret_cast<const uint32_t*>(kp + k_idx_off + 4 * i);
    const float nk_own = *reinterpret_cast<const float*>(kp + k_norm_off);
    uint32_t vw[4], vw_hi[4];
    float nv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint8_t* rowp = vp + v_row[j];
      vw_hi[j] = 0;
      if constexpr (VB == 4) {
        vw[j] = *reinterpret_cast<const uint32_t*>(rowp + v_byte);
      } else if constexpr (VB == 2) {
        vw[j] = *reinterpret_cast<const uint16_t*>(rowp + v_byte);
      } else {  // 3 or 5 bits: the VB bytes sit inside the 8 aligned bytes at v_dw
        const uint32_t w0 = *reinterpret_cast<const uint32_t*>(rowp + v_dw);
        const uint32_t w1 = *reinterpret_cast<const uint32_t*>(rowp + v_dw + 4);
        const uint64_t all = ((((uint64_t)w1) << 32) | w0) >> v_sh;
        vw[j] = (uint32_t)all;
        vw_hi[j] = (uint32_t)(all >> 32);
      }
      nv[j] = *reinterpret_cast<const float*>(rowp + a.v_row_bytes - 4);
    }

    // -- scores
    floatx4 sc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t ah[4], al[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t f = pair_field<KB>(kw, 4 * m + k);
        ah[k] = s_khi[f];
        al[k] = s_klo[f];
      }
      const half8 Ahi = __builtin_bit_cast(half8, u32x4{ah[0], ah[1], ah[2], ah[3]});
      const half8 Alo = __builtin_bit_cast(half8, u32x4{al[0], al[1], al[2], al[3]});
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, qhi[m], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, qlo[m], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, qhi[m], sc, 0, 0, 0);
    }

    // -- softmax bookkeeping (log2 domain)
    const int tok0 = p * kBlockSize + 4 * c;
    float sv[4], xv[4];
    float pmax = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float nk = __shfl(nk_own, 4 * c + r);
      const bool valid = tok0 + r < L;
      sv[r] = valid ? sc[r] * nk : -__builtin_inff();
      int e = 0;
      (void)__builtin_frexpf(nv[r], &e);
      const float ev = (nv[r] > 0.0f) ? (float)max(e, -64) : -64.0f;
      xv[r] = sv[r] + ev;
      pmax = fmaxf(pmax, xv[r]);
    }
    pmax = fmaxf(pmax, __shfl_xor(pmax, 16));
    pmax = fmaxf(pmax, __shfl_xor(pmax, 32));
    const bool grow = pmax > m_ref + 8.0f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = fmaxf(m_ref, pmax);
      const float alpha = (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= alpha;
      m_ref = m_new;
    }
    float wv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool valid = tok0 + r < L;
      const float pr = valid ? __builtin_amdgcn_exp2f(sv[r] - m_ref) : 0.0f;
      l_part += pr;
      wv[r] = valid ? pr * nv[r] : 0.0f;
    }
    half4 Whi, Wlo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const _Float16 hi = (_Float16)wv[r];
      Whi[r] = hi;
      Wlo[r] = (_Float16)(wv[r] - (float)hi);
    }

    // -- values
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t L4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t f;
        if constexpr (VB == 5) {
          const uint64_t all = ((uint64_t)vw_hi[j] << 32) | vw[j];
          f = (uint32_t)(all >> (10 * k)) & 0x3FFu;
        } else {
          f = (vw[j] >> (2 * VB * k)) & ((1u << (2 * VB)) - 1u);
        }
        L4[j] = s_vhi[f];
      }
      // block 2k takes the low halves (dim 8n+2k), block 2k+1 the high halves
      const uint32_t lo01 = __builtin_amdgcn_perm(L4[1], L4[0], 0x05040100u);
      const uint32_t lo23 = __builtin_amdgcn_perm(L4[3], L4[2], 0x05040100u);
      const uint32_t hi01 = __builtin_amdgcn_perm(L4[1], L4[0], 0x07060302u);
      const uint32_t hi23 = __builtin_amdgcn_perm(L4[3], L4[2], 0x07060302u);
      const half4 Ae = __builtin_bit_cast(half4, (uint64_t)lo01 | ((uint64_t)lo23 << 32));
      const half4 Ao = __builtin_bit_cast(half4, (uint64_t)hi01 | ((uint64_t)hi23 << 32));
      acc[2 * k] = __builtin_amdgcn_mfma_f32_16x16x16f16(Ae, Whi, acc[2 * k], 0, 0, 0);
      acc[2 * k] = __builtin_amdgcn_mfma_f32_16x16x16f16(Ae, Wlo, acc[2 * k], 0, 0, 0);
      acc[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(Ao, Whi, acc[2 * k + 1], 0, 0, 0);
      acc[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(Ao, Wlo, acc[2 * k + 1], 0, 0, 0);
    }
  }

  // ---- partial result of the split ---------------------------------------
  float l_tot = l_part + __shfl_xor(l_part, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (n < G) {
    const int h = g * G + n;
    const int64_t slot = ((int64_t)b * a.num_q_heads + h) * S + s;
    const float inv = 1.0f / l_tot;
    float* dst = a.part_acc + slot * kHeadDim + 32 * c;
    // acc[blk][r] holds dim 32c + 8r + blk
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
}

template <int KB, int VB>
static hipError_t launch_decode_kv(const DecodeArgs& a, int qt, hipStream_t st) {
  const long long units = (long long)a.batch * a.num_kv_heads * a.num_splits;
  const dim3 grid((unsigned)((units + kWavesPerBlock - 1) / kWavesPerBlock)), block(64 * kWavesPerBlock);
  if (qt == 0)
    hipLaunchKernelGGL((decode_split_kernel<KB, VB, 0>), grid, block, 0, st, a);
  else if (qt == 1)
    hipLaunchKernelGGL((decode_split_kernel<KB, VB, 1>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<KB, VB, 2>), grid, block, 0, st, a);
  return hipGetLastError();
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

// ==========================================================================
// Merge: one wave per (b, h).  Combines the splits' normalised rotated sums
// by their log2-sum-exp2, divides the value scale out, applies the inverse
// rotation s * H y / sqrt(128) and writes fp32 out.  Lane l owns dims l and
// l + 64.
// ==========================================================================
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
  float M = -__builtin_inff();
  for (int s = 0; s < ns; ++s) M = fmaxf(M, lse[s]);
  float den = 0.0f, y0 = 0.0f, y1 = 0.0f;
  for (int s = 0; s < ns; ++s) {
    const float wgt = __builtin_amdgcn_exp2f(lse[s] - M);
    den += wgt;
    y0 += wgt * pa[(int64_t)s * kHeadDim + lane];
    y1 += wgt * pa[(int64_t)s * kHeadDim + lane + 64];
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
    const float p0 = __shfl_xor(y0, h), p1 = __shfl_xor(y1, h);
    y0 = (lane & h) ? p0 - y0 : y0 + p0;
    y1 = (lane & h) ? p1 - y1 : y1 + p1;
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
