// Encoding of one TQ row by a 4-lane quad, shared by the row writer
// (tq_write.hip) and the decode kernels that append a sequence's new row
// themselves (tq_decode.hip, tq_decode_wave.hip).  Internal; not part of the ABI.
//
// Row format: TurboQuant docs, "vLLM Usage" section "TQ Byte Layout"
// (ceil(128*bits/8) bytes of LSB-first packed codebook indices, then the
// fp32 norm).  Per row: n = fp32(sqrt(sum x^2)) with the sum exact-rounded in
// float64 (fast path: plain float64 accumulation; when the error bound does
// not decide the fp32 rounding, the row is re-summed with double-double
// arithmetic); r = H (s * x) / (n sqrt(128)); idx = nearest centroid via the
// symmetric boundary count; LSB-first pack.  Lane q of the quad holds
// coordinates 32q .. 32q + 31.
#pragma once

#include "tq_internal.h"
#include "tq_device.h"

namespace tq {

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

// n = fp32(sqrt(sum x^2)) of the quad's row, the sum exact-rounded in
// float64: the fast sum has relative error below 40 * 2^-53 (the sqrt halves
// it); when that bound does not decide the fp32 rounding, the row is re-summed
// with double-double arithmetic.  Returns the float64 root.
__device__ __forceinline__ double row_norm(const float (&x)[32]) {
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < 32; ++j) s = __builtin_fma((double)x[j], (double)x[j], s);
  s += quad_xor<1>(s);
  s += quad_xor<2>(s);
  double n64 = sqrt_rn(s);
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
  return n64;
}

// x <- H (s * x) over the quad's 128 coordinates (lane q holds 32q .. 32q + 31):
// the sign flip, five butterfly stages in the lane, two across the quad.
__device__ __forceinline__ void rotate_row(const uint32_t* sign_bits, int q, float (&x)[32]) {
  uint32_t sw = pick4(sign_bits, q);
  asm volatile("" : "+v"(sw));  // one register, not 32 sign masks hoisted out of a caller's loop
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
}

// Encode the quad's row x (lane q: coordinates 32q .. 32q + 31) at BITS
// bits and store it at dst (row_bytes bytes): lane q writes index words
// BITS q .. BITS q + BITS - 1, lane 3 also the norm.  pos_bounds: the
// 2^(BITS-1) - 1 positive codebook boundaries, increasing.
template <int BITS>
__device__ __forceinline__ void encode_store_row(float (&x)[32], int q, const uint32_t* sign_bits,
                                                 const float* pos_bounds, uint8_t* dst, int row_bytes) {
  constexpr int N = 1 << BITS;
  constexpr int HALF = N / 2;
  const double n64 = row_norm(x);
  const float n32 = (float)n64;
  const float c = n64 > 0.0 ? (float)(1.0 / (n64 * 11.313708498984761)) : 0.0f;  // 1/(n sqrt(128))
  rotate_row(sign_bits, q, x);

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
    for (int k = 0; k < HALF - 1; ++k) cnt += (ar > pos_bounds[k]) ? 1 : 0;
    const uint32_t idx = (uint32_t)(r > 0.0f ? HALF + cnt : HALF - 1 - cnt);
    const int pos = BITS * j;
    w[pos >> 5] |= idx << (pos & 31);
    if ((pos & 31) + BITS > 32) w[(pos >> 5) + 1] |= idx >> (32 - (pos & 31));
  }

  uint32_t* d32 = reinterpret_cast<uint32_t*>(dst) + BITS * q;
#pragma unroll
  for (int k = 0; k < BITS; ++k) d32[k] = w[k];
  if (q == 3) *reinterpret_cast<float*>(dst + row_bytes - 4) = n32;
}

// load_row32 for a run-time dtype (0 fp32, 1 fp16, 2 bf16)
__device__ __forceinline__ void load_row_any(const void* raw, int dtype, int64_t elem_off, float (&x)[32]) {
  if (dtype == 0)
    load_row32<0>(raw, elem_off, x);
  else if (dtype == 1)
    load_row32<1>(raw, elem_off, x);
  else
    load_row32<2>(raw, elem_off, x);
}

// The same for a raw row of run-time dtype (0 fp32, 1 fp16, 2 bf16): the
// quad loads its row from raw at element elem_off + 32 q, then encodes it.
template <int BITS>
__device__ __forceinline__ void load_encode_store_row(const void* raw, int dtype, int64_t elem_off, int q,
                                                      const uint32_t* sign_bits, const float* pos_bounds,
                                                      uint8_t* dst, int row_bytes) {
  float x[32];
  load_row_any(raw, dtype, elem_off + 32 * q, x);
  encode_store_row<BITS>(x, q, sign_bits, pos_bounds, dst, row_bytes);
}

}  // namespace tq
