// Device-side helpers shared by the HIP kernels (vector types, lane
// exchanges, exact float64 arithmetic).  Internal; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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


// Word idx (0..3) of a four-word kernel-argument array.  The words come from
// scalar loads at fixed offsets: indexing the array with a per-lane value
// would read the argument segment with vector loads, one wait each.
__device__ __forceinline__ uint32_t pick4(const uint32_t* w, int idx) {
  const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
  return (idx & 2) ? ((idx & 1) ? w3 : w2) : ((idx & 1) ? w1 : w0);
}

// Centroid (lane & 31) of a kernel-argument table of 2^B entries (scalar
// loads, as in pick4); lookups gather from it with lane shuffles.
template <int B>
__device__ __forceinline__ float cent_of_lane(const float* cent, int lane) {
  float v = 0.0f;
#pragma unroll
  for (int j = 0; j < (1 << B); ++j) v = ((lane & 31) == j) ? cent[j] : v;
  return v;
}

// 2^(13 - floor(log2 mx)): scales values of magnitude <= mx into [2^13, 2^14)
// at most, where an fp16 hi + lo split keeps about 22 bits; 1 for mx = 0,
// denormal, inf or nan.  Exact (a power of two).
__device__ __forceinline__ float pow2_scale(float mx) {
  const int e = (int)((__float_as_uint(mx) >> 23) & 0xFF);
  if (e == 0 || e == 255) return 1.0f;
  const int k = min(max(13 - (e - 127), -100), 100);
  return __uint_as_float((uint32_t)(k + 127) << 23);
}

__device__ __forceinline__ uint32_t pack_half2(_Float16 lo, _Float16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

}  // namespace tq
