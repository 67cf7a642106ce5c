// Device helpers shared by the paged-decode kernels (tq_decode.hip and
// tq_decode_wave.hip): replicated centroid pair tables in LDS, index-field
// extraction, query loads and lane exchanges.  Internal; not part of the ABI.
#pragma once

#include "tq_internal.h"
#include "tq_device.h"

#include <type_traits>
#include <utility>

namespace tq {

// ---------------------------------------------------------------------------
// Replicated pair tables.  Row p = i0 | i1 << B holds, once per replica, an
// 8-byte entry of two dwords: hi = the fp16 pair (c[i0], c[i1]) and lo = the
// fp16 pair of their rounding residuals.  Replica k = lane & (kRep - 1) sits
// at (p << kShift) + 8k, so a half-wave's 8-byte reads hit distinct banks.
// Keys read the whole entry (the score MFMA multiplies both dwords by the
// same query pair, so their order does not matter); values read hi only
// (the centroids are scaled so that fp16 holds them to about 1e-4
// relative).  The upper half of the replicas stores (lo, hi), which puts
// the hi dwords of a half-wave on distinct banks too.
template <int B>
struct PairTable {
  static constexpr int kRows = 1 << (2 * B);
  static constexpr int kRep = (B == 5) ? 4 : 32;
  static constexpr int kShift = (B == 5) ? 5 : 8;
  static constexpr int kStride = 1 << kShift;  // = 8 * kRep
  static constexpr int kBytes = kRows * kStride;
};

template <int B>
__device__ __forceinline__ void fill_pair_table(uint8_t* base, const float* cent, int tid, int nthreads) {
  using T = PairTable<B>;
  constexpr int kQuads = T::kBytes / 16;  // 2 replicas per 16-byte store
  const float cl = cent_of_lane<B>(cent, tid & 63);
  for (int i0 = 0; i0 < kQuads; i0 += nthreads) {  // every lane runs every round (shuffles)
    const int i = min(i0 + tid, kQuads - 1);
    const int row = (2 * i) / T::kRep;
    const float c0 = __shfl(cl, row & ((1 << B) - 1)), c1 = __shfl(cl, row >> B);
    const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
    const uint32_t hi = pack_half2(h0, h1);
    const uint32_t lo = pack_half2((_Float16)(c0 - (float)h0), (_Float16)(c1 - (float)h1));
    const bool swap = ((2 * i) % T::kRep) >= T::kRep / 2;
    if (i0 + tid < kQuads) *reinterpret_cast<u32x4*>(base + 16 * i) = swap ? u32x4{lo, hi, lo, hi} : u32x4{hi, lo, hi, lo};
  }
}

// The same rows without the swapped upper replicas: every replica stores
// (hi, lo), so the lo dword of an entry is 4 bytes past its hi dword for
// every lane.  With 32 replicas the hi reads of a half-wave hit banks 2k and
// the lo reads banks 2k + 1, k = lane & 31: conflict-free either way.
template <int B>
__device__ __forceinline__ void fill_pair_table_flat(uint8_t* base, const float* cent, int tid, int nthreads) {
  using T = PairTable<B>;
  constexpr int kQuads = T::kBytes / 16;  // 2 replicas per 16-byte store
  const float cl = cent_of_lane<B>(cent, tid & 63);
  for (int i0 = 0; i0 < kQuads; i0 += nthreads) {  // every lane runs every round (shuffles)
    const int i = min(i0 + tid, kQuads - 1);
    const int row = (2 * i) / T::kRep;
    const float c0 = __shfl(cl, row & ((1 << B) - 1)), c1 = __shfl(cl, row >> B);
    const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
    const uint32_t hi = pack_half2(h0, h1);
    const uint32_t lo = pack_half2((_Float16)(c0 - (float)h0), (_Float16)(c1 - (float)h1));
    if (i0 + tid < kQuads) *reinterpret_cast<u32x4*>(base + 16 * i) = u32x4{hi, lo, hi, lo};
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

__device__ __forceinline__ float load_q(const void* q, int64_t i, int qt) {
  if (qt == 0) return static_cast<const float*>(q)[i];
  if (qt == 1) return (float)static_cast<const _Float16*>(q)[i];
  return bf16_to_f32(static_cast<const uint16_t*>(q)[i]);
}

template <int R>
__device__ __forceinline__ float quad_bcast(float v) {  // lane 4k + R of each quad to all four
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), R * 0x55, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_bcast_r(float v, int r) {  // r: compile-time after unrolling
  switch (r) {
    case 0: return quad_bcast<0>(v);
    case 1: return quad_bcast<1>(v);
    case 2: return quad_bcast<2>(v);
    default: return quad_bcast<3>(v);
  }
}

// max over the four 16-lane rows (lanes n, n + 16, n + 32, n + 48)
__device__ __forceinline__ float max_across_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float row_ror8(float v) {  // lane n <-> n ^ 8 inside a 16-lane row
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}

// f(integral_constant<0>), ..., f(integral_constant<N - 1>)
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Hadamard butterfly between lanes l and l ^ M: lanes with bit M clear get
// x_l + x_(l^M), the others x_(l^M) - x_l.  M = 16, 32: one permlane swap
// (both copies of x in, partner and self out) and one FMA with sign +-1
// (exact: the same rounding as the add or subtract); M = 1, 2: DPP quad
// permutes; M = 4, 8: LDS-free swizzle / row rotate.
template <int M>
__device__ __forceinline__ float lane_bfly(float x, int lane) {
  const bool upper = (lane & M) != 0;
  if constexpr (M == 16 || M == 32) {
    // the swap puts self in [0] and the partner in [1] on lanes with bit M
    // clear, partner in [0] and self in [1] on the others
    const auto s = M == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                           : __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaf(upper ? -1.0f : 1.0f, __uint_as_float(s[1]), __uint_as_float(s[0]));
  } else {
    float p;
    if constexpr (M == 1)
      p = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
    else if constexpr (M == 2)
      p = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
    else if constexpr (M == 8)
      p = row_ror8(x);
    else
      p = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (M << 10)));  // lane ^ M within 32
    return upper ? p - x : x + p;
  }
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// One buffer_load_dwordx4 with the lds modifier moves 64 16-byte chunks
// from global memory into LDS at M0 + 16 * lane without passing through
// registers.  It is inline assembly so that the compiler does not make the
// LDS reads of other slots wait for it; the kernel waits itself.
__device__ __forceinline__ void copy_chunk_to_lds(i32x4 rsrc, uint32_t lds_addr, uint32_t voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace tq
