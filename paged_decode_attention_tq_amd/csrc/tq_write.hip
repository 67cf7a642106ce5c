// Row writer kernel for gfx950: encodes raw K or V rows into TQ rows and
// stores them in the uint8 pages through flat slots.
//
// Row format: TurboQuant docs, "vLLM Usage" section "TQ Byte Layout"
// (ceil(128*bits/8) bytes of LSB-first packed codebook indices, then the
// fp32 norm); slots: "vLLM Usage" section "Slot Mapping" (negative slots are
// ignored, out-of-range slots are an error); pages: "Architecture" section
// "Cache Storage Objects" ([num_blocks, block_size, num_kv_heads, row_bytes]).

#include "tq_internal.h"
#include "tq_device.h"

#include <algorithm>

namespace tq {

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

// The rows of workgroup `wg` (64 rows, one per 4-lane quad) of one call.
template <int BITS, int DT>
__device__ __forceinline__ void write_rows(const WriteArgs& a, int64_t wg) {
  constexpr int N = 1 << BITS;
  constexpr int HALF = N / 2;
  const int q = threadIdx.x & 3;
  const int64_t row = wg * 64 + (threadIdx.x >> 2);
  if (row >= a.num_rows) return;  // uniform per quad
  const int64_t tok = row / a.num_kv_heads;
  const int head = (int)(row - tok * a.num_kv_heads);
  const int64_t slot = a.slots[tok];
  // the row is read before its slot is known (both loads in flight
  // together); a dropped row's read is wasted
  float x[32];
  load_row32<DT>(a.raw, row * kHeadDim + 32 * q, x);
  if (slot < 0) return;
  if (slot >= a.num_slots) {
    if (q == 0 && head == 0 && a.err_count) atomicAdd(a.err_count, 1);
    return;
  }

  const double n64 = row_norm(x);
  const float n32 = (float)n64;
  const float c = n64 > 0.0 ? (float)(1.0 / (n64 * 11.313708498984761)) : 0.0f;  // 1/(n sqrt(128))
  rotate_row(a.sign_bits, q, x);

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

template <int BITS, int DT>
__global__ __launch_bounds__(256) void write_rows_kernel(WriteArgs a) {
  write_rows<BITS, DT>(a, blockIdx.x);
}

// K and V rows of the same tokens in one launch: workgroups [0, k_groups)
// take the K rows, the others the V rows.
template <int KB, int VB, int DT>
__global__ __launch_bounds__(256) void write_pair_kernel(WriteArgs k, WriteArgs v, int64_t k_groups) {
  const int64_t wg = blockIdx.x;
  if (wg < k_groups)
    write_rows<KB, DT>(k, wg);
  else
    write_rows<VB, DT>(v, wg - k_groups);
}

// ==========================================================================
// Prod key rows (the inner-product codec): the rotated unit vector's indices
// at BITS - 1 bits, then a 1-bit sketch of its residual e = r - c[idx] under
// the d x d matrix S (sign of (S e)_i), and gamma = ||e||.  Row: index words,
// norm, 4 sign words (bit i of word q = sign of output 32 q + i), gamma.
//
// Quad per row as above.  Lane q forms outputs 32 q .. 32 q + 31 of S e: it
// takes the 32 residuals of each quad lane in turn (DPP broadcasts) and
// multiplies by its 32 x 32 block of S from LDS (kSkGroup below: the four
// quad lanes' reads fall on different banks).  Persistent grid: S is loaded
// once per workgroup.
// ==========================================================================
// S in LDS: rows 32 g .. 32 g + 31 at g * kSkGroup floats, row-major inside;
// the 4-float gap between groups puts the four quad lanes' reads on
// different banks
constexpr int kSkGroup = 32 * kHeadDim + 4;

template <int K>
__device__ __forceinline__ float quad_bcast(float v) {
  constexpr int ctrl = K | (K << 2) | (K << 4) | (K << 6);
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
}

// p[i] += sum_j S[32 q + i][32 K + j] e_K[j], e_K the residuals of quad lane K
template <int K>
__device__ __forceinline__ void sketch_part(const float* sk, int q, const float (&x)[32], float (&p)[32]) {
  float ek[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) ek[j] = quad_bcast<K>(x[j]);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float* srow = sk + q * kSkGroup + i * kHeadDim + 32 * K;  // constant offsets from one base
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const floatx4 s4 = *reinterpret_cast<const floatx4*>(srow + 4 * m);
      p[i] = fmaf(s4[0], ek[4 * m], p[i]);
      p[i] = fmaf(s4[1], ek[4 * m + 1], p[i]);
      p[i] = fmaf(s4[2], ek[4 * m + 2], p[i]);
      p[i] = fmaf(s4[3], ek[4 * m + 3], p[i]);
    }
    // one output row at a time: p[i] is complete before the next row's reads
    // are issued (the compiler would otherwise gather all 256 reads of the
    // block first, more values than the register file holds)
    asm volatile("" : "+v"(p[i]) :: "memory");
  }
}

template <int BITS, int DT>
__global__ __launch_bounds__(256) void write_prod_kernel(ProdWriteArgs pa) {
  constexpr int MB = BITS - 1, N = 1 << MB, HALF = N / 2;
  __shared__ float sk[4 * kSkGroup];
  const WriteArgs& a = pa.w;
  for (int e = threadIdx.x; e < kHeadDim * kHeadDim / 4; e += 256) {
    const int i = (4 * e) >> 7, j = (4 * e) & 127;
    *reinterpret_cast<floatx4*>(sk + (i >> 5) * kSkGroup + (i & 31) * kHeadDim + j) =
        *reinterpret_cast<const floatx4*>(pa.sketch + 4 * e);
  }
  __syncthreads();
  const int q = threadIdx.x & 3;
  const int64_t nblk = (a.num_rows + 63) / 64;
  for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int64_t row = blk * 64 + (threadIdx.x >> 2);
    if (row >= a.num_rows) continue;  // uniform per quad
    const int64_t tok = row / a.num_kv_heads;
    const int head = (int)(row - tok * a.num_kv_heads);
    const int64_t slot = a.slots[tok];
    float x[32];
    load_row32<DT>(a.raw, row * kHeadDim + 32 * q, x);
    if (slot < 0) continue;
    if (slot >= a.num_slots) {
      if (q == 0 && head == 0 && a.err_count) atomicAdd(a.err_count, 1);
      continue;
    }
    const double n64 = row_norm(x);
    const float n32 = (float)n64;
    const float c = n64 > 0.0 ? (float)(1.0 / (n64 * 11.313708498984761)) : 0.0f;  // 1/(n sqrt(128))
    rotate_row(a.sign_bits, q, x);

    // indices at MB bits and the residual (kept in x), its squared norm
    uint32_t w[MB];
#pragma unroll
    for (int k = 0; k < MB; ++k) w[k] = 0;
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float r = x[j] * c;
      const float ar = __builtin_fabsf(r);
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < HALF - 1; ++k) cnt += (ar > a.pos_bounds[k]) ? 1 : 0;
      const uint32_t idx = (uint32_t)(r > 0.0f ? HALF + cnt : HALF - 1 - cnt);
      const int pos = MB * j;
      w[pos >> 5] |= idx << (pos & 31);
      if ((pos & 31) + MB > 32) w[(pos >> 5) + 1] |= idx >> (32 - (pos & 31));
      float cp = pa.cpos[0];
#pragma unroll
      for (int k = 1; k < HALF; ++k) cp = cnt == k ? pa.cpos[k] : cp;
      x[j] = r - (r > 0.0f ? cp : -cp);
      ss = fmaf(x[j], x[j], ss);
    }
    ss += quad_xor<1>(ss);
    ss += quad_xor<2>(ss);
    const float gamma = __builtin_sqrtf(ss);

    // outputs 32 q + i of S e
    float p[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) p[i] = 0.0f;
    sketch_part<0>(sk, q, x, p);
    sketch_part<1>(sk, q, x, p);
    sketch_part<2>(sk, q, x, p);
    sketch_part<3>(sk, q, x, p);
    uint32_t zw = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) zw |= (p[i] >= 0.0f ? 1u : 0u) << i;

    uint8_t* dst = a.pages + (slot / a.block_size) * a.page_bytes +
                   ((slot % a.block_size) * a.num_kv_heads + head) * (int64_t)a.row_bytes;
    uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);
#pragma unroll
    for (int k = 0; k < MB; ++k) d32[MB * q + k] = w[k];
    d32[4 * MB + 1 + q] = zw;
    if (q == 3) {
      d32[4 * MB] = __float_as_uint(n32);
      d32[4 * MB + 5] = __float_as_uint(gamma);
    }
  }
}

template <int BITS>
static hipError_t launch_prod_bits(const ProdWriteArgs& a, int dt, int num_cus, hipStream_t st) {
  const int64_t nblk = (a.w.num_rows + 63) / 64;
  const dim3 grid((unsigned)std::min<int64_t>(nblk, 2LL * num_cus)), block(256);  // 64 KB of LDS: two per CU
  if (dt == 0)
    hipLaunchKernelGGL((write_prod_kernel<BITS, 0>), grid, block, 0, st, a);
  else if (dt == 1)
    hipLaunchKernelGGL((write_prod_kernel<BITS, 1>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((write_prod_kernel<BITS, 2>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_write_prod(const ProdWriteArgs& a, int raw_dtype, int bits, int num_cus, hipStream_t stream) {
  if (a.w.num_rows == 0) return hipSuccess;
  switch (bits) {
    case 2: return launch_prod_bits<2>(a, raw_dtype, num_cus, stream);
    case 3: return launch_prod_bits<3>(a, raw_dtype, num_cus, stream);
    case 4: return launch_prod_bits<4>(a, raw_dtype, num_cus, stream);
    case 5: return launch_prod_bits<5>(a, raw_dtype, num_cus, stream);
  }
  return hipErrorInvalidValue;
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

template <int KB, int VB>
static hipError_t launch_pair_kv(const WriteArgs& k, const WriteArgs& v, int dt, hipStream_t st) {
  const int64_t groups = (k.num_rows + 63) / 64;
  const dim3 grid((unsigned)(2 * groups)), block(256);
  if (dt == 0)
    hipLaunchKernelGGL((write_pair_kernel<KB, VB, 0>), grid, block, 0, st, k, v, groups);
  else if (dt == 1)
    hipLaunchKernelGGL((write_pair_kernel<KB, VB, 1>), grid, block, 0, st, k, v, groups);
  else
    hipLaunchKernelGGL((write_pair_kernel<KB, VB, 2>), grid, block, 0, st, k, v, groups);
  return hipGetLastError();
}

template <int KB>
static hipError_t launch_pair_k(const WriteArgs& k, const WriteArgs& v, int dt, int vb, hipStream_t st) {
  switch (vb) {
    case 2: return launch_pair_kv<KB, 2>(k, v, dt, st);
    case 3: return launch_pair_kv<KB, 3>(k, v, dt, st);
    case 4: return launch_pair_kv<KB, 4>(k, v, dt, st);
    case 5: return launch_pair_kv<KB, 5>(k, v, dt, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_write_pair(const WriteArgs& k, const WriteArgs& v, int raw_dtype, int k_bits, int v_bits,
                             hipStream_t stream) {
  if (k.num_rows == 0) return hipSuccess;
  switch (k_bits) {
    case 2: return launch_pair_k<2>(k, v, raw_dtype, v_bits, stream);
    case 3: return launch_pair_k<3>(k, v, raw_dtype, v_bits, stream);
    case 4: return launch_pair_k<4>(k, v, raw_dtype, v_bits, stream);
    case 5: return launch_pair_k<5>(k, v, raw_dtype, v_bits, stream);
  }
  return hipErrorInvalidValue;
}


}  // namespace tq
