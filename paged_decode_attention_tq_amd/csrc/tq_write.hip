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

// The same row slice as raw words: loads issued now, widened later.
template <int DT>
struct RawSlice {
  u32x4 v[DT == 0 ? 8 : 4];
};

template <int DT>
__device__ __forceinline__ void fetch_raw(const void* raw, int64_t elem_off, RawSlice<DT>& r) {
  const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(raw) + elem_off * (DT == 0 ? 4 : 2));
#pragma unroll
  for (int i = 0; i < (DT == 0 ? 8 : 4); ++i) r.v[i] = p[i];
}

template <int DT>
__device__ __forceinline__ void widen_raw(const RawSlice<DT>& r, float (&x)[32]) {
#pragma unroll
  for (int i = 0; i < (DT == 0 ? 8 : 4); ++i) {
    const uint32_t w[4] = {r.v[i].x, r.v[i].y, r.v[i].z, r.v[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (DT == 0) {
        x[4 * i + k] = __uint_as_float(w[k]);
      } else if constexpr (DT == 1) {
        x[8 * i + 2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] & 0xFFFF));
        x[8 * i + 2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] >> 16));
      } else {
        x[8 * i + 2 * k] = bf16_to_f32((uint16_t)(w[k] & 0xFFFF));
        x[8 * i + 2 * k + 1] = bf16_to_f32((uint16_t)(w[k] >> 16));
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
// A workgroup takes 64 rows at a time.  The front end is the MSE writer's,
// a quad per row (load, norm, rotation, boundary count), and leaves the
// residual in the quad's registers; they go to LDS as fp16 hi + lo after a
// power-of-two scaling per row.  The sketch P = E S^T of the 64 rows is a
// dense product on MFMA (v_mfma_f32_16x16x32_f16): wave w forms outputs
// 32 w .. 32 w + 31 of every row, with its 32 rows of S (fp16 hi + lo, a
// power-of-two scale per row) held in registers for the whole launch, as
// e_hi s_hi + e_lo s_hi + e_hi s_lo (the dropped lo lo term is below 2^-22
// of sum_j |S_ij e_j|).  Positive scales leave every sign as it is.  The
// signs are OR-ed across lanes into word w of each row, and the front
// end's quads store whole rows.  Persistent grid; a quad's next raw row is
// loaded while the current block's sketch runs.
// ==========================================================================
// E stage row stride in halves: 16 bytes of padding put the 16 rows that a
// quarter-wave of ds_read_b128 reads on distinct banks
constexpr int kEStride = 136;

template <int BITS, int DT>
__global__ __launch_bounds__(256, 2) void write_prod_kernel(ProdWriteArgs pa) {  // two workgroups per CU
  constexpr int MB = BITS - 1, N = 1 << MB, HALF = N / 2;
  __shared__ __align__(16) _Float16 ehi[64 * kEStride];
  __shared__ __align__(16) _Float16 elo[64 * kEStride];
  __shared__ uint32_t sgn[64 * 5];
  const WriteArgs& a = pa.w;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = tid & 3, rl = tid >> 2;     // front end: quad lane, row of the 64
  const int n = lane & 15, c = lane >> 4;   // MFMA: row / column n, k-slots 8 c .. 8 c + 7
  const uint32_t bit_lo = 1u << n, bit_hi = 1u << (n + 16);

  // B operand: S rows 32 wave + 16 t + n, coordinates 32 ks + 8 c .. + 7
  half8 sh[2][4], sl[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float* srow = pa.sketch + (int64_t)(32 * wave + 16 * t + n) * kHeadDim + 8 * c;
    float v[4][8];
    float mx = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const floatx4 v0 = *reinterpret_cast<const floatx4*>(srow + 32 * ks);
      const floatx4 v1 = *reinterpret_cast<const floatx4*>(srow + 32 * ks + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[ks][j] = v0[j], v[ks][4 + j] = v1[j];
        mx = fmaxf(mx, fmaxf(__builtin_fabsf(v0[j]), __builtin_fabsf(v1[j])));
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float sc = pow2_scale(mx);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float y = v[ks][j] * sc;
        const _Float16 h = (_Float16)y;
        sh[t][ks][j] = h;
        sl[t][ks][j] = (_Float16)(y - (float)h);
      }
    }
  }

  // lane l < 2^MB holds centroid l of the index codebook (-cpos[HALF - 1 - l]
  // below HALF, cpos[l - HALF] from HALF); the residual looks it up by index
  float cent = 0.0f;
#pragma unroll
  for (int k = 0; k < HALF; ++k) {
    cent = (lane & (N - 1)) == HALF + k ? pa.cpos[k] : cent;
    cent = (lane & (N - 1)) == HALF - 1 - k ? -pa.cpos[k] : cent;
  }
  const int64_t nblk = (a.num_rows + 63) / 64;
  // the raw slice and slot of this quad's row of block b, requested one
  // block ahead (in flight during the previous block's sketch and stores)
  RawSlice<DT> pre;
  int64_t pre_slot = -1;
  auto issue = [&](int64_t b) {
    const int64_t row = b * 64 + rl;
    if (b < nblk && row < a.num_rows) {  // uniform per quad
      pre_slot = a.slots[row / a.num_kv_heads];
      fetch_raw<DT>(a.raw, row * kHeadDim + 32 * q, pre);
    }
  };
  issue(blockIdx.x);
  for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    // ---- front end: row blk * 64 + rl on quad rl ---------------------------
    const int64_t row = blk * 64 + rl;
    int64_t slot = -1;
    int head = 0;
    float x[32];
    if (row < a.num_rows) {  // uniform per quad
      head = (int)(row % a.num_kv_heads);
      slot = pre_slot;
      widen_raw<DT>(pre, x);
      if (slot >= a.num_slots) {
        if (q == 0 && head == 0 && a.err_count) atomicAdd(a.err_count, 1);
        slot = -1;
      }
    }
    if (slot < 0) {  // nothing to store: the row's work runs on zeros
#pragma unroll
      for (int j = 0; j < 32; ++j) x[j] = 0.0f;
    }
    const double n64 = row_norm(x);
    const float n32 = (float)n64;
    const float cn = n64 > 0.0 ? (float)(1.0 / (n64 * 11.313708498984761)) : 0.0f;  // 1/(n sqrt(128))
    rotate_row(a.sign_bits, q, x);

    // indices at MB bits and the residual (kept in x), its squared norm
    uint32_t w[MB];
#pragma unroll
    for (int k = 0; k < MB; ++k) w[k] = 0;
    float ss = 0.0f, mx = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float r = x[j] * cn;
      const float ar = __builtin_fabsf(r);
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < HALF - 1; ++k) cnt += (ar > a.pos_bounds[k]) ? 1 : 0;
      const uint32_t idx = (uint32_t)(r > 0.0f ? HALF + cnt : HALF - 1 - cnt);
      const int pos = MB * j;
      w[pos >> 5] |= idx << (pos & 31);
      if ((pos & 31) + MB > 32) w[(pos >> 5) + 1] |= idx >> (32 - (pos & 31));
      x[j] = r - __shfl(cent, (int)idx);  // the same fp32 value as r - (+-cpos[cnt])
      ss = fmaf(x[j], x[j], ss);
      mx = fmaxf(mx, __builtin_fabsf(x[j]));
    }
    ss += quad_xor<1>(ss);
    ss += quad_xor<2>(ss);
    const float gamma = __builtin_sqrtf(ss);
    mx = fmaxf(mx, quad_xor<1>(mx));
    mx = fmaxf(mx, quad_xor<2>(mx));
    {
      // the residual, scaled by a power of two, as fp16 hi and lo
      const float sc = pow2_scale(mx);
      uint32_t hw[16], lw[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float y0 = x[2 * j] * sc, y1 = x[2 * j + 1] * sc;
        const _Float16 h0 = (_Float16)y0, h1 = (_Float16)y1;
        hw[j] = pack_half2(h0, h1);
        lw[j] = pack_half2((_Float16)(y0 - (float)h0), (_Float16)(y1 - (float)h1));
      }
      u32x4* dh = reinterpret_cast<u32x4*>(ehi + rl * kEStride + 32 * q);
      u32x4* dl = reinterpret_cast<u32x4*>(elo + rl * kEStride + 32 * q);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        dh[k] = u32x4{hw[4 * k], hw[4 * k + 1], hw[4 * k + 2], hw[4 * k + 3]};
        dl[k] = u32x4{lw[4 * k], lw[4 * k + 1], lw[4 * k + 2], lw[4 * k + 3]};
      }
    }
    __syncthreads();
    issue(blk + gridDim.x);

    // ---- sketch: outputs 32 wave .. 32 wave + 31 of the 64 rows ------------
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      floatx4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int at = (16 * rt + n) * kEStride + 32 * ks + 8 * c;
        const half8 ah = *reinterpret_cast<const half8*>(ehi + at);
        const half8 al = *reinterpret_cast<const half8*>(elo + at);
        p0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, sh[0][ks], p0, 0, 0, 0);
        p1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, sh[1][ks], p1, 0, 0, 0);
        p0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, sh[0][ks], p0, 0, 0, 0);
        p1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, sh[1][ks], p1, 0, 0, 0);
        p0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, sl[0][ks], p0, 0, 0, 0);
        p1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, sl[1][ks], p1, 0, 0, 0);
      }
      // lane (n, c) holds rows 16 rt + 4 c + r of outputs 32 wave + n (p0)
      // and 32 wave + 16 + n (p1): bits n and n + 16 of the row's word
      // `wave`, OR-ed across the 16 lanes of the row group
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t v = (p0[r] >= 0.0f ? bit_lo : 0u) | (p1[r] >= 0.0f ? bit_hi : 0u);
        v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
        v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
        v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false);  // row_ror:4
        v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
        if (n == 0) sgn[(16 * rt + 4 * c + r) * 5 + wave] = v;
      }
    }
    __syncthreads();

    // ---- the whole row -------------------------------------------------------
    if (slot >= 0) {
      const uint32_t zw = sgn[rl * 5 + q];
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
}

template <int BITS>
static hipError_t launch_prod_bits(const ProdWriteArgs& a, int dt, int num_cus, hipStream_t st) {
  const int64_t nblk = (a.w.num_rows + 63) / 64;
  const dim3 grid((unsigned)std::min<int64_t>(nblk, 2LL * num_cus)), block(256);  // two per CU (registers)
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
