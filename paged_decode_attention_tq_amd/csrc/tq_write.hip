// Row writer kernel for gfx950: encodes raw K or V rows into TQ rows and
// stores them in the uint8 pages through flat slots.
//
// Row format: TurboQuant docs, "vLLM Usage" section "TQ Byte Layout"
// (ceil(128*bits/8) bytes of LSB-first packed codebook indices, then the
// fp32 norm); slots: "vLLM Usage" section "Slot Mapping" (negative slots are
// ignored, out-of-range slots are an error); pages: "Architecture" section
// "Cache Storage Objects" ([num_blocks, block_size, num_kv_heads, row_bytes]).

#include "tq_encode.h"

#include <algorithm>

namespace tq {

// ==========================================================================
// Row writer: one row (token, head) per 4-lane quad, 32 elements per lane,
// encoded as tq_encode.h describes and stored at the row's slot.
// ==========================================================================

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

// The rows of workgroup `wg` (64 rows, one per 4-lane quad) of one call.
template <int BITS, int DT>
__device__ __forceinline__ void write_rows(const WriteArgs& a, int64_t wg) {
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

  uint8_t* dst = a.pages + (slot / a.block_size) * a.page_bytes +
                 ((slot % a.block_size) * a.num_kv_heads + head) * (int64_t)a.row_bytes;
  encode_store_row<BITS>(x, q, a.sign_bits, a.pos_bounds, dst, a.row_bytes);
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
// Appending row writer: one row per quad, row r = 2 (b Hkv + head) + comp.
// The last token of sequence b is L_b - 1 (L_b its length clamped to
// 0 .. max_len); an empty sequence has no new row, and a last page whose
// block id lies outside the pages is counted once (by its K row of head 0)
// and not written.
// ==========================================================================
template <int KB, int VB>
__global__ __launch_bounds__(256) void write_append_kernel(AppendWriteArgs a) {
  const int q = threadIdx.x & 3;
  const int64_t r = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
  if (r >= 2LL * a.batch * a.num_kv_heads) return;  // uniform per quad
  const int comp = (int)(r & 1);
  const int64_t bh = r >> 1;
  const int b = (int)(bh / a.num_kv_heads);
  const int head = (int)(bh - (int64_t)b * a.num_kv_heads);
  // the raw row and the length are read together; the block id follows
  float x[32];
  load_row_any(comp == 0 ? a.app.k_new : a.app.v_new, a.app.new_dtype, bh * kHeadDim + 32 * q, x);
  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  if (L <= 0) return;
  const int blk = a.block_table[(int64_t)b * a.max_blocks_per_seq + (L - 1) / kBlockSize];
  if (blk < 0 || (int64_t)blk >= a.num_blocks) {
    if (comp == 0 && head == 0 && q == 0 && a.app.err_count) atomicAdd(a.app.err_count, 1);
    return;
  }
  const int64_t tok_row = (int64_t)((L - 1) % kBlockSize) * a.num_kv_heads + head;
  if (comp == 0)
    encode_store_row<KB>(x, q, a.sign_bits, a.app.k_bounds,
                         a.k_pages + (int64_t)blk * a.k_page_bytes + tok_row * a.k_row_bytes, a.k_row_bytes);
  else
    encode_store_row<VB>(x, q, a.sign_bits, a.app.v_bounds,
                         a.v_pages + (int64_t)blk * a.v_page_bytes + tok_row * a.v_row_bytes, a.v_row_bytes);
}

template <int KB>
static hipError_t launch_write_append_k(const AppendWriteArgs& a, int v_bits, dim3 grid, hipStream_t st) {
  switch (v_bits) {
    case 2: hipLaunchKernelGGL((write_append_kernel<KB, 2>), grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL((write_append_kernel<KB, 3>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((write_append_kernel<KB, 4>), grid, dim3(256), 0, st, a); break;
    case 5: hipLaunchKernelGGL((write_append_kernel<KB, 5>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_write_append(const AppendWriteArgs& a, int k_bits, int v_bits, hipStream_t stream) {
  const long long rows = 2LL * a.batch * a.num_kv_heads;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 63) / 64));
  switch (k_bits) {
    case 2: return launch_write_append_k<2>(a, v_bits, grid, stream);
    case 3: return launch_write_append_k<3>(a, v_bits, grid, stream);
    case 4: return launch_write_append_k<4>(a, v_bits, grid, stream);
    case 5: return launch_write_append_k<5>(a, v_bits, grid, stream);
  }
  return hipErrorInvalidValue;
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
