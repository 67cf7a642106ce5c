// Dense readback of TQ rows for gfx950: rows stored in the uint8 pages are
// reconstructed as x = n * s * (H c[idx]) / sqrt(128) and written to a dense
// [num_tokens, num_kv_heads, 128] buffer through flat slots.
//
// Sources: TurboQuant docs, "Architecture" section "Data Flow" (packed bytes
// lead to a diagnostic dense reconstruction, separate from compressed
// attention) and "vLLM Reference Audit", File Map row "TQ4 unpack kernel"
// (packed index bytes and norms in, rows out, into a caller's buffer); row
// format "vLLM Usage" section "TQ Byte Layout"; slots "vLLM Usage" section
// "Slot Mapping".

#include "tq_internal.h"
#include "tq_device.h"

#include <algorithm>

namespace tq {

// ==========================================================================
// One row (token, head) per 4-lane quad, 32 coordinates per lane, 64 rows per
// 256-thread workgroup.  Lane q of a quad holds indices 32q..32q+31, which
// are exactly the BITS dwords q*BITS..q*BITS+BITS-1 of the row's bit stream,
// so each lane reads its own words.  The kernel is bound by VALU issue (about
// twelve instructions per coordinate), so each step takes the fewest:
//
// * centroids: lane l holds c[l mod 2^BITS], and ds_bpermute picks its source
//   lane from bits 2..7 of a byte address and ignores the bits above, so one
//   shift (or funnel shift) that moves an index field to bit 2 is the whole
//   address: the neighbouring fields above it only select another copy;
// * inverse transform: the Walsh-Hadamard butterfly, five stages inside the
//   lane (one add or subtract per coordinate) and two across the quad as one
//   fused DPP multiply-add per coordinate, x += s * partner(x) with s = +-1
//   per lane.  That form leaves lanes whose quad index has odd parity
//   holding the negated value; the final sign step absorbs it;
// * signs and scale: one multiply by n / sqrt(128), then the sign bit of the
//   coordinate (the rotation sign times that parity, a word per quad lane
//   built on the host) XORed in.
//
// The output rows leave through a per-wave LDS transpose (see the kernel).
// ==========================================================================

// The output words of a lane's 32 coordinates: 32 fp32 words, or 16 words of
// two fp16 / bf16 values each (packed conversions, round to nearest even).
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int ODT>
__device__ __forceinline__ void out_words(const float (&x)[32], uint32_t (&w)[ODT == 0 ? 32 : 16]) {
#pragma unroll
  for (int k = 0; k < (ODT == 0 ? 32 : 16); ++k) {
    if constexpr (ODT == 0) {
      w[k] = __float_as_uint(x[k]);
    } else {
      const floatx2 v = {x[2 * k], x[2 * k + 1]};
      if constexpr (ODT == 1)
        w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, halfx2));
      else
        w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    }
  }
}

// This lane's row of 64-row block blk (clamped to the last row, so a block
// past the end reads valid memory) and the slot of its token.
struct RowRef {
  uint32_t row;
  int head;
  int64_t slot;
};

__device__ __forceinline__ RowRef row_ref(const ReadArgs& a, uint32_t blk) {
  const uint32_t r = min(blk * 64u + (threadIdx.x >> 2), a.num_rows - 1);
  const uint32_t tok = a.hkv_shift >= 0 ? r >> a.hkv_shift : r / (uint32_t)a.num_kv_heads;
  return RowRef{r, (int)(r - tok * (uint32_t)a.num_kv_heads), a.slots[tok]};
}

// Lane q's BITS index words of the row and its norm (zeros for a slot that
// names no stored row).
template <int BITS>
__device__ __forceinline__ void load_words(const ReadArgs& a, const RowRef& r, int q, uint32_t (&w)[BITS],
                                           float& nrm) {
#pragma unroll
  for (int k = 0; k < BITS; ++k) w[k] = 0;
  nrm = 0.0f;
  if (r.slot >= 0 && r.slot < a.num_slots) {
    const uint8_t* row;
    if (a.num_slots <= (int64_t)0xFFFFFFFF) {  // 32-bit slot arithmetic
      const uint32_t s32 = (uint32_t)r.slot;
      const uint32_t page = a.bs_shift >= 0 ? s32 >> a.bs_shift : s32 / (uint32_t)a.block_size;
      const uint32_t off = s32 - page * (uint32_t)a.block_size;
      row = a.pages + (uint64_t)page * (uint32_t)a.page_bytes +
            (off * (uint32_t)a.num_kv_heads + (uint32_t)r.head) * (uint32_t)a.row_bytes;
    } else {
      const int64_t page = r.slot / a.block_size, off = r.slot - page * a.block_size;
      row = a.pages + page * a.page_bytes + (off * a.num_kv_heads + r.head) * (int64_t)a.row_bytes;
    }
    const uint32_t* src = reinterpret_cast<const uint32_t*>(row);
#pragma unroll
    for (int k = 0; k < BITS; ++k) w[k] = src[BITS * q + k];
    nrm = __uint_as_float(src[4 * BITS]);  // the norm follows the 16 * BITS index bytes
  }
}

// x[j] += s * (x[j] of the lane XOR-paired by CTRL), for 16 coordinates, as
// fused DPP multiply-adds.  The leading s_nop gives the two wait states a DPP
// read needs after a VALU write of its source; inside the block every read
// register was written at least 16 instructions earlier.
#define TQ_FMAC_DPP16(CTRL)                                                                              \
  asm volatile(                                                                                          \
      "s_nop 1\n"                                                                                        \
      "v_fmac_f32_dpp %0, %0, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"                                 \
      "v_fmac_f32_dpp %1, %1, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"                                 \
      "v_fmac_f32_dpp %2, %2, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"                                 \
      "v_fmac_f32_dpp %3, %3, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"                                 \
      "v_fmac_f32_dpp %4, %4, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"                                 \
      "v_fmac_f32_dpp %5, %5, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"                                 \
      "v_fmac_f32_dpp %6, %6, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"                                 \
      "v_fmac_f32_dpp %7, %7, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"                                 \
      "v_fmac_f32_dpp %8, %8, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"                                 \
      "v_fmac_f32_dpp %9, %9, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"                                 \
      "v_fmac_f32_dpp %10, %10, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"                               \
      "v_fmac_f32_dpp %11, %11, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"                               \
      "v_fmac_f32_dpp %12, %12, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"                               \
      "v_fmac_f32_dpp %13, %13, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"                               \
      "v_fmac_f32_dpp %14, %14, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"                               \
      "v_fmac_f32_dpp %15, %15, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"                               \
      : "+v"(x[o + 0]), "+v"(x[o + 1]), "+v"(x[o + 2]), "+v"(x[o + 3]), "+v"(x[o + 4]), "+v"(x[o + 5]),    \
        "+v"(x[o + 6]), "+v"(x[o + 7]), "+v"(x[o + 8]), "+v"(x[o + 9]), "+v"(x[o + 10]), "+v"(x[o + 11]),  \
        "+v"(x[o + 12]), "+v"(x[o + 13]), "+v"(x[o + 14]), "+v"(x[o + 15])                                \
      : "v"(s))

// Reconstruct lane q's 32 coordinates of one row from its words and norm.
template <int BITS>
__device__ __forceinline__ void reconstruct(const ReadArgs& a, float cl, int q, const uint32_t (&w)[BITS], float nrm,
                                            float (&x)[32]) {
  // indices -> centroids (byte address = the field moved to bit 2)
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int pos = BITS * j, wi = pos >> 5, sh = pos & 31;
    uint32_t addr;
    if (sh + BITS > 32)
      addr = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh - 2);  // field split over two words
    else if (sh >= 2)
      addr = w[wi] >> (sh - 2);
    else
      addr = w[wi] << (2 - sh);
    x[j] = __int_as_float(__builtin_amdgcn_ds_bpermute((int)addr, __float_as_int(cl)));
  }
  // inverse transform: five butterfly stages inside the lane
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
  // two across the quad: the upper lane of each pair keeps its negated
  // butterfly output, which the sign masks undo
  {
    const float s = (q & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int o = 0; o < 32; o += 16) TQ_FMAC_DPP16("quad_perm:[1,0,3,2]");
  }
  {
    const float s = (q & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int o = 0; o < 32; o += 16) TQ_FMAC_DPP16("quad_perm:[2,3,0,1]");
  }
  // n / sqrt(128), then the sign of each coordinate: bit j of the lane's
  // negation word moved to the float sign bit
  const float f = nrm * 0.08838834764831845f;
  uint32_t nw = pick4(a.neg_bits, q);
  asm volatile("" : "+v"(nw));  // one register per block, not 32 masks kept live across the loop
#pragma unroll
  for (int j = 0; j < 32; ++j) x[j] = __uint_as_float(__float_as_uint(x[j] * f) ^ ((nw << (31 - j)) & 0x80000000u));
}

#undef TQ_FMAC_DPP16

// Grid-stride over 64-row blocks, software-pipelined: the slots of the block
// two steps ahead and the words of the block one step ahead are loaded
// before the current block is reconstructed and stored, so both dependent
// loads overlap the work of a whole block.
template <int BITS, int ODT>
__global__ __launch_bounds__(256) void decompress_rows_kernel(ReadArgs a) {
  const int q = threadIdx.x & 3;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // lanes 0..2^BITS-1 hold the centroid table; every lane stays active
  // through the shuffles, so a lane past the last row computes a clamped row
  // and only skips its store
  const float cl = cent_of_lane<BITS>(a.cent, lane & ((1 << BITS) - 1));
  const uint32_t nblk = (a.num_rows + 63) / 64;
  const uint32_t step = gridDim.x;

  // The wave's 16 rows are consecutive in out.  Each lane's 16-byte chunks go
  // to a wave-private LDS block in row order (one spare chunk after every
  // four, so the writes of neighbouring lanes fall on different banks), then
  // every lane takes chunk lane + 64 i back: each store instruction of the
  // wave covers 1 KB of contiguous output instead of 64 strided pieces.
  constexpr int kWords = ODT == 0 ? 32 : 16;       // output words per lane
  constexpr int kChunks = kWords / 4;              // 16-byte chunks per lane
  constexpr int kWaveChunks = 64 * kChunks;        // chunks of the wave's 16 rows
  constexpr int kRowChunks = 4 * kChunks;          // chunks of one output row
  __shared__ u32x4 stage[4][kWaveChunks + kWaveChunks / 4];

  uint32_t blk = blockIdx.x;
  RowRef cur = row_ref(a, blk), nxt = row_ref(a, blk + step);
  uint32_t w[BITS];
  float nrm;
  load_words<BITS>(a, cur, q, w, nrm);
  for (; blk < nblk; blk += step) {
    const RowRef nn = row_ref(a, blk + 2 * step);
    uint32_t wn[BITS];
    float nrmn;
    load_words<BITS>(a, nxt, q, wn, nrmn);

    const bool live = blk * 64u + (threadIdx.x >> 2) < a.num_rows;
    if (live && q == 0 && cur.head == 0 && cur.slot >= a.num_slots && a.err_count) atomicAdd(a.err_count, 1);
    float x[32];
    reconstruct<BITS>(a, cl, q, w, nrm, x);

    uint32_t ow[kWords];
    out_words<ODT>(x, ow);
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int c = lane * kChunks + j;
      stage[wave][c + (c >> 2)] = u32x4{ow[4 * j], ow[4 * j + 1], ow[4 * j + 2], ow[4 * j + 3]};
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint32_t row0 = blk * 64u + wave * 16u;  // first row of the wave
    u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint8_t*>(a.out) + (int64_t)row0 * (16 * kRowChunks));
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = lane + 64 * i;
      if (row0 + (uint32_t)(c / kRowChunks) < a.num_rows) dst[c] = stage[wave][c + (c >> 2)];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // the block's reads of the stage precede the next block's writes

    cur = nxt;
    nxt = nn;
#pragma unroll
    for (int k = 0; k < BITS; ++k) w[k] = wn[k];
    nrm = nrmn;
  }
}

// Workgroups per CU, all resident at once: 6 with fp16 / bf16 out (20 KB of
// LDS and at most 80 VGPRs: 6 waves per SIMD), 4 with fp32 out (40 KB of LDS).
template <int BITS>
static hipError_t launch_decompress_bits(const ReadArgs& a, int odt, int num_cus, hipStream_t st) {
  const uint32_t nblk = (a.num_rows + 63) / 64;
  const dim3 grid(std::min<uint32_t>(nblk, (uint32_t)num_cus * (odt == 0 ? 4u : 6u))), block(256);
  if (odt == 0)
    hipLaunchKernelGGL((decompress_rows_kernel<BITS, 0>), grid, block, 0, st, a);
  else if (odt == 1)
    hipLaunchKernelGGL((decompress_rows_kernel<BITS, 1>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((decompress_rows_kernel<BITS, 2>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decompress(const ReadArgs& a, int bits, int out_dtype, int num_cus, hipStream_t stream) {
  if (a.num_rows == 0) return hipSuccess;
  switch (bits) {
    case 2: return launch_decompress_bits<2>(a, out_dtype, num_cus, stream);
    case 3: return launch_decompress_bits<3>(a, out_dtype, num_cus, stream);
    case 4: return launch_decompress_bits<4>(a, out_dtype, num_cus, stream);
    case 5: return launch_decompress_bits<5>(a, out_dtype, num_cus, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
