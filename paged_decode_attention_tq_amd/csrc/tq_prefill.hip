// Multi-query (prefill / verify chunk) attention over packed pages for
// gfx950: the layout kernels around the decode.
//
// Sources: TurboQuant docs, "vLLM Usage", "Runtime Dispatch" (with a cache
// present, mixed prefill / decode batches attend through the packed cache)
// and "Architecture", "Cache Lifecycle".  Query j of the last q_len tokens
// of a sequence of length L sits at position P + j, P = L - q_len, and sees
// tokens 0 .. P + j.  Every query of the chunk sees the prefix 0 .. P, so the
// chunk's q_len x G queries of one KV head are decoded together as that
// many query heads over the prefix (the pages are read once); the chunk's
// other tokens P + 1 .. L - 1 are read back densely and attended causally by
// the window kernel, which merges both parts by their log-sum-exps.

#include "tq_internal.h"
#include "tq_device.h"

namespace tq {

namespace {

__device__ __forceinline__ int seq_len_of(const PrefillArgs& a, int b) { return min(max(a.seq_lens[b], 0), a.max_len); }
__device__ __forceinline__ int q_len_of(const PrefillArgs& a, int b, int L) {
  return min(max(a.q_lens[b], 0), min(a.q_len, L));
}

}  // namespace

// One workgroup of 256 threads per sequence b: the lengths and tail slots of
// b, and the query rows of b in decode order (16 bytes per thread and step).
__global__ __launch_bounds__(256) void prefill_prep_kernel(PrefillArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int L = seq_len_of(a, b), n = q_len_of(a, b, L), P = L - n;
  if (tid == 0) {
    a.prefix_lens[b] = n > 0 ? P + 1 : 0;
    a.tail_lens[b] = n > 0 ? n - 1 : 0;
  }
  for (int r = tid; r < a.q_len - 1; r += 256) {
    int64_t slot = -1;
    if (r < n - 1) {
      const int t = P + 1 + r;  // < L <= max_blocks_per_seq * block_size
      const int64_t blk = a.block_table[(int64_t)b * a.max_blocks_per_seq + t / a.block_size];
      slot = blk >= 0 ? blk * a.block_size + t % a.block_size : -1;  // a negative id names no page
    }
    a.tail_slots[(int64_t)b * (a.q_len - 1) + r] = slot;
  }
  const int Hq = a.num_q_heads, G = Hq / a.num_kv_heads, Lq = a.q_len;
  const int esz = a.q_dtype == 0 ? 4 : 2;
  const int rows = Lq * Hq, chunks = 128 * esz / 16;  // 16-byte pieces per row
  const uint8_t* src = static_cast<const uint8_t*>(a.q) + (int64_t)b * rows * 128 * esz;
  uint8_t* dst = static_cast<uint8_t*>(a.vq) + (int64_t)b * rows * 128 * esz;
  for (int e = tid; e < rows * chunks; e += 256) {
    const int row = e / chunks, c = e - row * chunks;  // row = j Hq + h of the input
    const int j = row / Hq, h = row - j * Hq, g = h / G, i = h - g * G;
    const int vrow = (g * Lq + j) * G + i;
    *reinterpret_cast<u32x4*>(dst + ((int64_t)vrow * chunks + c) * 16) =
        *reinterpret_cast<const u32x4*>(src + ((int64_t)row * chunks + c) * 16);
  }
}

// One wave per output row (b, j, h): out[b, j, h] = the decode-order row, or
// zeros for j >= q_len.
__global__ __launch_bounds__(256) void prefill_out_kernel(PrefillArgs a) {
  const int Hq = a.num_q_heads, G = Hq / a.num_kv_heads, Lq = a.q_len;
  const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= (int64_t)a.batch * Lq * Hq) return;
  const int lane = threadIdx.x & 63;
  const int b = (int)(unit / ((int64_t)Lq * Hq));
  const int row = (int)(unit - (int64_t)b * Lq * Hq), j = row / Hq, h = row - j * Hq;
  const int g = h / G, i = h - g * G;
  const int L = seq_len_of(a, b), n = q_len_of(a, b, L);
  float* o = a.out + unit * 128;
  if (j >= n) {
    *reinterpret_cast<float2*>(o + 2 * lane) = float2{0.0f, 0.0f};
    return;
  }
  const float* s = a.vout + ((int64_t)b * Lq * Hq + (g * Lq + j) * G + i) * 128;
  *reinterpret_cast<float2*>(o + 2 * lane) = *reinterpret_cast<const float2*>(s + 2 * lane);
}

hipError_t launch_prefill_prep(const PrefillArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_prep_kernel, dim3(a.batch), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill_out(const PrefillArgs& a, hipStream_t stream) {
  const int64_t units = (int64_t)a.batch * a.q_len * a.num_q_heads;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_out_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tq
