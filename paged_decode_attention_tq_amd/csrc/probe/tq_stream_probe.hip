// Streaming-read ceiling for the decode's roofline: how fast plain 16-byte
// loads stream a large buffer from HBM on this device.  Measurement support
// for bench.py (library libtq_probe.so); not part of the TQ path or its ABI.
//
// Every thread reads 16-byte words with the non-temporal hint (the decode's
// page loads use the same hint), consecutive lanes at consecutive addresses
// (1 KB per wave instruction), eight loads in flight per thread, and folds
// them into one word that it writes once, so the loads are live.

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 512;
constexpr int kInFlight = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                               uint32_t* __restrict__ sink) {
  const size_t tid = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  size_t i = tid;
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[tid] = acc;
}

}  // namespace

// Read `bytes` (a multiple of 16) from `buf` once.  `sink` receives
// blocks * 512 words.  Device pointers; `stream` a hipStream_t (NULL: the
// default stream).  Returns the hipError_t of the launch.
extern "C" int tq_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, void* stream) {
  if (!buf || !sink || blocks <= 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15))
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return (int)hipGetLastError();
}
