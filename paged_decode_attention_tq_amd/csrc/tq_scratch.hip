// Scratch memory of the allocation-free decode entry point
// (tq_paged_decode_noalloc): one static device array, of which every GPU the
// library runs on holds its own copy from module load until the process
// ends.  Its device address is looked up once per device, with that device
// current, and kept; host code never uses the array's name as an address.

#include "tq_internal.h"

#include <mutex>

namespace tq {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

size_t scratch_bytes() { return kScratchBytes; }

void* scratch_device_ptr(hipError_t* err) {
  static std::mutex mu;
  static void* cache[64] = {};
  *err = hipSuccess;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!cache[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    cache[dev] = p;
  }
  return cache[dev];
}

}  // namespace tq
