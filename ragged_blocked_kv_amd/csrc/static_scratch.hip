// The library's own split-K scratch for ragged_blocked_attention_noalloc: a fixed-size
// device array, one copy per GPU the library runs on, held until the process ends.
//
// Host code never passes the array's name to a kernel (on the host it is only a stand-in
// for the symbol): static_scratch() resolves the array's address on the current device
// once, with hipGetSymbolAddress, keeps it per device, and every later use (kernel
// arguments) takes that address.
#include <mutex>

#include "rbkv_internal.h"

namespace rbkv {

__device__ __align__(256) unsigned char scratch[RBKV_STATIC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace rbkv
