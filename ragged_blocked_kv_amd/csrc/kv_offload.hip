// KV block offload (pool blocks -> page-locked host memory) and restore (host -> pool
// blocks).  A pool block [2][Hkv][bs][d] is one contiguous slab, so a transfer is a list
// of slab copies between scattered pool blocks and consecutive host slabs.  One kernel
// does the whole list: a workgroup copies a 16 KiB slice of one slab, reading the slab's
// block id once from the id list the host staged at the end of the host buffer, and
// every lane issues its four 16-byte loads before its stores.  The host side of the copy
// goes straight over the host link (the buffer is mapped into the device address space),
// so no device staging memory is needed and the list costs one launch.
#include "rbkv_internal.h"

namespace rbkv {
namespace {

constexpr int KT_THREADS = 256;
constexpr int KU = 4;                    // 16-byte words per lane
constexpr int KW = KT_THREADS * KU;      // words per workgroup slice

typedef int32_t w16 __attribute__((ext_vector_type(4)));

// DIR 0: pool block ids[k] -> host slab k;  DIR 1: host slab k -> pool block ids[k].
template <int DIR>
__global__ __launch_bounds__(KT_THREADS) void kv_block_copy_kernel(w16* __restrict__ pool,
                                                                   w16* __restrict__ host,
                                                                   const int32_t* __restrict__ ids,
                                                                   uint32_t wpb,
                                                                   uint32_t chunks) {
  const uint32_t k = blockIdx.x / chunks;
  const uint32_t c0 = (blockIdx.x - k * chunks) * (uint32_t)KW + threadIdx.x;
  const int32_t id = ids[k];
  w16* dev = pool + (size_t)id * wpb;
  w16* hst = host + (size_t)k * wpb;
  const w16* src = DIR == 0 ? dev : hst;
  w16* dst = DIR == 0 ? hst : dev;
  w16 v[KU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const uint32_t c = c0 + (uint32_t)u * KT_THREADS;
    v[u] = __builtin_nontemporal_load(src + (c < wpb ? c : wpb - 1));
  }
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const uint32_t c = c0 + (uint32_t)u * KT_THREADS;
    if (c < wpb) __builtin_nontemporal_store(v[u], dst + c);
  }
}

}  // namespace

hipError_t launch_kv_block_copy(int dir, void* pool, void* host_dev, const int32_t* ids_dev,
                                int32_t n, size_t block_bytes, hipStream_t stream) {
  const uint32_t wpb = (uint32_t)(block_bytes / 16);
  if (n == 0 || wpb == 0) return hipSuccess;
  const uint32_t chunks = (wpb + KW - 1) / KW;
  const dim3 grid((uint32_t)n * chunks);
  if (dir == 0) {
    hipLaunchKernelGGL(kv_block_copy_kernel<0>, grid, dim3(KT_THREADS), 0, stream, (w16*)pool,
                       (w16*)host_dev, ids_dev, wpb, chunks);
  } else {
    hipLaunchKernelGGL(kv_block_copy_kernel<1>, grid, dim3(KT_THREADS), 0, stream, (w16*)pool,
                       (w16*)host_dev, ids_dev, wpb, chunks);
  }
  return hipGetLastError();
}

}  // namespace rbkv
