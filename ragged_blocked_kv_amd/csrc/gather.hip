// Row gathers at the two ends of the ragged stream: the embedding rows of the packed
// tokens, and the last-token row of every sequence.  Both are pure HBM copies.  A
// workgroup copies one slice of up to 256 x U 16-byte words of one output row: its source
// row is looked up once (a uniform scalar load), then every lane issues its U loads
// before its U stores.  U (1, 2 or 4) follows the row width, so narrow rows do not leave
// lanes idle and wide rows still keep four loads in flight per lane.
#include "rbkv_internal.h"

namespace rbkv {
namespace {

constexpr int GT = 256;  // threads per workgroup

typedef int32_t w16 __attribute__((ext_vector_type(4)));  // one 16-byte word

// MODE 0: source row of output row r is idx[r] (zero row when outside [0, n_src));
// MODE 1: source row is idx[r + 1] - 1 (the last token of sequence r).
template <int MODE, int U>
__device__ __forceinline__ void gather_rows(const w16* __restrict__ src, w16* __restrict__ dst,
                                            const int32_t* __restrict__ idx, int32_t n_src,
                                            uint32_t vpr, uint32_t chunks) {
  const uint32_t r = blockIdx.x / chunks;
  const uint32_t c0 = (blockIdx.x - r * chunks) * (uint32_t)(GT * U) + threadIdx.x;
  const int32_t s = MODE == 0 ? idx[r] : idx[r + 1] - 1;
  const bool ok = MODE == 1 || (s >= 0 && s < n_src);
  const w16* sp = src + (size_t)(ok ? s : 0) * vpr;
  w16* dp = dst + (size_t)r * vpr;
  w16 v[U];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const uint32_t c = c0 + (uint32_t)k * GT;
    v[k] = __builtin_nontemporal_load(sp + (c < vpr ? c : vpr - 1));
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const uint32_t c = c0 + (uint32_t)k * GT;
    if (c < vpr) dp[c] = ok ? v[k] : w16{0, 0, 0, 0};
  }
}

template <int U>
__global__ __launch_bounds__(GT) void embedding_gather_kernel(const w16* __restrict__ src,
                                                              w16* __restrict__ dst,
                                                              const int32_t* __restrict__ ids,
                                                              int32_t n_src, uint32_t vpr,
                                                              uint32_t chunks) {
  gather_rows<0, U>(src, dst, ids, n_src, vpr, chunks);
}

template <int U>
__global__ __launch_bounds__(GT) void logits_gather_kernel(const w16* __restrict__ src,
                                                           w16* __restrict__ dst,
                                                           const int32_t* __restrict__ cu,
                                                           int32_t n_src, uint32_t vpr,
                                                           uint32_t chunks) {
  gather_rows<1, U>(src, dst, cu, n_src, vpr, chunks);
}

template <int MODE, int U>
void launch_u(const void* src, void* dst, const int32_t* idx, int32_t n_src, int32_t rows,
              uint32_t vpr, hipStream_t stream) {
  const uint32_t chunks = (vpr + GT * U - 1) / (GT * U);
  if (MODE == 0) {
    hipLaunchKernelGGL((embedding_gather_kernel<U>), dim3((uint32_t)rows * chunks), dim3(GT),
                       0, stream, (const w16*)src, (w16*)dst, idx, n_src, vpr, chunks);
  } else {
    hipLaunchKernelGGL((logits_gather_kernel<U>), dim3((uint32_t)rows * chunks), dim3(GT),
                       0, stream, (const w16*)src, (w16*)dst, idx, n_src, vpr, chunks);
  }
}

template <int MODE>
void launch_mode(const void* src, void* dst, const int32_t* idx, int32_t n_src, int32_t rows,
                 uint32_t vpr, hipStream_t stream) {
  if (vpr <= GT) {
    launch_u<MODE, 1>(src, dst, idx, n_src, rows, vpr, stream);
  } else if (vpr <= 2 * GT) {
    launch_u<MODE, 2>(src, dst, idx, n_src, rows, vpr, stream);
  } else {
    launch_u<MODE, 4>(src, dst, idx, n_src, rows, vpr, stream);
  }
}

}  // namespace

hipError_t launch_gather_rows(int mode, const void* src, void* dst, const int32_t* idx,
                              int32_t n_src, int32_t rows, size_t row_bytes,
                              hipStream_t stream) {
  const uint32_t vpr = (uint32_t)(row_bytes / 16);
  if (rows == 0 || vpr == 0) return hipSuccess;
  if (mode == 0) {
    launch_mode<0>(src, dst, idx, n_src, rows, vpr, stream);
  } else {
    launch_mode<1>(src, dst, idx, n_src, rows, vpr, stream);
  }
  return hipGetLastError();
}

}  // namespace rbkv
