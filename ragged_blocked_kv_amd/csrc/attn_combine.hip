// Log-sum-exp combine of split-K partials.  A split s of one (token, query head) left
// m_s (running max of the log2-scaled scores), l_s = sum 2^(z - m_s) and
// acc_s = sum 2^(z - m_s) v; with M = max_s m_s the output is
// sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s, rounded once to the storage dtype.
// (The blocked attention kernel of "DeepSpeed Inference v2 source tour", section
// "Ragged batches", writes through an output scratch; this is that scratch's reduction.)
#include "rbkv_device.h"
#include "rbkv_internal.h"

namespace rbkv {
namespace {

constexpr int CB_THREADS = 256;

template <typename T, int D>
__global__ __launch_bounds__(CB_THREADS) void combine_kernel(
    const float* __restrict__ ws, T* __restrict__ out, const int4* __restrict__ work,
    int32_t Hq, int32_t G) {
  const int4 w = work[blockIdx.x];
  const int32_t token = w.x, kvh = w.y, slot0 = w.z, ns = w.w;
  const size_t stride = (size_t)G * (D + 2);
  for (int u = threadIdx.x; u < G * D; u += CB_THREADS) {
    const int h = u / D, dim = u % D;
    const float* p0 = ws + (size_t)slot0 * stride;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, p0[s * stride + h]);
    float num = 0.f, den = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float* p = p0 + s * stride;
      const float c = exp2f(p[h] - M);
      den = fmaf(c, p[G + h], den);
      num = fmaf(c, p[2 * G + h * D + dim], num);
    }
    const float r = num / den;
    T* dst = out + ((size_t)token * Hq + (size_t)kvh * G + h) * D + dim;
    if constexpr (sizeof(T) == 2)
      ((uint16_t*)dst)[0] = (uint16_t)bf16_rne_f32(r);
    else
      ((float*)dst)[0] = r;
  }
}

template <typename T, int D>
hipError_t launch_t(const rbkv_shape& s, const rbkv_batch& b, const float* ws, void* out,
                    hipStream_t stream) {
  hipLaunchKernelGGL((combine_kernel<T, D>), dim3(b.n_combine_items), dim3(CB_THREADS), 0,
                     stream, ws, (T*)out, (const int4*)b.combine_work, s.n_q_heads,
                     s.n_q_heads / s.n_kv_heads);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const rbkv_shape& s, const rbkv_batch& b, const float* ws,
                          void* out, hipStream_t stream) {
  const bool bf = s.dtype == RBKV_DTYPE_BF16;
  if (s.head_dim == 128)
    return bf ? launch_t<bf16_t, 128>(s, b, ws, out, stream)
              : launch_t<float, 128>(s, b, ws, out, stream);
  return bf ? launch_t<bf16_t, 64>(s, b, ws, out, stream)
            : launch_t<float, 64>(s, b, ws, out, stream);
}

}  // namespace rbkv
