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
constexpr int CB_UNROLL = 8;  // splits whose partials are in flight together per lane

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
    // One pass with a running maximum, CB_UNROLL splits at a time so that their loads
    // overlap: rescaling by 2^(M_old - M_new) keeps num and den relative to the current
    // maximum, which gives the same quotient as scaling everything by 2^(m_s - max m).
    // The last batch re-reads the last split in its spare slots and gives them weight 0
    // (m = -inf), so every batch issues all its loads at once.
    float M = -INFINITY, num = 0.f, den = 0.f;
    for (int s = 0; s < ns; s += CB_UNROLL) {
      float mv[CB_UNROLL], lv[CB_UNROLL], av[CB_UNROLL];
#pragma unroll
      for (int j = 0; j < CB_UNROLL; ++j) {
        const float* p = p0 + (size_t)min(s + j, ns - 1) * stride;
        mv[j] = s + j < ns ? p[h] : -INFINITY;
        lv[j] = p[G + h];
        av[j] = p[2 * G + h * D + dim];
      }
      float mb = mv[0];
#pragma unroll
      for (int j = 1; j < CB_UNROLL; ++j) mb = fmaxf(mb, mv[j]);
      const float Mn = fmaxf(M, mb);
      const float sc = exp2f(M - Mn);  // 0 on the first batch (M = -inf)
      num *= sc;
      den *= sc;
#pragma unroll
      for (int j = 0; j < CB_UNROLL; ++j) {
        const float c = exp2f(mv[j] - Mn);
        den = fmaf(c, lv[j], den);
        num = fmaf(c, av[j], num);
      }
      M = Mn;
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
