// Rotary position embedding of the new Q and K rows and append of K/V into the block
// pool.  One workgroup per packed token: the d/2 angles p * base^(-2j/d) with their
// sines and cosines are computed once in float64 and shared by all heads of the token;
// each pair (x_j, x_{j+d/2}) is rotated in float64 and rounded once to the storage
// dtype.  Rotated Q goes back to its row; rotated K and raw V go to the token's slot
// (block_ids[p / bs], p % bs) of its sequence.  Block-indexed pools addressed through
// per-sequence block ids: "DeepSpeed Inference v2 source tour", sections "The front
// desk: put, query, can_schedule" and "Ragged batches".  The rotation itself is the
// textbook rotary embedding with half-split pairs (the pages do not describe it).
#include "rbkv_device.h"
#include "rbkv_internal.h"

namespace rbkv {
namespace {

constexpr int AP_THREADS = 256;

template <typename T, int D>
__global__ __launch_bounds__(AP_THREADS) void append_rotary_kernel(
    T* __restrict__ qkv, T* __restrict__ pool, const int32_t* __restrict__ tok2seq,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ block_off,
    const int32_t* __restrict__ block_ids, int32_t Hq, int32_t Hkv, int32_t bs, double base) {
#pragma clang fp contract(off)
  constexpr int VW = Elem<T>::VW;  // elements per 16 bytes
  constexpr int HV = (D / 2) / VW; // 16-byte vectors per half head
  constexpr int RV = D / VW;       // 16-byte vectors per head
  __shared__ double cs[D / 2], sn[D / 2];

  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t p = pos[t];
  const int32_t i = tok2seq[t];
  const bool rot = base > 0.0;
  if (rot) {
    for (int j = tid; j < D / 2; j += AP_THREADS) {
      const double theta = pow(base, -2.0 * (double)j / (double)D);
      const double a = (double)p * theta;
      double s, c;
      sincos(a, &s, &c);
      cs[j] = c;
      sn[j] = s;
    }
  }
  __syncthreads();

  const int64_t blk = block_ids[block_off[i] + p / bs];
  const int32_t slot = p % bs;
  T* row = qkv + (size_t)t * (Hq + 2 * Hkv) * D;
  const size_t kbase = ((size_t)blk * 2 + 0) * Hkv * bs * D + (size_t)slot * D;
  const size_t vbase = ((size_t)blk * 2 + 1) * Hkv * bs * D + (size_t)slot * D;
  const size_t head_stride = (size_t)bs * D;

  // Q heads (rotated in place) and K heads (rotated into the pool).
  const int nrot = (Hq + Hkv) * HV;
  for (int u = tid; u < nrot; u += AP_THREADS) {
    const int h = u / HV, c = u % HV;
    const T* x = row + (size_t)h * D;
    union V { u32x4 v; T e[VW]; } lo, hi, lo2, hi2;
    lo.v = ld16(x + c * VW);
    hi.v = ld16(x + D / 2 + c * VW);
    if (rot) {
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        const int j = c * VW + e;
        const double a = Elem<T>::to_f64(lo.e[e]);
        const double b = Elem<T>::to_f64(hi.e[e]);
        lo2.e[e] = Elem<T>::from_f64(a * cs[j] - b * sn[j]);
        hi2.e[e] = Elem<T>::from_f64(b * cs[j] + a * sn[j]);
      }
    } else {
      lo2 = lo;
      hi2 = hi;
    }
    if (h < Hq) {
      if (rot) {
        st16(row + (size_t)h * D + c * VW, lo2.v);
        st16(row + (size_t)h * D + D / 2 + c * VW, hi2.v);
      }
    } else {
      T* dst = pool + kbase + (size_t)(h - Hq) * head_stride;
      st16(dst + c * VW, lo2.v);
      st16(dst + D / 2 + c * VW, hi2.v);
    }
  }
  // V heads: copied unrotated.
  for (int u = tid; u < Hkv * RV; u += AP_THREADS) {
    const int g = u / RV, c = u % RV;
    const T* src = row + (size_t)(Hq + Hkv + g) * D + c * VW;
    T* dst = pool + vbase + (size_t)g * head_stride + c * VW;
    st16(dst, ld16(src));
  }
}

template <typename T, int D>
hipError_t launch_t(const rbkv_shape& s, const rbkv_batch& b, void* qkv, void* pool,
                    double base, hipStream_t stream) {
  hipLaunchKernelGGL((append_rotary_kernel<T, D>), dim3(b.T), dim3(AP_THREADS), 0, stream,
                     (T*)qkv, (T*)pool, b.token_to_seq, b.pos, b.block_offsets, b.block_ids,
                     s.n_q_heads, s.n_kv_heads, s.block_size, base);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append_rotary(const rbkv_shape& s, const rbkv_batch& b, void* qkv,
                                void* pool, double rope_base, hipStream_t stream) {
  const bool bf = s.dtype == RBKV_DTYPE_BF16;
  if (s.head_dim == 128)
    return bf ? launch_t<bf16_t, 128>(s, b, qkv, pool, rope_base, stream)
              : launch_t<float, 128>(s, b, qkv, pool, rope_base, stream);
  return bf ? launch_t<bf16_t, 64>(s, b, qkv, pool, rope_base, stream)
            : launch_t<float, 64>(s, b, qkv, pool, rope_base, stream);
}

}  // namespace rbkv
