// Device-side helpers for the gfx950 kernels: storage types, conversions, 16-byte
// vector access and wavefront reductions (64 lanes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rbkv {

// bfloat16 is carried as its 16-bit pattern.
struct bf16_t {
  uint16_t bits;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bfloat16 pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_f32(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
typedef float f32x2v __attribute__((ext_vector_type(2)));
// Two floats -> packed bfloat16 pair (lo in bits 0..15), round to nearest even; one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// float64 -> bfloat16 pattern, round to nearest even in one step from binary64: drop
// the low 45 fraction bits with RNE, the result is exact in binary32.
__device__ __forceinline__ uint16_t bf16_rne_f64(double x) {
  unsigned long long u = (unsigned long long)__double_as_longlong(x);
  u = (u + ((1ull << 44) - 1ull) + ((u >> 45) & 1ull)) & ~((1ull << 45) - 1ull);
  const float f = (float)__longlong_as_double((long long)u);
  return (uint16_t)(__float_as_uint(f) >> 16);
}

// Storage traits: element <-> float32/float64 and how many elements fill 16 bytes.
template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int VW = 4;
  __device__ static __forceinline__ double to_f64(float v) { return (double)v; }
  __device__ static __forceinline__ float from_f64(double v) { return (float)v; }
};
template <>
struct Elem<bf16_t> {
  static constexpr int VW = 8;
  __device__ static __forceinline__ double to_f64(bf16_t v) {
    return (double)__uint_as_float((uint32_t)v.bits << 16);
  }
  __device__ static __forceinline__ bf16_t from_f64(double v) { return bf16_t{bf16_rne_f64(v)}; }
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *(u32x4*)p = v; }

// DPP lane moves within a row of 16 lanes (row_mask / bank_mask all set).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xF, 0xF, false));
}
// Max / sum over each row of 16 lanes, result in every lane of the row: swap neighbours,
// swap pairs, mirror within 8, mirror within 16.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  return fmaxf(v, dpp_mov<0x140>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  return v + dpp_mov<0x140>(v);
}
__device__ __forceinline__ float lane_of(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// Wavefront-wide max / sum, uniform result (rows reduced with DPP, then 4 lane reads).
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_of(v, 0), lane_of(v, 16)), fmaxf(lane_of(v, 32), lane_of(v, 48)));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = row16_sum(v);
  return (lane_of(v, 0) + lane_of(v, 16)) + (lane_of(v, 32) + lane_of(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// HBM -> LDS without registers (global_load_lds_dwordx4): lane l writes its 16 bytes at
// LDS byte address m0 + 16*l, m0 = lds (wave-uniform).  Written as inline assembly so the
// compiler does not track the LDS write: it cannot tell the ring stages apart and would
// otherwise wait for every load in flight before each LDS read, which serialises the
// tile pipeline.  The kernel orders these writes against its reads itself (explicit
// vmcnt waits, then a workgroup barrier).  The compiler writes m0 for the operand; one
// wait state separates that write from the load that uses it.
__device__ __forceinline__ void load_lds16(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds) : "memory");
}
// The same with the non-temporal cache policy, for data read once.
__device__ __forceinline__ void load_lds16_nt(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(src), "{m0}"(lds) : "memory");
}

// From a uniform 64-bit base (scalar registers) plus a 32-bit lane offset, which keeps one
// vector register per load address instead of two.
__device__ __forceinline__ void load_lds16_s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(lds) : "memory");
}
// The same with the non-temporal cache policy.
__device__ __forceinline__ void load_lds16_nt_s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(off), "s"(base), "{m0}"(lds) : "memory");
}

// Wait until at most n vector-memory operations of this wave are outstanding (the LDS
// DMA loads of later tiles stay in flight); expcnt and lgkmcnt are left alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace rbkv
