// Decode of one split-K work item on the matrix cores, for bf16 caches at head dim 128 over
// blocks of at least 64 keys and groups of up to 16 query heads.  Device code shared by the
// decode kernel (four wavefronts per workgroup) and the mixed prefill/decode kernel (eight).
//
// The NW wavefronts of the workgroup split the item's keys into steps of 16 NW keys; wave w
// takes keys 16w .. 16w+15 of every step (a 16-key slice never crosses a block) and runs its
// own pipeline with no workgroup barrier: its K and V rows go from HBM straight into its own
// LDS slices (global_load_lds_dwordx4, ST stages, the next slices in flight while this one
// is computed).  Per step and wave:
//   S^T = K Q^T     v_mfma_f32_16x16x32_bf16 over four 32-dim steps: rows are the wave's 16
//                   keys, columns the group's query heads (columns past G hold zeros), K
//                   fragments from LDS, Q^T in registers for the whole item;
//   online softmax  lane (g, j) holds the scores of keys 4g..4g+3 for head j, so the
//                   running maximum of head j is lane-local once the four lane groups
//                   agree; it moves only past a slack of 2^8 (a cross-lane max when a lane
//                   asks for it), and the weights are rounded to bf16 as they are summed;
//   O^T += V^T P^T  v_mfma_f32_16x16x16_bf16 per 16-dim block: the weights are already in
//                   the operand layout (the S^T accumulator layout), V^T fragments come from
//                   transposing LDS reads (ds_read_b64_tr_b16).
// K slices carry the XOR swizzle chunk ^ key % 16 (fragment reads hit 16 distinct bank
// groups), V slices chunk ^ 2 (key % 8) (each half-wave of a transposing read covers 64
// banks).  At the end of the item each wave leaves its unnormalised output in its own LDS
// region and the NW are merged like split-K partials (one workgroup barrier).
//
// Blocked flash attention over per-head work atoms with an output scratch:
// "DeepSpeed Inference v2 source tour", section "Ragged batches: packing a whole server
// into four tensors".
#pragma once

#include "rbkv_device.h"
#include "rbkv_internal.h"

namespace rbkv {
namespace mfma_decode {

typedef short s16x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4v lds_s16x4v;

constexpr int D = 128;
constexpr int TE = 16 * D;  // elements of a wave's K (or V) slice of one step
constexpr int RS = D + 4;   // row stride (floats) of a wave's output in the merge

// LDS of one workgroup: ST stages of a K and a V slice per wave (bf16 elements), and the
// per-wave (m, l) of every head for the merge.
template <int ST, int NW>
constexpr int buf_elems() { return NW * ST * 2 * TE; }
template <int NW>
constexpr int ml_floats() { return NW * 16 * 2; }

__device__ __forceinline__ bf16x2v pair(uint32_t w) { return __builtin_bit_cast(bf16x2v, w); }


// Work item `item` by the workgroup's first NW wavefronts (every thread of the workgroup
// must call it: the merge takes a workgroup barrier).  buf: buf_elems<ST, NW>() elements
// of LDS, ml: ml_floats<NW>() floats of LDS.  On return the workgroup may reuse both.  The
// pointers must be the calling kernel's own restrict parameters, so that the metadata
// reads go through the scalar cache.
template <int ST, int NW>
__device__ __forceinline__ void run_item(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ pool,
    uint16_t* __restrict__ out, float* __restrict__ ws, const int4* __restrict__ work,
    const int32_t* __restrict__ tok2seq, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ block_off, const int32_t* __restrict__ block_ids, int32_t Hq,
    int32_t Hkv, int32_t G, int32_t bs, int32_t split_tiles, float scale_log2, int32_t item,
    uint16_t* buf, float* ml) {
  constexpr int NT = NW * 64;
  constexpr float SLACK = 8.f;
  static_assert(ST >= 2 && ST <= 3, "stages");
  static_assert(16 * RS * 4 <= ST * 2 * TE * 2, "merge rows fit the wave's region");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // provably uniform: scalar bases
  const int g = lane >> 4, j = lane & 15;

  // Loader: instruction n of a slice writes LDS bytes 1024n + 16 lane, i.e. key 4n + g,
  // chunk slot j; the source chunk is chosen so the slot carries the swizzle.
  uint32_t ld_k[4], ld_v[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int key = 4 * n + g;
    ld_k[n] = (uint32_t)((j ^ (key & 15)) * 16);
    ld_v[n] = (uint32_t)((j ^ (2 * (key & 7))) * 16);
  }
  // K fragment of step s for key j: chunk 4s + g.  V^T fragment of dim block d: source
  // lane (g, a, r) (a = lane / 4 % 4, r = lane % 4) reads key 4g + a, dims 16d + 4r .. +3.
  uint32_t kfo[4], vfo[8];
#pragma unroll
  for (int s = 0; s < 4; ++s) kfo[s] = (uint32_t)(j * D + (((4 * s + g) ^ j) * 8));
  {
    const int a = (lane >> 2) & 3, r = lane & 3, key = 4 * g + a;
#pragma unroll
    for (int d = 0; d < 8; ++d)
      vfo[d] = (uint32_t)(TE + key * D + ((2 * d + (r >> 1)) ^ (2 * (key & 7))) * 8 + (r & 1) * 4);
  }
  uint16_t* wbuf = buf + wave * (ST * 2 * TE);  // this wave's stages
  const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(lds_addr(wbuf));

  item = __builtin_amdgcn_readfirstlane(item);  // uniform: the metadata comes through the scalar cache
  const int4 w = work[item];
  const int32_t token = w.x, kvh = w.y, split = w.z, slot = w.w;
  const int32_t seq = tok2seq[token];
  const int32_t nkeys = pos[token] + 1;
  const int32_t tiles_total = (nkeys + 63) >> 6;
  const int32_t t_begin = slot < 0 ? 0 : split * split_tiles;
  const int32_t t_end = slot < 0 ? tiles_total : min(tiles_total, t_begin + split_tiles);
  const int32_t key_end = min(nkeys, t_end * 64);
  // The wave's slice of step u starts at key k_first + 16 NW u; it has nsteps steps with a
  // key of the item (none at all for a wave past the end of a short item).
  const int32_t k_first = t_begin * 64 + 16 * wave;
  const int32_t nsteps = k_first < key_end ? (key_end - k_first + 16 * NW - 1) / (16 * NW) : 0;
  const int32_t* bids = block_ids + block_off[seq];
  const int bsh = 31 - __builtin_clz(bs);
  const size_t head_stride = (size_t)bs * D;
  const size_t blk_stride = (size_t)2 * Hkv * head_stride;
  const uint32_t v_bytes = (uint32_t)(Hkv * head_stride * 2);
  const uint16_t* pool_g = pool + (size_t)kvh * head_stride;

  // The wave's 16 keys of step u into stage st.  Rows past the end of the split load its
  // last key, whose weight is 0.
  auto issue = [&](int32_t u, int st) {
    const int32_t key0 = k_first + 16 * NW * u;
    const uint16_t* base = pool_g + (size_t)bids[key0 >> bsh] * blk_stride + (size_t)(key0 & (bs - 1)) * D;
    const int32_t rmax = key_end - 1 - key0;
    const uint32_t dst = lds_wave + (uint32_t)st * (2 * TE * 2);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const uint32_t roff = (uint32_t)min(4 * n + g, rmax) * (D * 2);
      load_lds16_nt_s(base, roff + ld_k[n], dst + n * 1024);
      load_lds16_nt_s(base, v_bytes + roff + ld_v[n], dst + TE * 2 + n * 1024);
    }
  };

  u32x4 qb[4];
  float m = -1e30f, l = 0.f;  // finite start: a wave may see no valid key of a short item
  f32x4 o[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int32_t u, int st) {
    const uint16_t* kt = wbuf + st * (2 * TE);
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 kf = *(const u32x4*)(kt + kfo[s]);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, kf),
                                                     __builtin_bit_cast(bf16x8v, qb[s]), sacc, 0, 0, 0);
    }
    const int32_t k0 = k_first + 16 * NW * u + 4 * g;
    float sc[4], mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = k0 + i < key_end ? sacc[i] * scale_log2 : -INFINITY;
      mt = fmaxf(mt, sc[i]);
    }
    if (__any(mt > m + SLACK)) {
      float M = fmaxf(mt, __shfl_xor(mt, 16, 64));
      M = fmaxf(M, __shfl_xor(M, 32, 64));
      const float mnew = M > m + SLACK ? M : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < 8; ++d) o[d] *= alpha;
      m = mnew;
    }
    const uint32_t p01 = pack_bf16x2(__builtin_amdgcn_exp2f(sc[0] - m), __builtin_amdgcn_exp2f(sc[1] - m));
    const uint32_t p23 = pack_bf16x2(__builtin_amdgcn_exp2f(sc[2] - m), __builtin_amdgcn_exp2f(sc[3] - m));
    l = __builtin_amdgcn_fdot2_f32_bf16(pair(p01), pair(0x3f803f80u), l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16(pair(p23), pair(0x3f803f80u), l, false);
    const s16x4v pb = __builtin_bit_cast(s16x4v, j < G ? u32x2{p01, p23} : u32x2{0u, 0u});
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const s16x4v vf = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4v*)(kt + vfo[d]));
      o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pb, o[d], 0, 0, 0);
    }
  };

  // The wave's own pipeline: its first ST steps go out at once, then each step's stage is
  // refilled with the step ST further as soon as it has been computed; before a step is
  // read only the loads of later steps (8 per step) may be outstanding.
#pragma unroll
  for (int u = 0; u < ST; ++u)
    if (u < nsteps) issue(u, u);
  // Q^T operand of step s: head j (clamped to the group), dims 32s + 8g .. +8.  The empty
  // asm makes the compiler complete these loads here (together with the first slices,
  // which are needed first anyway), so that no wait it tracks for them falls inside the
  // step loop, where it would also drain the next slices' loads.
  {
    const uint16_t* qrow = qkv + ((size_t)token * (Hq + 2 * Hkv) + (size_t)kvh * G + min(j, G - 1)) * D;
#pragma unroll
    for (int s = 0; s < 4; ++s) qb[s] = ld16(qrow + (4 * s + g) * 8);
    if (j >= G) {  // padding columns multiply zeros (less switching in the matrix cores)
#pragma unroll
      for (int s = 0; s < 4; ++s) qb[s] = u32x4{0u, 0u, 0u, 0u};
    }
    asm volatile("" : : "v"(qb[0]), "v"(qb[1]), "v"(qb[2]), "v"(qb[3]));
  }
  int st = 0;
  for (int32_t u = 0; u < nsteps; ++u) {
    const int32_t later = min(nsteps - 1 - u, ST - 1);
    if (ST == 3 && later >= 2) wait_vmcnt<16>();
    else if (later >= 1) wait_vmcnt<8>();
    else wait_vmcnt<0>();
    compute(u, st);
    if (u + ST < nsteps) issue(u + ST, st);
    st = st + 1 == ST ? 0 : st + 1;
  }

  // Merge: each wave's weight sum over its lane groups, then the NW waves through LDS.
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  float* ro = (float*)wbuf;  // this wave's region: its reads of it are done
  if (j < G) {
#pragma unroll
    for (int d = 0; d < 8; ++d) *(f32x4*)(ro + j * RS + 16 * d + 4 * g) = o[d];
    if (g == 0) {
      ml[(wave * 16 + j) * 2] = m;
      ml[(wave * 16 + j) * 2 + 1] = l;
    }
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += NT) {
    const int h = e / D, dim = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) M = fmaxf(M, ml[(wv * 16 + h) * 2]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) {
      const float a = __builtin_amdgcn_exp2f(ml[(wv * 16 + h) * 2] - M);
      num = fmaf(a, ((const float*)(buf + wv * (ST * 2 * TE)))[h * RS + dim], num);
      den = fmaf(a, ml[(wv * 16 + h) * 2 + 1], den);
    }
    if (slot < 0) {
      out[((size_t)token * Hq + (size_t)kvh * G + h) * D + dim] = (uint16_t)bf16_rne_f32(num / den);
    } else {
      float* part = ws + (size_t)slot * G * (D + 2);
      if (dim == 0) {
        part[h] = M;
        part[G + h] = den;
      }
      part[2 * G + (size_t)h * D + dim] = num;
    }
  }
}

}  // namespace mfma_decode
}  // namespace rbkv
