// Split-K streaming attention on the vector ALUs.  One 64-lane wavefront per work item
// (token, kv head, split): it streams the split's keys in tiles of 64 (one key per lane
// for Q.K, lanes spread over head-dim columns for P.V), keeps a running max and sum per
// query head (online softmax with wavefront max reductions), and writes either the
// finished output or an unnormalised partial (m, l, acc) for the combine kernel.
//
// All G query heads of a kv group share one pass over the keys (grouped-query reuse).
// Tiles are fetched with coalesced 16-byte loads (each instruction covers whole rows of
// one block) and K is staged through LDS with an XOR swizzle so that the transposed
// one-row-per-lane reads are free of bank conflicts.  Used for single-token decodes
// (split-K over long histories) and, in float32, for every token of a chunk.
//
// Blocked flash attention over per-head work atoms with an output scratch:
// "DeepSpeed Inference v2 source tour", section "Ragged batches: packing a whole server
// into four tensors"; FlashAttention-2-style integration: "DeepSpeed-Inference and
// DeepSpeed-MII", section 10.3.
#include <algorithm>

#include "decode_mfma.h"
#include "rbkv_device.h"
#include "rbkv_internal.h"

namespace rbkv {
namespace {

// K/V tile rows are read once per work item: non-temporal loads (measured 4-7% faster
// decode than plain loads on the MHA, SplitFuse and full-budget batches).
__device__ __forceinline__ u32x4 ldnt(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

template <typename T, int D>
struct DecGeom {
  static constexpr int RB = D * (int)sizeof(T);  // bytes per key row
  static constexpr int CPR = RB / 16;            // 16-byte chunks per row
  static constexpr int KPI = 64 / CPR;           // keys per load instruction
  static constexpr int NI = CPR;                 // load instructions per 64-key tile
  static constexpr int VW = 16 / (int)sizeof(T); // elements per chunk
};

// Swizzled chunk slot of (row, chunk) in the LDS key tile.  Rows are CPR chunks long;
// the XOR spreads 16 consecutive rows over 16 distinct 16-byte bank groups.
template <int CPR>
__device__ __forceinline__ int kslot(int row, int c) {
  constexpr int SH = CPR >= 16 ? 0 : (CPR == 8 ? 1 : 2);
  const int swz = CPR >= 16 ? (row & 15) : ((row >> SH) & (CPR - 1));
  return row * CPR + (c ^ swz);
}

// The bf16 pair reinterpretation goes through a by-value word: a bit cast applied
// directly to a vector-element lvalue (q.y, ...) is lowered as a read of element 0.
__device__ __forceinline__ bf16x2v as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2v, w); }

__device__ __forceinline__ float dot_chunk(u32x4 q, u32x4 k, float acc, bf16_t) {
  const uint32_t q0 = q.x, q1 = q.y, q2 = q.z, q3 = q.w;
  const uint32_t k0 = k.x, k1 = k.y, k2 = k.z, k3 = k.w;
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q0), as_bf16x2(k0), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q1), as_bf16x2(k1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q2), as_bf16x2(k2), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q3), as_bf16x2(k3), acc, false);
  return acc;
}
__device__ __forceinline__ float dot_chunk(u32x4 q, u32x4 k, float acc, float) {
  acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
  acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
  acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
  acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  return acc;
}

template <typename T>
__device__ __forceinline__ void unpack_chunk(u32x4 v, float* f);
template <>
__device__ __forceinline__ void unpack_chunk<bf16_t>(u32x4 v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}
template <>
__device__ __forceinline__ void unpack_chunk<float>(u32x4 v, float* f) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

template <typename T>
__device__ __forceinline__ u32x4 pack_chunk(const float* f);
template <>
__device__ __forceinline__ u32x4 pack_chunk<bf16_t>(const float* f) {
  u32x4 r;
  r.x = pack_bf16x2(f[0], f[1]); r.y = pack_bf16x2(f[2], f[3]);
  r.z = pack_bf16x2(f[4], f[5]); r.w = pack_bf16x2(f[6], f[7]);
  return r;
}
template <>
__device__ __forceinline__ u32x4 pack_chunk<float>(const float* f) {
  u32x4 r;
  r.x = __float_as_uint(f[0]); r.y = __float_as_uint(f[1]);
  r.z = __float_as_uint(f[2]); r.w = __float_as_uint(f[3]);
  return r;
}

// Waves per SIMD the kernel is compiled for: two where the registers allow it (tile data
// in flight is what hides HBM latency), one otherwise.
template <typename T, int GMAX>
constexpr int dec_waves_per_simd() { return (sizeof(T) == 4 || GMAX >= 16) ? 1 : 2; }

// ONE_BLK: blocks hold at least 64 keys, so every 64-key tile lies inside one block.
template <typename T, int D, int GMAX, bool ONE_BLK>
__global__ __launch_bounds__(64)
__attribute__((amdgpu_waves_per_eu(dec_waves_per_simd<T, GMAX>(), dec_waves_per_simd<T, GMAX>())))
void decode_attn_kernel(
    const T* __restrict__ qkv, const T* __restrict__ pool, T* __restrict__ out,
    float* __restrict__ ws, const int4* __restrict__ work, const int32_t* __restrict__ tok2seq,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ block_off,
    const int32_t* __restrict__ block_ids, int32_t Hq, int32_t Hkv, int32_t G, int32_t bs,
    int32_t split_tiles, float scale_log2) {
  using Gm = DecGeom<T, D>;
  constexpr int CPR = Gm::CPR, KPI = Gm::KPI, NI = Gm::NI, VW = Gm::VW;
  constexpr int MAXNB = 4;  // blocks a 64-key tile can span (block size 16)
  __shared__ u32x4 ktile[64 * CPR];
  __shared__ u32x4 qs[GMAX * CPR];
  __shared__ __attribute__((aligned(16))) float ps[64 * GMAX];

  const int lane = threadIdx.x;
  const int4 w = work[blockIdx.x];
  const int32_t token = w.x, kvh = w.y, split = w.z, slot = w.w;
  const int32_t seq = tok2seq[token];
  const int32_t nkeys = pos[token] + 1;
  const int32_t tiles_total = (nkeys + 63) >> 6;
  const int32_t t_begin = slot < 0 ? 0 : split * split_tiles;
  const int32_t t_end = slot < 0 ? tiles_total : min(tiles_total, t_begin + split_tiles);
  const int32_t key_end = min(nkeys, t_end * 64);
  const int32_t* bids = block_ids + block_off[seq];
  const int bsh = 31 - __builtin_clz(bs);             // block sizes are powers of two
  const int32_t last_blk = (key_end - 1) >> bsh;
  const size_t head_stride = (size_t)bs * D;          // one (block, kv, head) slab
  const size_t blk_stride = (size_t)2 * Hkv * head_stride;
  const size_t v_off = (size_t)Hkv * head_stride;     // keys -> values of the same block
  const T* pool_g = pool + (size_t)kvh * head_stride;
  // Query rows of the group into LDS (read back as broadcasts); heads past G (padding up
  // to GMAX) repeat the last real head, so the head loops need no branches.
  {
    const T* qrow = qkv + (size_t)token * (Hq + 2 * Hkv) * D + (size_t)kvh * G * D;
    for (int u = lane; u < GMAX * CPR; u += 64)
      qs[u] = ld16(qrow + (size_t)min(u / CPR, G - 1) * D + (u % CPR) * VW);
  }

  float m[GMAX], lsum[GMAX], o[GMAX][VW];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VW; ++e) o[h][e] = 0.f;
  }
  const int cl = lane % CPR;  // chunk column this lane loads / accumulates
  const int kg = lane / CPR;  // key sub-row within a load instruction
  const int lane_off = kg * D + cl * VW;  // element offset of this lane inside a row group

  // Block ids of a tile are uniform: they come through the scalar cache, a tile ahead.
  auto fetch_ids = [&](int32_t tt, int32_t* ids) {
    const int32_t b0 = min((tt * 64) >> bsh, last_blk);
#pragma unroll
    for (int j = 0; j < MAXNB; ++j) ids[j] = bids[min(b0 + j, last_blk)];
  };
  // Uniform base of row group i of a tile: keys key0 + i*KPI .. +KPI-1 share one block
  // (KPI <= 8 <= bs).  A group wholly past key_end re-reads the tile's first group.
  auto row_base = [&](int32_t tt, const int32_t* ids, int i) -> const T* {
    const int32_t key0 = tt * 64;
    if constexpr (ONE_BLK)  // the tile lies in one block: fixed row offsets from one base
      return pool_g + (size_t)ids[0] * blk_stride + (size_t)(key0 & (bs - 1)) * D +
             (size_t)(i * KPI) * D;
    int32_t k = key0 + i * KPI;
    k = k < key_end ? k : key0;
    const int jb = (k >> bsh) - (key0 >> bsh);
    const int32_t id = jb == 0 ? ids[0] : jb == 1 ? ids[1] : jb == 2 ? ids[2] : ids[3];
    return pool_g + (size_t)id * blk_stride + (size_t)(k & (bs - 1)) * D;
  };

  u32x4 kr[NI], vr[NI];
  int32_t ids_cur[MAXNB], ids_next[MAXNB];
  fetch_ids(t_begin, ids_cur);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const T* rb = row_base(t_begin, ids_cur, i);
    kr[i] = ldnt(rb + lane_off);
    vr[i] = ldnt((rb + v_off) + lane_off);
  }
  fetch_ids(min(t_begin + 1, t_end - 1), ids_next);

  for (int32_t tt = t_begin; tt < t_end; ++tt) {
    // The next tile is always prefetched (the last tile re-reads itself, an L2 hit), so
    // the loads need no branches and the V registers are refilled in place.
    const int32_t tn = min(tt + 1, t_end - 1);
    __syncthreads();  // previous tile's readers of ktile / ps are done
#pragma unroll
    for (int i = 0; i < NI; ++i) ktile[kslot<CPR>(i * KPI + kg, cl)] = kr[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NI; ++i) kr[i] = ldnt(row_base(tn, ids_next, i) + lane_off);

    // Scores: lane = key; every padding head repeats a real one, so no branches.
    const int32_t key0 = tt * 64;
    float s[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) s[h] = 0.f;
#pragma unroll
    for (int c = 0; c < CPR; ++c) {
      const u32x4 kc = ktile[kslot<CPR>(lane, c)];
#pragma unroll
      for (int h = 0; h < GMAX; ++h) s[h] = dot_chunk(qs[h * CPR + c], kc, s[h], T{});
    }
    const bool valid = key0 + lane < key_end;
    float alpha[GMAX];
    float pe[GMAX];
    bool any_moved = false;  // uniform: some running max changed this tile
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      const float sc = valid ? s[h] * scale_log2 : -INFINITY;
      const float mn = fmaxf(m[h], wave_max_dpp(sc));
      any_moved |= mn != m[h];
      alpha[h] = __builtin_amdgcn_exp2f(m[h] - mn);
      m[h] = mn;
      pe[h] = __builtin_amdgcn_exp2f(sc - mn);
      lsum[h] = lsum[h] * alpha[h] + pe[h];
    }
#pragma unroll
    for (int h = 0; h < GMAX; h += (GMAX >= 4 ? 4 : GMAX)) {
      if constexpr (GMAX >= 4)
        *(f32x4*)(ps + lane * GMAX + h) = f32x4{pe[h], pe[h + 1], pe[h + 2], pe[h + 3]};
      else
#pragma unroll
        for (int j = 0; j < GMAX; ++j) ps[lane * GMAX + j] = pe[j];
    }
    __syncthreads();

    // P.V: lane accumulates VW columns over keys i*KPI + kg; each V register is
    // refilled with the next tile's row as soon as it has been used.
    if (any_moved) {
#pragma unroll
      for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int e = 0; e < VW; ++e) o[h][e] *= alpha[h];
    }
    const bool partial = key0 + 64 > key_end;  // keys past the end: zero their values
    if constexpr (sizeof(T) == 2 && GMAX <= 4) {
      // bf16, up to 4 heads: two keys per v_dot2_f32_bf16 (measured faster than fp32 FMAs
      // there; with 8+ heads the extra registers cost more than the saved issue slots).  Rows i and i+1 (keys k and k + KPI) are
      // interleaved per column with v_perm_b32 and their weights packed to a bf16 pair.
#pragma unroll
      for (int i = 0; i < NI; i += 2) {
        u32x4 a = vr[i], b = vr[i + 1];
        if (partial && key0 + i * KPI + kg >= key_end) a = u32x4{0, 0, 0, 0};
        if (partial && key0 + (i + 1) * KPI + kg >= key_end) b = u32x4{0, 0, 0, 0};
        vr[i] = ldnt((row_base(tn, ids_next, i) + v_off) + lane_off);
        vr[i + 1] = ldnt((row_base(tn, ids_next, i + 1) + v_off) + lane_off);
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
        uint32_t vp[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vp[2 * j] = __builtin_amdgcn_perm(bw[j], aw[j], 0x05040100u);
          vp[2 * j + 1] = __builtin_amdgcn_perm(bw[j], aw[j], 0x07060302u);
        }
        const float* pa = ps + (i * KPI + kg) * GMAX;
        const float* pb = ps + ((i + 1) * KPI + kg) * GMAX;
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
          const bf16x2v pp = as_bf16x2(pack_bf16x2(pa[h], pb[h]));
#pragma unroll
          for (int e = 0; e < VW; ++e)
            o[h][e] = __builtin_amdgcn_fdot2_f32_bf16(pp, as_bf16x2(vp[e]), o[h][e], false);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float v[VW];
        u32x4 vi = vr[i];
        if (partial && key0 + i * KPI + kg >= key_end) vi = u32x4{0, 0, 0, 0};
        unpack_chunk<T>(vi, v);
        vr[i] = ldnt((row_base(tn, ids_next, i) + v_off) + lane_off);
        const float* pk = ps + (i * KPI + kg) * GMAX;
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
          const float ph = pk[h];
#pragma unroll
          for (int e = 0; e < VW; ++e) o[h][e] = fmaf(ph, v[e], o[h][e]);
        }
      }
    }
    fetch_ids(min(tt + 2, t_end - 1), ids_next);
  }

  // Reduce over the lanes that share a chunk column, and the row sums over all lanes.
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
#pragma unroll
    for (int e = 0; e < VW; ++e) {
#pragma unroll
      for (int off = CPR; off < 64; off <<= 1) o[h][e] += __shfl_xor(o[h][e], off, 64);
    }
    lsum[h] = wave_sum_dpp(lsum[h]);
  }
  if (slot < 0) {
    if (lane < CPR) {
#pragma unroll
      for (int h = 0; h < GMAX; ++h)
        if (h < G) {
          const float inv = 1.f / lsum[h];
          float r[VW];
#pragma unroll
          for (int e = 0; e < VW; ++e) r[e] = o[h][e] * inv;
          st16(out + ((size_t)token * Hq + (size_t)kvh * G + h) * D + cl * VW, pack_chunk<T>(r));
        }
    }
  } else {
    float* part = ws + (size_t)slot * G * (D + 2);
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < GMAX; ++h)
        if (h < G) {
          part[h] = m[h];
          part[G + h] = lsum[h];
        }
    }
    if (lane < CPR) {
#pragma unroll
      for (int h = 0; h < GMAX; ++h)
        if (h < G) {
          float* dst = part + 2 * G + (size_t)h * D + cl * VW;
#pragma unroll
          for (int e = 0; e < VW; ++e) dst[e] = o[h][e];
        }
    }
  }
}

// Grouped-query decode for bf16 caches (groups of 9-16 heads, and 5-8 heads over blocks of
// fewer than 64 keys): one wavefront per query head of the kv group
// (NW >= G waves; waves past G repeat the last head and write nothing).  Each 64-key K/V
// tile is loaded once per workgroup, straight from HBM into LDS (global_load_lds), and
// every wave streams its own head over it: Q in registers, one key per lane for Q.K (K
// rows XOR-swizzled in LDS), a wave-level online softmax, and P.V with lanes over
// head-dim chunks (two keys per v_dot2_f32_bf16).  Two LDS stages (the next tile loads
// while this one is computed) keep the workgroup at 66 KB and its waves at 128 registers,
// so two workgroups share a CU: what hides the memory latency here is the number of
// independent waves, not a deeper prefetch.  The work item, the split-K partition and
// the partial layout are those of the per-wave kernel above.
template <int D, int NW, bool ONE_BLK>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 4)))
void decode_group_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ pool,
    uint16_t* __restrict__ out, float* __restrict__ ws, const int4* __restrict__ work,
    const int32_t* __restrict__ tok2seq, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ block_off, const int32_t* __restrict__ block_ids, int32_t Hq,
    int32_t Hkv, int32_t G, int32_t bs, int32_t split_tiles, float scale_log2) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per key row
  constexpr int NT = NW * 64;                // threads
  constexpr int TILE_CHUNKS = 64 * CPR;      // chunks per K (or V) tile
  constexpr int LDT = NT < TILE_CHUNKS ? NT : TILE_CHUNKS;  // loading threads (whole waves)
  constexpr int NLD = TILE_CHUNKS / LDT;     // direct loads per loading thread per K (or V) tile
  constexpr int KPI = 64 / CPR;              // P.V: keys per row group (lanes per chunk column)
  constexpr int NI = CPR;                    // P.V: row groups per tile
  constexpr int STG = 2;                     // tiles resident: one computed, one in flight
  constexpr int MAXNB = 4;                   // blocks a 64-key tile can span (block size 16)
  static_assert(TILE_CHUNKS % LDT == 0 && LDT % 64 == 0, "loader geometry");
  __shared__ __attribute__((aligned(16))) uint16_t Kt[STG][64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[STG][64 * D];
  __shared__ float ps[NW][64];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int4 w = work[blockIdx.x];
  const int32_t token = w.x, kvh = w.y, split = w.z, slot = w.w;
  const int32_t seq = tok2seq[token];
  const int32_t nkeys = pos[token] + 1;
  const int32_t tiles_total = (nkeys + 63) >> 6;
  const int32_t t_begin = slot < 0 ? 0 : split * split_tiles;
  const int32_t t_end = slot < 0 ? tiles_total : min(tiles_total, t_begin + split_tiles);
  const int32_t key_end = min(nkeys, t_end * 64);
  const int32_t* bids = block_ids + block_off[seq];
  const int bsh = 31 - __builtin_clz(bs);  // block sizes are powers of two
  const int32_t last_blk = (key_end - 1) >> bsh;
  const size_t head_stride = (size_t)bs * D;
  const size_t blk_stride = (size_t)2 * Hkv * head_stride;
  const size_t v_off = (size_t)Hkv * head_stride;
  const uint16_t* pool_g = pool + (size_t)kvh * head_stride;
  // This wave's head within the group; uniform, so its query row comes through the scalar
  // cache and no register load is pending while the tile loads are in flight.
  const int32_t hg = min(wave, G - 1);

  // Loader: direct load i of thread tid fills LDS chunk p = i*LDT + tid of a tile, i.e.
  // key row p / CPR.  K chunks carry an XOR swizzle (chunk c of row r at c ^ swz(r)) so
  // that the one-row-per-lane Q.K reads are free of bank conflicts; V rows are stored as
  // they are (a P.V read covers whole rows).
  auto kswz = [](int r) { return CPR >= 16 ? (r & 15) : ((r >> 1) & (CPR - 1)); };
  auto fetch_ids = [&](int32_t t, int32_t* ids) {
    const int32_t b0 = min((t * 64) >> bsh, last_blk);
#pragma unroll
    for (int j = 0; j < MAXNB; ++j) ids[j] = bids[min(b0 + j, last_blk)];
  };
  constexpr uint32_t TILE_BYTES = 64 * D * 2;
  const uint32_t k_dst0 = __builtin_amdgcn_readfirstlane(lds_addr(&Kt[0][0]) + wave * 64 * 16);
  const uint32_t v_dst0 = __builtin_amdgcn_readfirstlane(lds_addr(&Vt[0][0]) + wave * 64 * 16);
  // Each tile is read once per item: direct loads with the non-temporal policy (2%
  // faster on the long-decode batch than the default policy).
  auto issue_tile = [&](int32_t t, const int32_t* ids, int buf) {
    if (LDT < NT && tid >= LDT) return;  // waves past the tile's chunk count load nothing
    const int32_t key0 = t * 64;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int p = i * LDT + tid;
      const int r = p / CPR, c = p % CPR;
      // Rows past the end of the split load its last key (never read unmasked).
      int32_t k = min(key0 + r, key_end - 1);
      const uint16_t* row;
      if constexpr (ONE_BLK) {
        row = pool_g + (size_t)ids[0] * blk_stride + (size_t)(k & (bs - 1)) * D;
      } else {
        const int jb = (k >> bsh) - (key0 >> bsh);
        const int32_t id = jb == 0 ? ids[0] : jb == 1 ? ids[1] : jb == 2 ? ids[2] : ids[3];
        row = pool_g + (size_t)id * blk_stride + (size_t)(k & (bs - 1)) * D;
      }
      const uint32_t off = buf * TILE_BYTES + i * LDT * 16;
      load_lds16_nt(row + (c ^ kswz(r)) * 8, k_dst0 + off);
      load_lds16_nt(row + v_off + c * 8, v_dst0 + off);
    }
  };

  // This wave's query row in registers: chunk c holds dims 8c .. 8c+7.
  u32x4 q[CPR];
  {
    const uint16_t* qrow = qkv + ((size_t)token * (Hq + 2 * Hkv) + (size_t)kvh * G + hg) * D;
#pragma unroll
    for (int c = 0; c < CPR; ++c) q[c] = ld16(qrow + c * 8);
  }
  int32_t ids[MAXNB];
  fetch_ids(t_begin, ids);
  issue_tile(t_begin, ids, 0);
  fetch_ids(min(t_begin + 1, t_end - 1), ids);
  wait_vmcnt<0>();  // Q and the first tile; afterwards only tile loads are in flight
  __syncthreads();

  float m_run = -INFINITY, lsum = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  const int cl = lane % CPR, kg = lane / CPR;  // P.V: chunk column and key sub-row
  const int kchunk0 = lane * CPR;              // Q.K: this lane's key row (in chunks)

  for (int32_t tt = t_begin; tt < t_end; ++tt) {
    const int j = tt - t_begin;
    if (j > 0) {
      // Tile tt resident (the only load in flight); every wave past tile tt-1, whose
      // stage takes tile tt+1.
      wait_vmcnt<0>();
      __syncthreads();
    }
    if (tt + 1 < t_end) {
      issue_tile(tt + 1, ids, (j + 1) % STG);
      fetch_ids(min(tt + 2, t_end - 1), ids);
    }
    const u32x4* kt = (const u32x4*)Kt[j % STG];
    const u32x4* vt = (const u32x4*)Vt[j % STG];
    const int32_t key0 = tt * 64;

    // Scores: lane = key.
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CPR; ++c) s = dot_chunk(q[c], kt[kchunk0 + (c ^ kswz(lane))], s, bf16_t{});
    const float sc = key0 + lane < key_end ? s * scale_log2 : -INFINITY;
    const float mn = fmaxf(m_run, wave_max_dpp(sc));
    const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
    const float pe = __builtin_amdgcn_exp2f(sc - mn);
    m_run = mn;
    lsum = lsum * alpha + pe;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= alpha;
    ps[wave][lane] = pe;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // P.V: lane accumulates the 8 columns of chunk cl over keys i*KPI + kg, two keys per
    // v_dot2 (rows i and i+1 interleaved per column with v_perm_b32); the weight of key r
    // comes from lane r.
#pragma unroll
    for (int i = 0; i < NI; i += 2) {
      const int ra = i * KPI + kg, rb = ra + KPI;
      const u32x4 a = vt[ra * CPR + cl], b = vt[rb * CPR + cl];
      const bf16x2v pp = as_bf16x2(pack_bf16x2(ps[wave][ra], ps[wave][rb]));
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        o[2 * jj] = __builtin_amdgcn_fdot2_f32_bf16(
            pp, as_bf16x2(__builtin_amdgcn_perm(bw[jj], aw[jj], 0x05040100u)), o[2 * jj], false);
        o[2 * jj + 1] = __builtin_amdgcn_fdot2_f32_bf16(
            pp, as_bf16x2(__builtin_amdgcn_perm(bw[jj], aw[jj], 0x07060302u)), o[2 * jj + 1], false);
      }
    }
  }

  // Reduce over the lanes that share a chunk column, and the row sums over all lanes.
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1) o[e] += __shfl_xor(o[e], off, 64);
  lsum = wave_sum_dpp(lsum);
  if (wave >= G) return;  // padding head
  if (slot < 0) {
    if (lane < CPR) {
      const float inv = 1.f / lsum;
      float r[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = o[e] * inv;
      st16(out + ((size_t)token * Hq + (size_t)kvh * G + hg) * D + cl * 8, pack_chunk<bf16_t>(r));
    }
  } else {
    float* part = ws + (size_t)slot * G * (D + 2);
    if (lane == 0) {
      part[hg] = m_run;
      part[G + hg] = lsum;
    }
    if (lane < CPR) {
      float* dst = part + 2 * G + (size_t)hg * D + cl * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = o[e];
    }
  }
}

// Lean grouped decode for bf16 caches over blocks of at least 64 keys, groups of up to
// four heads (used at head dim 64; head dim 128 runs on the matrix-core kernel below):
// NW = 4 wavefronts of at most 96 registers, one per query head of the kv group (waves
// past G repeat the last head and write nothing), and one 64-key K/V tile in LDS with
// nothing else there: the softmax weights reach the P.V lanes through ds_bpermute, which
// needs no LDS allocation, and the query row sits in scalar registers.  The tile is
// loaded straight from HBM into LDS by all the waves from a uniform block base.  Each lane
// copies its V chunks to registers before the barrier that frees the tile, so the next
// tile's loads fly while P.V is summed, and the other workgroups on the CU (five fit)
// hide the rest of the latency.  Arithmetic and order are those of the kernels above
// (same results, bit for bit).  Work items, split-K partition and partial layout are
// those of the kernels above; with a claim counter the workgroups are persistent and take
// items from it.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(5, 5)))
void decode_lean_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ pool,
    uint16_t* __restrict__ out, float* __restrict__ ws, const int4* __restrict__ work,
    const int32_t* __restrict__ tok2seq, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ block_off, const int32_t* __restrict__ block_ids, int32_t Hq,
    int32_t Hkv, int32_t G, int32_t bs, int32_t split_tiles, float scale_log2,
    int32_t* __restrict__ claim, int32_t n_items) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per key row
  constexpr int NT = NW * 64;                // threads
  constexpr int TILE_CHUNKS = 64 * CPR;      // chunks per K (or V) tile
  constexpr int NLD = TILE_CHUNKS / NT;      // direct loads per thread per K (or V) tile
  constexpr int KPI = 64 / CPR;              // P.V: keys per row group
  constexpr int NI = CPR;                    // P.V: row groups per tile
  // The loader takes one K swizzle per thread: each load must cover a multiple of 16 rows.
  static_assert(TILE_CHUNKS % NT == 0 && (NT / CPR) % 16 == 0, "loader geometry");
  __shared__ __attribute__((aligned(16))) uint16_t Kt[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[64 * D];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // With a claim counter the workgroup is persistent: it takes item after item from the
  // counter until the list is exhausted (the two-stream call runs the decodes as two such
  // launches draining one list).  The claimed index is broadcast through the first word
  // of the K tile, between barriers, before any tile load can overwrite it.
  auto next_item = [&]() -> int32_t {
    __syncthreads();  // every wave is done with the previous item's tile
    if (tid == 0) {
      const uint32_t c = (uint32_t)atomicAdd(claim, 1);
      Kt[0] = (uint16_t)c;
      Kt[1] = (uint16_t)(c >> 16);
    }
    __syncthreads();
    const int32_t it = __builtin_amdgcn_readfirstlane((int32_t)(Kt[0] | ((uint32_t)Kt[1] << 16)));
    __syncthreads();  // read by every wave before the next tile lands there
    return it;
  };
  for (int32_t item = claim ? next_item() : (int32_t)blockIdx.x; item < n_items;
       item = claim ? next_item() : n_items) {
    const int4 w = work[item];
    const int32_t token = w.x, kvh = w.y, split = w.z, slot = w.w;
    const int32_t seq = tok2seq[token];
    const int32_t nkeys = pos[token] + 1;
    const int32_t tiles_total = (nkeys + 63) >> 6;
    const int32_t t_begin = slot < 0 ? 0 : split * split_tiles;
    const int32_t t_end = slot < 0 ? tiles_total : min(tiles_total, t_begin + split_tiles);
    const int32_t key_end = min(nkeys, t_end * 64);
    const int32_t* bids = block_ids + block_off[seq];
    const int bsh = 31 - __builtin_clz(bs);  // block sizes are powers of two
    const int32_t last_blk = (key_end - 1) >> bsh;
    const size_t head_stride = (size_t)bs * D;
    const size_t blk_stride = (size_t)2 * Hkv * head_stride;
    const size_t v_off = (size_t)Hkv * head_stride;
    const uint16_t* pool_g = pool + (size_t)kvh * head_stride;
    // This wave's head in the group, made provably uniform so that the query row is read
    // into scalar registers (the vector registers cannot hold it beside the rest).
    const int32_t hg = __builtin_amdgcn_readfirstlane(min(wave, G - 1));

    // Direct load i of thread tid fills LDS chunk p = i*NT + tid of a tile (key row p / CPR);
    // K chunks carry the XOR swizzle of the kernels above, V rows are stored as they are.
    auto kswz = [](int r) { return CPR >= 16 ? (r & 15) : ((r >> 1) & (CPR - 1)); };
    auto fetch_ids = [&](int32_t t, int32_t* ids) { ids[0] = bids[min((t * 64) >> bsh, last_blk)]; };
    const uint32_t k_dst0 = __builtin_amdgcn_readfirstlane(lds_addr(&Kt[0]) + wave * 64 * 16);
    const uint32_t v_dst0 = __builtin_amdgcn_readfirstlane(lds_addr(&Vt[0]) + wave * 64 * 16);
    // Loader lanes: row tid / CPR + i * (NT / CPR) of the tile, chunk tid % CPR; the K
    // swizzle of a row depends on row % 16 only, which is the same for every i.
    const int ld_r0 = tid / CPR, ld_c = tid % CPR;
    const uint32_t ld_kc = (uint32_t)(ld_c ^ kswz(ld_r0)) * 16u, ld_vc = (uint32_t)ld_c * 16u;
    // Blocks hold at least 64 keys, so a tile lies in one block: a uniform base and 32-bit
    // lane offsets.  Rows past the end of the split load its last key (never read unmasked).
    auto issue_tile = [&](int32_t t, const int32_t* ids) {
      const int32_t key0 = t * 64;
      const uint16_t* base = pool_g + (size_t)ids[0] * blk_stride + (size_t)(key0 & (bs - 1)) * D;
      const int32_t rmax = key_end - 1 - key0;
  #pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const uint32_t roff = (uint32_t)min(ld_r0 + i * (NT / CPR), rmax) * (D * 2);
        const uint32_t off = i * NT * 16;
        load_lds16_nt_s(base, roff + ld_kc, k_dst0 + off);
        load_lds16_nt_s(base + v_off, roff + ld_vc, v_dst0 + off);
      }
    };

    u32x4 q[CPR];
    {
      const uint16_t* qrow = qkv + ((size_t)token * (Hq + 2 * Hkv) + (size_t)kvh * G + hg) * D;
  #pragma unroll
      for (int c = 0; c < CPR; ++c) q[c] = ld16(qrow + c * 8);
    }
    int32_t ids[1];
    fetch_ids(t_begin, ids);
    issue_tile(t_begin, ids);
    fetch_ids(min(t_begin + 1, t_end - 1), ids);

    float m_run = -INFINITY, lsum = 0.f, o[8];
  #pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    const int cl = lane % CPR, kg = lane / CPR;  // P.V: chunk column and key sub-row
    // Q.K: byte offset of this lane's key row with its swizzle; chunk c of the row is at
    // krow ^ 16c.  Re-declared opaque every tile so that the sixteen chunk addresses are
    // recomputed (one XOR each) rather than held across the loop in registers.
    uint32_t krow = (uint32_t)(lane * CPR + kswz(lane)) * 16u;
    // P.V: byte offset of this lane's V chunk in row group 0 and the ds_bpermute address of
    // the weight of its key in row group 0; row group i adds a constant (an instruction
    // offset).  Opaque per tile for the same reason.
    uint32_t vcol = (uint32_t)(kg * CPR + cl) * 16u;
    uint32_t pidx = (uint32_t)kg * 4u;

    for (int32_t tt = t_begin; tt < t_end; ++tt) {
      wait_vmcnt<0>();  // this wave's share of tile tt
      __syncthreads();  // every wave's share
      const int32_t key0 = tt * 64;
      asm volatile("" : "+v"(krow), "+v"(vcol), "+v"(pidx));
      const uint32_t kr = krow, vc = vcol;

      // Scores: lane = key.
      float s = 0.f;
  #pragma unroll
      for (int c = 0; c < CPR; ++c)
        s = dot_chunk(q[c], *(const u32x4*)((const char*)Kt + (kr ^ (16u * c))), s, bf16_t{});
      const float sc = key0 + lane < key_end ? s * scale_log2 : -INFINITY;
      const float mn = fmaxf(m_run, wave_max_dpp(sc));
      const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
      const float pe = __builtin_amdgcn_exp2f(sc - mn);
      m_run = mn;
      lsum = lsum * alpha + pe;
      // P.V: lane accumulates the 8 columns of chunk cl over keys i*KPI + kg, two keys per
      // v_dot2 (rows i and i+1 interleaved per column with v_perm_b32).  The lane's V
      // chunks go into registers before the barrier, so the next tile's loads are issued
      // first and fly while the products are summed; the weight of key r is then fetched
      // from lane r (ds_bpermute reads no LDS memory).
      u32x4 vr[NI];
  #pragma unroll
      for (int i = 0; i < NI; ++i)
        vr[i] = *(const u32x4*)((const char*)Vt + vc + i * (KPI * CPR * 16));
      if (tt + 1 < t_end) {
        __syncthreads();  // every wave is done with the tile before it is overwritten
        issue_tile(tt + 1, ids);
        fetch_ids(min(tt + 2, t_end - 1), ids);
      }
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= alpha;
      const int pe_bits = __float_as_int(pe);
  #pragma unroll
      for (int i = 0; i < NI; i += 2) {
        const float pa = __int_as_float(__builtin_amdgcn_ds_bpermute((int)(pidx + i * KPI * 4), pe_bits));
        const float pb = __int_as_float(__builtin_amdgcn_ds_bpermute((int)(pidx + (i + 1) * KPI * 4), pe_bits));
        const bf16x2v pp = as_bf16x2(pack_bf16x2(pa, pb));
        const uint32_t aw[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
        const uint32_t bw[4] = {vr[i + 1].x, vr[i + 1].y, vr[i + 1].z, vr[i + 1].w};
  #pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          o[2 * jj] = __builtin_amdgcn_fdot2_f32_bf16(
              pp, as_bf16x2(__builtin_amdgcn_perm(bw[jj], aw[jj], 0x05040100u)), o[2 * jj], false);
          o[2 * jj + 1] = __builtin_amdgcn_fdot2_f32_bf16(
              pp, as_bf16x2(__builtin_amdgcn_perm(bw[jj], aw[jj], 0x07060302u)), o[2 * jj + 1], false);
        }
      }
    }

    // Reduce over the lanes that share a chunk column, and the row sums over all lanes.
  #pragma unroll
    for (int e = 0; e < 8; ++e)
  #pragma unroll
      for (int off = CPR; off < 64; off <<= 1) o[e] += __shfl_xor(o[e], off, 64);
    lsum = wave_sum_dpp(lsum);
    if (wave >= G) continue;  // padding head
    if (slot < 0) {
      if (lane < CPR) {
        const float inv = 1.f / lsum;
        float r[8];
  #pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = o[e] * inv;
        st16(out + ((size_t)token * Hq + (size_t)kvh * G + hg) * D + cl * 8, pack_chunk<bf16_t>(r));
      }
    } else {
      float* part = ws + (size_t)slot * G * (D + 2);
      if (lane == 0) {
        part[hg] = m_run;
        part[G + hg] = lsum;
      }
      if (lane < CPR) {
        float* dst = part + 2 * G + (size_t)hg * D + cl * 8;
  #pragma unroll
        for (int e = 0; e < 8; ++e) dst[e] = o[e];
      }
    }
  }  // items
}

// claim == nullptr: one workgroup per item.  Otherwise `workgroups` persistent
// workgroups (at most one per item) drain the list through the counter.
// Lean decode with two query heads per wavefront, for bf16 groups of 5 to 8 heads over
// blocks of at least 64 keys: four wavefronts cover up to eight heads, so each K and V
// chunk a lane reads from LDS serves two heads and a workgroup is half the size of an
// eight-wave one (four fit on a CU instead of two: more tiles in flight per CU).  The
// group's query rows sit in LDS (2 KB at head dim 128, read as broadcasts); the tile,
// the loader, the online softmax (one per head), P.V with the V chunks copied to
// registers before the barrier that frees the tile, the work items and the claim loop are
// those of the one-head kernel above, and so is each head's arithmetic and its order.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW == 4 ? 4 : 2, NW == 4 ? 4 : 2)))
void decode_lean2_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ pool,
    uint16_t* __restrict__ out, float* __restrict__ ws, const int4* __restrict__ work,
    const int32_t* __restrict__ tok2seq, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ block_off, const int32_t* __restrict__ block_ids, int32_t Hq,
    int32_t Hkv, int32_t G, int32_t bs, int32_t split_tiles, float scale_log2,
    int32_t* __restrict__ claim, int32_t n_items) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per key row
  constexpr int NT = NW * 64;                // threads
  constexpr int TILE_CHUNKS = 64 * CPR;      // chunks per K (or V) tile
  constexpr int NLD = TILE_CHUNKS / NT;      // direct loads per thread per K (or V) tile
  constexpr int KPI = 64 / CPR;              // P.V: keys per row group
  constexpr int NI = CPR;                    // P.V: row groups per tile
  constexpr int NH = 2 * NW;                 // heads the workgroup covers
  static_assert(TILE_CHUNKS % NT == 0 && NH * CPR <= NT, "loader geometry");
  __shared__ __attribute__((aligned(16))) uint16_t Kt[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t Qs[NH * D];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  auto next_item = [&]() -> int32_t {
    __syncthreads();  // every wave is done with the previous item's tile and query rows
    if (tid == 0) {
      const uint32_t c = (uint32_t)atomicAdd(claim, 1);
      Kt[0] = (uint16_t)c;
      Kt[1] = (uint16_t)(c >> 16);
    }
    __syncthreads();
    const int32_t it = __builtin_amdgcn_readfirstlane((int32_t)(Kt[0] | ((uint32_t)Kt[1] << 16)));
    __syncthreads();  // read by every wave before the next tile lands there
    return it;
  };
  for (int32_t item = claim ? next_item() : (int32_t)blockIdx.x; item < n_items;
       item = claim ? next_item() : n_items) {
    const int4 w = work[item];
    const int32_t token = w.x, kvh = w.y, split = w.z, slot = w.w;
    const int32_t seq = tok2seq[token];
    const int32_t nkeys = pos[token] + 1;
    const int32_t tiles_total = (nkeys + 63) >> 6;
    const int32_t t_begin = slot < 0 ? 0 : split * split_tiles;
    const int32_t t_end = slot < 0 ? tiles_total : min(tiles_total, t_begin + split_tiles);
    const int32_t key_end = min(nkeys, t_end * 64);
    const int32_t* bids = block_ids + block_off[seq];
    const int bsh = 31 - __builtin_clz(bs);  // block sizes are powers of two
    const int32_t last_blk = (key_end - 1) >> bsh;
    const size_t head_stride = (size_t)bs * D;
    const size_t blk_stride = (size_t)2 * Hkv * head_stride;
    const size_t v_off = (size_t)Hkv * head_stride;
    const uint16_t* pool_g = pool + (size_t)kvh * head_stride;
    // This wave's two heads (uniform); heads past G repeat the last one.
    const int32_t h0 = __builtin_amdgcn_readfirstlane(min(2 * wave, G - 1));
    const int32_t h1 = __builtin_amdgcn_readfirstlane(min(2 * wave + 1, G - 1));

    auto kswz = [](int r) { return CPR >= 16 ? (r & 15) : ((r >> 1) & (CPR - 1)); };
    auto fetch_ids = [&](int32_t t, int32_t* ids) { ids[0] = bids[min((t * 64) >> bsh, last_blk)]; };
    const uint32_t k_dst0 = __builtin_amdgcn_readfirstlane(lds_addr(&Kt[0]) + wave * 64 * 16);
    const uint32_t v_dst0 = __builtin_amdgcn_readfirstlane(lds_addr(&Vt[0]) + wave * 64 * 16);
    // Loader lanes: row tid / CPR + i * (NT / CPR) of the tile, chunk tid % CPR.  The K
    // swizzle depends on the row's low four bits, which change with i when a load covers
    // fewer than 16 rows (two waves at head dim 128), so it is taken per load.
    const int ld_r0 = tid / CPR, ld_c = tid % CPR;
    const uint32_t ld_vc = (uint32_t)ld_c * 16u;
    auto issue_tile = [&](int32_t t, const int32_t* ids) {
      const int32_t key0 = t * 64;
      const uint16_t* base = pool_g + (size_t)ids[0] * blk_stride + (size_t)(key0 & (bs - 1)) * D;
      const int32_t rmax = key_end - 1 - key0;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const uint32_t roff = (uint32_t)min(ld_r0 + i * (NT / CPR), rmax) * (D * 2);
        const uint32_t ld_kc = (uint32_t)(ld_c ^ kswz(ld_r0 + i * (NT / CPR))) * 16u;
        const uint32_t off = i * NT * 16;
        load_lds16_nt_s(base, roff + ld_kc, k_dst0 + off);
        load_lds16_nt_s(base + v_off, roff + ld_vc, v_dst0 + off);
      }
    };

    // The group's query rows into LDS (head slots past G repeat the last head); made
    // visible by the barrier at the top of the first tile.
    if (tid < NH * CPR) {
      const int hq = min(tid / CPR, G - 1), c = tid % CPR;
      const uint16_t* qrow = qkv + ((size_t)token * (Hq + 2 * Hkv) + (size_t)kvh * G + hq) * D;
      *(u32x4*)(Qs + tid * 8) = ld16(qrow + c * 8);
    }
    int32_t ids[1];
    fetch_ids(t_begin, ids);
    issue_tile(t_begin, ids);
    fetch_ids(min(t_begin + 1, t_end - 1), ids);

    float m_run[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f}, o[2][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[0][e] = o[1][e] = 0.f;
    const int cl = lane % CPR, kg = lane / CPR;  // P.V: chunk column and key sub-row
    uint32_t krow = (uint32_t)(lane * CPR + kswz(lane)) * 16u;
    uint32_t vcol = (uint32_t)(kg * CPR + cl) * 16u;
    uint32_t pidx = (uint32_t)kg * 4u;
    const u32x4* q0 = (const u32x4*)(Qs + h0 * D);
    const u32x4* q1 = (const u32x4*)(Qs + h1 * D);

    for (int32_t tt = t_begin; tt < t_end; ++tt) {
      wait_vmcnt<0>();  // this wave's share of tile tt (and its query-row load)
      __syncthreads();  // every wave's share
      const int32_t key0 = tt * 64;
      asm volatile("" : "+v"(krow), "+v"(vcol), "+v"(pidx));

      // Scores of both heads: lane = key, each K chunk read once.
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int c = 0; c < CPR; ++c) {
        const u32x4 kc = *(const u32x4*)((const char*)Kt + (krow ^ (16u * c)));
        s0 = dot_chunk(q0[c], kc, s0, bf16_t{});
        s1 = dot_chunk(q1[c], kc, s1, bf16_t{});
      }
      const bool valid = key0 + lane < key_end;
      float pe[2], alpha[2];
      {
        const float sc0 = valid ? s0 * scale_log2 : -INFINITY;
        const float sc1 = valid ? s1 * scale_log2 : -INFINITY;
        const float mn0 = fmaxf(m_run[0], wave_max_dpp(sc0));
        const float mn1 = fmaxf(m_run[1], wave_max_dpp(sc1));
        alpha[0] = __builtin_amdgcn_exp2f(m_run[0] - mn0);
        alpha[1] = __builtin_amdgcn_exp2f(m_run[1] - mn1);
        pe[0] = __builtin_amdgcn_exp2f(sc0 - mn0);
        pe[1] = __builtin_amdgcn_exp2f(sc1 - mn1);
        m_run[0] = mn0;
        m_run[1] = mn1;
        lsum[0] = lsum[0] * alpha[0] + pe[0];
        lsum[1] = lsum[1] * alpha[1] + pe[1];
      }
      u32x4 vr[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i)
        vr[i] = *(const u32x4*)((const char*)Vt + vcol + i * (KPI * CPR * 16));
      if (tt + 1 < t_end) {
        __syncthreads();  // every wave is done with the tile before it is overwritten
        issue_tile(tt + 1, ids);
        fetch_ids(min(tt + 2, t_end - 1), ids);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[0][e] *= alpha[0];
        o[1][e] *= alpha[1];
      }
      const int pb0 = __float_as_int(pe[0]), pb1 = __float_as_int(pe[1]);
#pragma unroll
      for (int i = 0; i < NI; i += 2) {
        const int ia = (int)(pidx + i * KPI * 4), ib = (int)(pidx + (i + 1) * KPI * 4);
        const bf16x2v pp0 = as_bf16x2(pack_bf16x2(__int_as_float(__builtin_amdgcn_ds_bpermute(ia, pb0)),
                                                  __int_as_float(__builtin_amdgcn_ds_bpermute(ib, pb0))));
        const bf16x2v pp1 = as_bf16x2(pack_bf16x2(__int_as_float(__builtin_amdgcn_ds_bpermute(ia, pb1)),
                                                  __int_as_float(__builtin_amdgcn_ds_bpermute(ib, pb1))));
        const uint32_t aw[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
        const uint32_t bw[4] = {vr[i + 1].x, vr[i + 1].y, vr[i + 1].z, vr[i + 1].w};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const bf16x2v lo = as_bf16x2(__builtin_amdgcn_perm(bw[jj], aw[jj], 0x05040100u));
          const bf16x2v hi = as_bf16x2(__builtin_amdgcn_perm(bw[jj], aw[jj], 0x07060302u));
          o[0][2 * jj] = __builtin_amdgcn_fdot2_f32_bf16(pp0, lo, o[0][2 * jj], false);
          o[0][2 * jj + 1] = __builtin_amdgcn_fdot2_f32_bf16(pp0, hi, o[0][2 * jj + 1], false);
          o[1][2 * jj] = __builtin_amdgcn_fdot2_f32_bf16(pp1, lo, o[1][2 * jj], false);
          o[1][2 * jj + 1] = __builtin_amdgcn_fdot2_f32_bf16(pp1, hi, o[1][2 * jj + 1], false);
        }
      }
    }

    // Reduce over the lanes that share a chunk column, and the row sums over all lanes.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int off = CPR; off < 64; off <<= 1) o[h][e] += __shfl_xor(o[h][e], off, 64);
      lsum[h] = wave_sum_dpp(lsum[h]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int32_t hh = h == 0 ? h0 : h1;
      if (2 * wave + h >= G) continue;  // padding head
      if (slot < 0) {
        if (lane < CPR) {
          const float inv = 1.f / lsum[h];
          float r[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) r[e] = o[h][e] * inv;
          st16(out + ((size_t)token * Hq + (size_t)kvh * G + hh) * D + cl * 8, pack_chunk<bf16_t>(r));
        }
      } else {
        float* part = ws + (size_t)slot * G * (D + 2);
        if (lane == 0) {
          part[hh] = m_run[h];
          part[G + hh] = lsum[h];
        }
        if (lane < CPR) {
          float* dst = part + 2 * G + (size_t)hh * D + cl * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) dst[e] = o[h][e];
        }
      }
    }
  }  // items
}

// Register-only decode for bf16 caches at head dim 128 over blocks of at least 64 keys,
// for groups of up to GP query heads (heads past G repeat the last one and write nothing);
// launched for single-head groups (GP = 1), where the lean kernel's four waves would
// compute one head four times: MHA decode 167 -> 155 us (the matrix-core kernel, one of
// its 16 columns used, 165-169 us), while groups of four heads measured equal to the lean
// kernel and groups of eight 21% slower (the per-lane score reduction grows with the
// group).  No LDS tile and no per-tile barrier: the four wavefronts of a workgroup
// each take 16 keys of every 64-key tile of the item, loading them straight into
// registers with coalesced non-temporal 16-byte loads (a wave instruction covers four
// whole key rows), the next tile's loads issued before the current tile is computed.
// Lane (r, c) of a wave (r = lane / 16, c = lane % 16) holds chunk c (dims 8c..8c+7) of
// the keys 16w + r + 4i, i = 0..3: Q.K is summed over the 16 lanes of the row with DPP,
// after which all 16 lanes of a row hold the same scores, weights and running maxima;
// each lane accumulates P.V for its own 8 dims.  Each row keeps its own online softmax
// (running maximum moved only by more than 2^8); at the end of the item the four rows
// and then the four waves (through 17 KB of LDS) are merged like split-K partials.
template <int GP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(GP >= 8 ? 1 : GP >= 4 ? 2 : 3, GP >= 8 ? 1 : GP >= 4 ? 2 : 3)))
void decode_reg_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ pool,
    uint16_t* __restrict__ out, float* __restrict__ ws, const int4* __restrict__ work,
    const int32_t* __restrict__ tok2seq, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ block_off, const int32_t* __restrict__ block_ids, int32_t Hq,
    int32_t Hkv, int32_t G, int32_t bs, int32_t split_tiles, float scale_log2,
    int32_t* __restrict__ claim, int32_t n_items) {
  constexpr int D = 128, NW = 4, NT = NW * 64;
  constexpr float SLACK = 8.f;
  __shared__ float red[NW][GP][D + 2];  // per wave: acc[D], then m, l
  __shared__ int32_t claimed;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane >> 4, c = lane & 15;

  auto next_item = [&]() -> int32_t {
    __syncthreads();
    if (tid == 0) claimed = atomicAdd(claim, 1);
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(claimed);
  };
  for (int32_t item = claim ? next_item() : (int32_t)blockIdx.x; item < n_items;
       item = claim ? next_item() : n_items) {
    const int4 w = work[item];
    const int32_t token = w.x, kvh = w.y, split = w.z, slot = w.w;
    const int32_t seq = tok2seq[token];
    const int32_t nkeys = pos[token] + 1;
    const int32_t tiles_total = (nkeys + 63) >> 6;
    const int32_t t_begin = slot < 0 ? 0 : split * split_tiles;
    const int32_t t_end = slot < 0 ? tiles_total : min(tiles_total, t_begin + split_tiles);
    const int32_t key_end = min(nkeys, t_end * 64);
    const int32_t* bids = block_ids + block_off[seq];
    const int bsh = 31 - __builtin_clz(bs);
    const size_t head_stride = (size_t)bs * D;
    const size_t blk_stride = (size_t)2 * Hkv * head_stride;
    const size_t v_off = (size_t)Hkv * head_stride;
    const uint16_t* pool_g = pool + (size_t)kvh * head_stride;

    u32x4 q[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h)
      q[h] = ld16(qkv + ((size_t)token * (Hq + 2 * Hkv) + (size_t)kvh * G + min(h, G - 1)) * D + c * 8);

    // Tile t into registers: rows 16*wave + r + 4i of the tile (clamped to the last key).
    typedef u32x4 Tile[4];
    auto load = [&](int32_t t, Tile& kt, Tile& vt) {
      const int32_t bid = bids[(t * 64) >> bsh];
      const uint16_t* base = pool_g + (size_t)bid * blk_stride + (size_t)((t * 64) & (bs - 1)) * D + c * 8;
      const int32_t rmax = key_end - 1 - t * 64;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t row = min(16 * wave + r + 4 * i, rmax);
        kt[i] = ldnt(base + (size_t)row * D);
        vt[i] = ldnt(base + v_off + (size_t)row * D);
      }
    };

    // The running maxima start finite (a row or wave may see no valid key of a short item:
    // its weights are then 2^-inf = 0 rather than 2^(-inf + inf)).
    float m[GP], l[GP], acc[GP][8];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      m[h] = -1e30f;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }
    // One tile: the next tile's loads go out first, then this tile is computed.
    auto step = [&](int32_t t, Tile& kc, Tile& vc, Tile& kn, Tile& vn) {
      if (t + 1 < t_end) load(t + 1, kn, vn);
      // scores of the row's four keys for every head, summed over the row's 16 lanes
      float sc[4][GP];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < GP; ++h) sc[i][h] = row16_sum(dot_chunk(q[h], kc[i], 0.f, bf16_t{}));
      bool moved = false;
      float mn[GP];
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        float mt = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool valid = t * 64 + 16 * wave + r + 4 * i < key_end;
          sc[i][h] = valid ? sc[i][h] * scale_log2 : -INFINITY;
          mt = fmaxf(mt, sc[i][h]);
        }
        mn[h] = fmaxf(m[h], mt);
        moved |= mn[h] > m[h] + SLACK;
      }
      if (__any(moved)) {
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          const float mnew = mn[h] > m[h] + SLACK ? mn[h] : m[h];
          const float alpha = __builtin_amdgcn_exp2f(m[h] - mnew);
          l[h] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
          m[h] = mnew;
        }
      }
      // P.V: two keys per v_dot2 (keys i and i+1 interleaved per column with v_perm_b32)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const uint32_t aw[4] = {vc[i].x, vc[i].y, vc[i].z, vc[i].w};
        const uint32_t bw[4] = {vc[i + 1].x, vc[i + 1].y, vc[i + 1].z, vc[i + 1].w};
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = __builtin_amdgcn_perm(bw[e], aw[e], 0x05040100u);
          hi[e] = __builtin_amdgcn_perm(bw[e], aw[e], 0x07060302u);
        }
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          const float pa = __builtin_amdgcn_exp2f(sc[i][h] - m[h]);
          const float pb = __builtin_amdgcn_exp2f(sc[i + 1][h] - m[h]);
          const uint32_t pp = pack_bf16x2(pa, pb);
          l[h] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pp), as_bf16x2(0x3f803f80u), l[h], false);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[h][2 * e] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pp), as_bf16x2(lo[e]), acc[h][2 * e], false);
            acc[h][2 * e + 1] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pp), as_bf16x2(hi[e]), acc[h][2 * e + 1], false);
          }
        }
      }
    };
    Tile k0, v0, k1, v1;
    load(t_begin, k0, v0);
    int32_t t = t_begin;
    for (; t + 1 < t_end; t += 2) {
      step(t, k0, v0, k1, v1);
      step(t + 1, k1, v1, k0, v0);
    }
    if (t < t_end) step(t, k0, v0, k1, v1);

    // Merge the wave's four rows (lanes c, c+16, c+32, c+48): common maximum, then sums.
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      float M = fmaxf(m[h], __shfl_xor(m[h], 16, 64));
      M = fmaxf(M, __shfl_xor(M, 32, 64));
      const float a = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[h] - M);
      l[h] *= a;
      l[h] += __shfl_xor(l[h], 16, 64);
      l[h] += __shfl_xor(l[h], 32, 64);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[h][e] * a;
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        acc[h][e] = v;
      }
      m[h] = M;
    }
    // Merge the four waves through LDS.
    if (r == 0) {
#pragma unroll
      for (int h = 0; h < GP; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[wave][h][c * 8 + e] = acc[h][e];
        if (c == 0) {
          red[wave][h][D] = m[h];
          red[wave][h][D + 1] = l[h];
        }
      }
    }
    __syncthreads();
    for (int u = tid; u < G * D; u += NT) {
      const int h = u / D, dim = u % D;
      float M = -INFINITY;
#pragma unroll
      for (int wv = 0; wv < NW; ++wv) M = fmaxf(M, red[wv][h][D]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int wv = 0; wv < NW; ++wv) {
        const float mw = red[wv][h][D];
        const float a = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        num = fmaf(a, red[wv][h][dim], num);
        den = fmaf(a, red[wv][h][D + 1], den);
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
    if (!claim) break;
  }  // items
}

// Decode on the matrix cores (bf16, head dim 128, blocks of 64+ keys, groups of up to 16
// heads): four wavefronts per workgroup, each streaming a 16-key slice of every 64-key
// step through its own LDS stages (mfma_decode::run_item).  With a claim counter the
// workgroups are persistent and take items from it.  Two stages (66 KB of LDS) let two
// workgroups share a CU, three (97 KB) one: the occupancy target follows.
template <int ST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4 - ST, 4 - ST)))
void decode_mfma_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ pool,
    uint16_t* __restrict__ out, float* __restrict__ ws, const int4* __restrict__ work,
    const int32_t* __restrict__ tok2seq, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ block_off, const int32_t* __restrict__ block_ids, int32_t Hq,
    int32_t Hkv, int32_t G, int32_t bs, int32_t split_tiles, float scale_log2,
    int32_t* __restrict__ claim, int32_t n_items) {
  __shared__ __attribute__((aligned(16))) uint16_t buf[mfma_decode::buf_elems<ST, 4>()];
  __shared__ float ml[mfma_decode::ml_floats<4>()];
  __shared__ int32_t claimed;
  auto next_item = [&]() -> int32_t {
    __syncthreads();  // the previous item's merge is read by every wave
    if (threadIdx.x == 0) claimed = atomicAdd(claim, 1);
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(claimed);
  };
  for (int32_t item = claim ? next_item() : (int32_t)blockIdx.x; item < n_items;
       item = claim ? next_item() : n_items)
    mfma_decode::run_item<ST, 4>(qkv, pool, out, ws, work, tok2seq, pos, block_off, block_ids, Hq,
                                 Hkv, G, bs, split_tiles, scale_log2, item, buf, ml);
}

template <int ST>
hipError_t launch_mfma(const rbkv_shape& s, const rbkv_batch& b, const void* qkv,
                       const void* pool, void* out, float* ws, hipStream_t stream,
                       int32_t* claim = nullptr, int32_t workgroups = 0) {
  const float scale_log2 = 1.4426950408889634f / sqrtf(128.f);
  const int G = s.n_q_heads / s.n_kv_heads;
  const int32_t grid = claim ? std::min(workgroups, b.n_decode_items) : b.n_decode_items;
  hipLaunchKernelGGL((decode_mfma_kernel<ST>), dim3(grid), dim3(256), 0, stream,
                     (const uint16_t*)qkv, (const uint16_t*)pool, (uint16_t*)out, ws,
                     (const int4*)b.decode_work, b.token_to_seq, b.pos, b.block_offsets,
                     b.block_ids, s.n_q_heads, s.n_kv_heads, G, s.block_size, b.split_tiles,
                     scale_log2, claim, b.n_decode_items);
  return hipGetLastError();
}

template <int GP>
hipError_t launch_reg(const rbkv_shape& s, const rbkv_batch& b, const void* qkv,
                      const void* pool, void* out, float* ws, hipStream_t stream,
                      int32_t* claim = nullptr, int32_t workgroups = 0) {
  const float scale_log2 = 1.4426950408889634f / sqrtf(128.f);
  const int G = s.n_q_heads / s.n_kv_heads;
  const int32_t grid = claim ? std::min(workgroups, b.n_decode_items) : b.n_decode_items;
  hipLaunchKernelGGL((decode_reg_kernel<GP>), dim3(grid), dim3(256), 0, stream,
                     (const uint16_t*)qkv, (const uint16_t*)pool, (uint16_t*)out, ws,
                     (const int4*)b.decode_work, b.token_to_seq, b.pos, b.block_offsets,
                     b.block_ids, s.n_q_heads, s.n_kv_heads, G, s.block_size, b.split_tiles,
                     scale_log2, claim, b.n_decode_items);
  return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_lean2(const rbkv_shape& s, const rbkv_batch& b, const void* qkv,
                        const void* pool, void* out, float* ws, hipStream_t stream,
                        int32_t* claim = nullptr, int32_t workgroups = 0) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  const int G = s.n_q_heads / s.n_kv_heads;
  const int32_t grid = claim ? std::min(workgroups, b.n_decode_items) : b.n_decode_items;
  hipLaunchKernelGGL((decode_lean2_kernel<D, NW>), dim3(grid), dim3(NW * 64), 0, stream,
                     (const uint16_t*)qkv, (const uint16_t*)pool, (uint16_t*)out, ws,
                     (const int4*)b.decode_work, b.token_to_seq, b.pos, b.block_offsets,
                     b.block_ids, s.n_q_heads, s.n_kv_heads, G, s.block_size, b.split_tiles,
                     scale_log2, claim, b.n_decode_items);
  return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_lean(const rbkv_shape& s, const rbkv_batch& b, const void* qkv,
                       const void* pool, void* out, float* ws, hipStream_t stream,
                       int32_t* claim = nullptr, int32_t workgroups = 0) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  const int G = s.n_q_heads / s.n_kv_heads;
  const int32_t grid = claim ? std::min(workgroups, b.n_decode_items) : b.n_decode_items;
  hipLaunchKernelGGL((decode_lean_kernel<D, NW>), dim3(grid), dim3(NW * 64), 0, stream,
                     (const uint16_t*)qkv, (const uint16_t*)pool, (uint16_t*)out, ws,
                     (const int4*)b.decode_work, b.token_to_seq, b.pos, b.block_offsets,
                     b.block_ids, s.n_q_heads, s.n_kv_heads, G, s.block_size, b.split_tiles,
                     scale_log2, claim, b.n_decode_items);
  return hipGetLastError();
}

// Zeroes the item counters of a call (a kernel rather than a memset, so that a captured
// graph holds no memset node).
__global__ void claims_reset_kernel(int32_t* claims, int n) {
  if ((int)threadIdx.x < n)
    __hip_atomic_store(claims + threadIdx.x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int NW>
hipError_t launch_group(const rbkv_shape& s, const rbkv_batch& b, const void* qkv,
                        const void* pool, void* out, float* ws, hipStream_t stream) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  const int G = s.n_q_heads / s.n_kv_heads;
  if (s.block_size >= 64)
    hipLaunchKernelGGL((decode_group_kernel<D, NW, true>), dim3(b.n_decode_items), dim3(NW * 64),
                       0, stream, (const uint16_t*)qkv, (const uint16_t*)pool, (uint16_t*)out, ws,
                       (const int4*)b.decode_work, b.token_to_seq, b.pos, b.block_offsets,
                       b.block_ids, s.n_q_heads, s.n_kv_heads, G, s.block_size, b.split_tiles,
                       scale_log2);
  else
    hipLaunchKernelGGL((decode_group_kernel<D, NW, false>), dim3(b.n_decode_items),
                       dim3(NW * 64), 0, stream, (const uint16_t*)qkv, (const uint16_t*)pool,
                       (uint16_t*)out, ws, (const int4*)b.decode_work, b.token_to_seq, b.pos,
                       b.block_offsets, b.block_ids, s.n_q_heads, s.n_kv_heads, G,
                       s.block_size, b.split_tiles, scale_log2);
  return hipGetLastError();
}

template <typename T, int D, int GMAX>
hipError_t launch_t(const rbkv_shape& s, const rbkv_batch& b, const void* qkv, const void* pool,
                    void* out, float* ws, hipStream_t stream) {
  const int G = s.n_q_heads / s.n_kv_heads;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  if (s.block_size >= 64)
    hipLaunchKernelGGL((decode_attn_kernel<T, D, GMAX, true>), dim3(b.n_decode_items), dim3(64),
                       0, stream, (const T*)qkv, (const T*)pool, (T*)out, ws,
                       (const int4*)b.decode_work, b.token_to_seq, b.pos, b.block_offsets,
                       b.block_ids, s.n_q_heads, s.n_kv_heads, G, s.block_size, b.split_tiles,
                       scale_log2);
  else
    hipLaunchKernelGGL((decode_attn_kernel<T, D, GMAX, false>), dim3(b.n_decode_items),
                       dim3(64), 0, stream, (const T*)qkv, (const T*)pool, (T*)out, ws,
                       (const int4*)b.decode_work, b.token_to_seq, b.pos, b.block_offsets,
                       b.block_ids, s.n_q_heads, s.n_kv_heads, G, s.block_size, b.split_tiles,
                       scale_log2);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_g(const rbkv_shape& s, const rbkv_batch& b, const void* qkv, const void* pool,
                    void* out, float* ws, hipStream_t stream) {
  const int G = s.n_q_heads / s.n_kv_heads;
  if constexpr (sizeof(T) == 2) {
    // Blocks of 64+ keys.  Head dim 128: groups of 2-16 heads on the matrix cores,
    // single-head groups on the register-only kernel.  Head dim 64, groups of up to 8
    // heads: one K/V tile per workgroup, one wave per head up to 4 heads, two for 5-8.
    if constexpr (D == 128) {
      if (decode_mfma_ok(s)) return launch_mfma<2>(s, b, qkv, pool, out, ws, stream);
      if (decode_reg_ok(s)) return launch_reg<1>(s, b, qkv, pool, out, ws, stream);
    } else {
      if (decode_lean_ok(s))
        return G <= 4 ? launch_lean<D, 4>(s, b, qkv, pool, out, ws, stream)
                      : launch_lean2<D, 4>(s, b, qkv, pool, out, ws, stream);
    }
    // Other bf16 groups of 5 or more heads: one wave per head over two LDS tile stages.
    if (decode_grouped(s))
      return G <= 8 ? launch_group<D, 8>(s, b, qkv, pool, out, ws, stream)
                    : launch_group<D, 16>(s, b, qkv, pool, out, ws, stream);
  }
  if (G <= 1) return launch_t<T, D, 1>(s, b, qkv, pool, out, ws, stream);
  if (G <= 2) return launch_t<T, D, 2>(s, b, qkv, pool, out, ws, stream);
  if (G <= 4) return launch_t<T, D, 4>(s, b, qkv, pool, out, ws, stream);
  if (G <= 8) return launch_t<T, D, 8>(s, b, qkv, pool, out, ws, stream);
  return launch_t<T, D, 16>(s, b, qkv, pool, out, ws, stream);
}

}  // namespace

hipError_t launch_claims_reset(int32_t* claims, int n, hipStream_t stream) {
  if (n < 1 || n > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(claims_reset_kernel, dim3(1), dim3(64), 0, stream, claims, n);
  return hipGetLastError();
}


hipError_t launch_decode_persistent(const rbkv_shape& s, const rbkv_batch& b, const void* qkv,
                                    const void* pool, void* out, float* ws, int32_t* claim,
                                    int32_t workgroups, hipStream_t stream, int stages) {
  if (decode_mfma_ok(s))
    return stages >= 3 ? launch_mfma<3>(s, b, qkv, pool, out, ws, stream, claim, workgroups)
                       : launch_mfma<2>(s, b, qkv, pool, out, ws, stream, claim, workgroups);
  if (decode_reg_ok(s)) return launch_reg<1>(s, b, qkv, pool, out, ws, stream, claim, workgroups);
  return s.n_q_heads / s.n_kv_heads <= 4
             ? launch_lean<64, 4>(s, b, qkv, pool, out, ws, stream, claim, workgroups)
             : launch_lean2<64, 4>(s, b, qkv, pool, out, ws, stream, claim, workgroups);
}

hipError_t launch_decode(const rbkv_shape& s, const rbkv_batch& b, const void* qkv,
                         const void* pool, void* out, float* ws, hipStream_t stream) {
  const bool bf = s.dtype == RBKV_DTYPE_BF16;
  if (s.head_dim == 128)
    return bf ? launch_g<bf16_t, 128>(s, b, qkv, pool, out, ws, stream)
              : launch_g<float, 128>(s, b, qkv, pool, out, ws, stream);
  return bf ? launch_g<bf16_t, 64>(s, b, qkv, pool, out, ws, stream)
            : launch_g<float, 64>(s, b, qkv, pool, out, ws, stream);
}

}  // namespace rbkv
