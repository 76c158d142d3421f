// Causal attention of bf16 prefill chunks on the gfx950 matrix cores.
//
// A workgroup takes one work item: (sequence, kv head, a run of up to 256/G of the chunk's
// tokens).  Its 256 query rows are (token, head-in-group) pairs, so every K/V tile in LDS
// serves all G query heads of the kv group.  Eight wavefronts own 32 rows each and, per
// 64-key tile, compute
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16, keys x rows, K from LDS, Q in registers),
//   an online softmax down each column (a lane owns one row: a column max is 16 register
//                 maxima plus one exchange with the partner lane 32 away),
//   O^T += V^T P^T (same instruction; P comes straight from the S^T accumulators, the V^T
//                 fragments from transposing LDS reads, ds_read_b64_tr_b16),
// with the causal mask applied bottom-right (the query at position p sees keys 0..p,
// p = seen + offset in the chunk) on the tiles that reach the diagonal only.
//
// Scheduling: waves w and w + 4 share a SIMD.  The two groups (waves 0-3, 4-7) alternate
// between a matrix-core block (P.V of tile k-1 and S^T of tile k) and a VALU block (the
// softmax of tile k), one block apart, so each SIMD's matrix core is fed by one wave while
// the other computes weights; the matrix-core block runs at raised issue priority.
//
// Data movement: K and V tiles go from HBM straight into LDS (global_load_lds_dwordx4, no
// staging registers) through a four-stage ring, two tiles ahead of use; block ids come
// through the scalar cache two tiles ahead of that.  In the prefill kernel four more
// wavefronts (one per SIMD, waves 8-11) issue every tile load and do nothing else, so the
// load issue (tens of cycles per instruction while the texture path is busy) stays off
// the compute waves; in the mixed kernel, which keeps eight wavefronts, group 1 issues
// them during its VALU block.  Each lane's source address is chosen so that the LDS image
// carries an XOR swizzle: K fragments (16 consecutive rows, one 16-byte chunk each) and
// transposing V reads are both free of bank conflicts.  Work items are mapped onto block
// indices so that the query tiles of one (sequence, kv head) run on the same XCD and share
// its L2.
//
// Dynamic SplitFuse chunks continuing a sequence with seen cached tokens:
// "DeepSpeed-Inference and DeepSpeed-MII", sections 10.3 and 10.10; query-tile sizing per
// head and blocked attention over work atoms: "DeepSpeed Inference v2 source tour",
// section "Ragged batches: packing a whole server into four tensors".
#include "decode_mfma.h"
#include "rbkv_device.h"
#include "rbkv_internal.h"

#include <type_traits>

namespace rbkv {
namespace {

constexpr int PF_WAVES = PF_ROWS / 32;
constexpr int PF_THREADS = 64 * PF_WAVES;
constexpr int PF_LW_THREADS = PF_THREADS + 256;  // eight compute and four loader wavefronts
constexpr int STAGES = 4;  // K/V tiles resident in LDS: one computed, up to three in flight
constexpr int N_XCD = 8;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// K tile: row = key (CPR 16-byte chunks); chunk c of row r sits at c ^ (r % 16)
// (r / 2 % 8 for 8-chunk rows): the 16 rows of one fragment read hit 16 bank groups.
template <int CPR>
__device__ __forceinline__ int kswz(int row) {
  return CPR >= 16 ? (row & 15) : ((row >> 1) & 7);
}
// V tile: row = key; chunk u of row r sits at u ^ (4 * (r % 4)) (CPR = 16) or
// u ^ (2 * (r % 4)) (CPR = 8): one transposing read (4 rows x 2 chunks per half-wave
// pair) covers all 64 banks.
template <int CPR>
__device__ __forceinline__ int vswz(int row) {
  return CPR >= 16 ? 4 * (row & 3) : 2 * (row & 3);
}

__device__ __forceinline__ bf16x8v as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8v, v); }

// 2^x with one v_exp_f32: results below the normal range flush to 0, which only drops
// softmax weights under 2^-126 of the running maximum.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum of a value and its copy 32 lanes away.  v_permlane32_swap of a register with
// itself hands every lane the pair (v[l % 32], v[l % 32 + 32]); being a VALU operation it
// does not wait on the LDS/scalar-memory counter that the scalar block-id loads in flight
// also hold.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) { return v + __shfl_xor(v, 32, 64); }

// One work item (kv group gidx = (sequence, kv head), query tile jq of the sequence's nqt)
// by the whole workgroup, with Ks / Vs the STAGES-tile K and V rings in LDS.  Every thread
// of the workgroup calls it; it ends with every wave past its last barrier.  LW: the
// workgroup has PF_THREADS + 256 threads and waves 8-11 are the loaders; otherwise it has
// PF_THREADS and group 1 loads.  BIG: blocks of 64 keys or more (bs >= 64), so a 64-key
// tile lies in one block (one block id per tile, one scalar base per load; the form for
// smaller blocks stays out of the code).  Ks and Vs must be 256-byte aligned (the
// fragment addresses are formed by XOR).  The pointers must be the calling kernel's own
// restrict parameters (the block ids are read through the scalar cache).
template <int D, bool LW, bool BIG>
__device__ __forceinline__ void prefill_item(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ pool,
    uint16_t* __restrict__ out, int32_t qtt, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ seen_arr, const int32_t* __restrict__ block_off,
    const int32_t* __restrict__ block_ids, int32_t Hq, int32_t Hkv, int32_t G, int32_t bs,
    float scale_log2, uint16_t (*Ks)[64 * D], uint16_t (*Vs)[64 * D], int32_t gidx,
    int32_t seq, int32_t nqt, int32_t jq) {
  constexpr int CPR = D / 8;                   // 16-byte chunks per key row
  constexpr int TILE_CHUNKS = 64 * CPR;        // chunks per K (or V) tile
  constexpr int LOADERS = PF_THREADS / 2;      // loader threads (group 1, or waves 8-11)
  constexpr int NLD = TILE_CHUNKS / LOADERS;   // direct loads per loader per K (or V) tile
  constexpr int LPT = 2 * NLD;                 // vector-memory operations per loader per tile
  constexpr int ROWS_PER_LD = LOADERS / CPR;   // key rows between a loader's loads (16 or 32)
  constexpr int KSTEPS = D / 16;               // MFMA k-steps over the head dim
  constexpr int DB = D / 32;                   // 32-wide dim blocks of the output
  constexpr int MAXNB = BIG ? 1 : 4;           // blocks a 64-key tile can span (1, or 4 at bs 16)
  static_assert(NLD >= 1 && ROWS_PER_LD % 16 == 0, "loader geometry");
  const int32_t kvh = gidx % Hkv;
  const int32_t qt = nqt - 1 - jq;
  const int32_t q0 = qt * qtt;
  const int32_t q1 = min(cu[seq + 1] - cu[seq], q0 + qtt);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  // Wave w and wave w + 4 of a workgroup share a SIMD: group 0 (waves 0-3) and group 1
  // (waves 4-7) take turns on each SIMD's matrix core.
  const int32_t grp = __builtin_amdgcn_readfirstlane(tid >> 8);
  const int hl = lane >> 5;     // half of the wave
  const int col = lane & 31;    // query row within the wave's 32

  const int32_t n_tok = q1 - q0;
  const int32_t rows = n_tok * G;
  const int32_t seen = seen_arr[seq];
  const int32_t tok0 = cu[seq] + q0;           // packed index of the item's first token
  const int32_t n_keys = seen + q1;            // keys visible to the last token
  const int32_t ntile = (n_keys + 63) >> 6;
  const int32_t* bids = block_ids + block_off[seq];
  const int bsh = 31 - __builtin_clz(bs);  // block sizes are powers of two
  const int32_t last_blk = (n_keys - 1) >> bsh;
  const size_t head_stride = (size_t)bs * D;
  const size_t v_off = (size_t)Hkv * head_stride;
  const uint16_t* pool_g = pool + (size_t)kvh * head_stride;

  // This lane's query row (clamped into range for the padding rows of the last item).
  const int32_t row = wave * 32 + col;
  const bool row_valid = row < rows;
  const int32_t rr = row_valid ? row : rows - 1;
  const int32_t rtok = rr / G, rhead = kvh * G + rr % G;
  const int32_t rpos = seen + q0 + rtok;

  // Loader role.  Direct load i of loader lt fills LDS chunk i*LOADERS + lt of a
  // tile: key row i*ROWS_PER_LD + lt/CPR and, after the swizzle, one of its chunks.  The
  // swizzles depend on the row's low four bits only, so they are the same for every i.
  const int lt = tid & (LOADERS - 1);
  const int lrow = lt / CPR;
  const int k_src = lrow * D + ((lt % CPR) ^ kswz<CPR>(lrow)) * 8;
  const int v_src = lrow * D + ((lt % CPR) ^ vswz<CPR>(lrow)) * 8;
  // Block ids of a tile: uniform across the workgroup, so they come through the scalar
  // cache and never hold up the vector-memory queue that carries the tile data.
  auto fetch_ids = [&](int32_t t, int32_t* ids) {
    const int32_t b0 = min((t * 64) >> bsh, last_blk);
#pragma unroll
    for (int j = 0; j < MAXNB; ++j) ids[j] = bids[min(b0 + j, last_blk)];
  };
  const size_t blk_stride = (size_t)2 * Hkv * head_stride;  // elements per pool block
  // LDS byte address where this wave's first direct load of a K tile lands (stage 0); a
  // V tile's sits STAGES tiles further.  Stage buf adds buf * TILE_BYTES, load i adds
  // i * LOADERS * 16.
  constexpr uint32_t TILE_BYTES = 64 * D * 2;
  const uint32_t k_dst0 = __builtin_amdgcn_readfirstlane(lds_addr(&Ks[0][0]) + (wave & 3) * 64 * 16);
  const uint32_t v_dst0 = __builtin_amdgcn_readfirstlane(lds_addr(&Vs[0][0]) + (wave & 3) * 64 * 16);
  auto issue_loads = [&](int32_t t, const int32_t* ids, int buf) {
    const uint32_t kd = k_dst0 + buf * TILE_BYTES, vd = v_dst0 + buf * TILE_BYTES;
    if constexpr (BIG) {
      // The tile sits in one block: a uniform base in scalar registers and 32-bit
      // per-thread offsets (measured 4% faster than 64-bit per-lane addresses).  Rows past
      // the end of a partial last tile load its last key (never read unmasked).
      const uint16_t* base = pool_g + (size_t)ids[0] * blk_stride + (size_t)((t * 64) & (bs - 1)) * D;
      const uint16_t* vbase = base + v_off;
      if (t * 64 + 63 < n_keys) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          load_lds16_s(base, (uint32_t)(i * ROWS_PER_LD * D + k_src) * 2u, kd + i * LOADERS * 16);
          load_lds16_s(vbase, (uint32_t)(i * ROWS_PER_LD * D + v_src) * 2u, vd + i * LOADERS * 16);
        }
      } else {
        const int32_t rmax = n_keys - 1 - t * 64;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const int32_t shift = (min(i * ROWS_PER_LD + lrow, rmax) - lrow) * D;
          load_lds16_s(base, (uint32_t)(shift + k_src) * 2u, kd + i * LOADERS * 16);
          load_lds16_s(vbase, (uint32_t)(shift + v_src) * 2u, vd + i * LOADERS * 16);
        }
      }
    } else {
      const int32_t b0 = (t * 64) >> bsh;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        // Rows past the end load the last key (never read unmasked).
        const int32_t key = min(t * 64 + i * ROWS_PER_LD + lrow, n_keys - 1);
        const int jb = (key >> bsh) - b0;
        const int32_t id = jb == 0 ? ids[0] : jb == 1 ? ids[1] : jb == 2 ? ids[2] : ids[3];
        const uint16_t* src = pool_g + (size_t)id * blk_stride + (size_t)(key & (bs - 1)) * D - lrow * D;
        load_lds16(src + k_src, kd + i * LOADERS * 16);
        load_lds16(src + v_off + v_src, vd + i * LOADERS * 16);
      }
    }
  };

  // Loader waves: the tile loads and waits that group 1 makes in the eight-wave form
  // (described with the block sequence below), at the same barriers, and nothing else.
  if constexpr (LW) {
    if (wave >= PF_WAVES) {
      int32_t ids[MAXNB];
      fetch_ids(0, ids);
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        if (j < ntile) issue_loads(j, ids, j);
        fetch_ids(j + 1, ids);
      }
      if (ntile > 2) wait_vmcnt<LPT>();
      else wait_vmcnt<0>();
      __syncthreads();
      for (int32_t p = 0; p <= 2 * ntile; ++p) {  // phase p ends at the next barrier
        if (p & 1) {
          const int32_t k = p >> 1;
          if (k + 2 < ntile) wait_vmcnt<LPT>();
          else wait_vmcnt<0>();
        } else if (p >= 2) {
          const int32_t k = (p >> 1) - 1;
          if (k + 3 < ntile) {
            issue_loads(k + 3, ids, (k + 3) % STAGES);
            fetch_ids(k + 4, ids);
          }
        }
        __syncthreads();
      }
      return;
    }
  }
  u32x4 qb[KSTEPS];  // Q^T operand: k-step s holds dims 16s + 8*hl .. +8 of this lane's row
  f32x16 oacc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 sacc[2];  // S^T of the current tile: block kb holds keys 32kb .. 32kb+31
  u32x4 pb[4];     // its weights in bf16, P^T operand of the four 16-key steps

  // Transposing-read addresses of the V^T fragments (element offsets into a V tile):
  // source lane 16g + 4j + r reads key kbase + 4(g/2) + j, dims 32d + 16(g%2) + 4r .. +4.
  const int tg = lane >> 4, tj = (lane >> 2) & 3, trr = lane & 3;
  const int vkey_in = 4 * (tg >> 1) + tj;                  // + kbase (multiple of 8)
  const int vdim_in = 16 * (tg & 1) + 4 * trr;             // + 32d
  // K fragment of k-step s for key row col (row 32 + col sits 32 rows further: the
  // swizzle depends on the row's low bits only): element offset in a K tile.

  // The two transposing reads that form the V^T fragment of step (kb, s2), dim block d.
  // Byte offsets, within a stage of the K (V) ring, of this lane's first K fragment read
  // (k-step 0, keys 0-31) and first V^T read (step 0, dim block 0).  With the swizzles
  // above, k-step s sits at kA ^ (s << 5) (+ 32 rows for keys 32-63) and V^T step st,
  // dim block d at (vB ^ (d << 6)) + 16 st rows (+ 8 rows for the second read): one XOR
  // per fragment from a stage base that is a multiple of 256 bytes.
  constexpr uint32_t RB = CPR * 16;  // bytes per key row
  const uint32_t kA = [&] {
    const int x = kswz<CPR>(col);
    return (uint32_t)(col * RB + 32 * (x >> 1) + 16 * (hl ^ (x & 1)));
  }();
  const uint32_t vB = [&] {
    const int r0 = vkey_in, u = vdim_in >> 3;
    return (uint32_t)(2 * ((r0 * CPR + (u ^ vswz<CPR>(r0))) * 8 + (vdim_in & 7)));
  }();
  auto vfrag = [&](uint32_t vbase, int step, int d) {
    const uint32_t a = (vbase ^ (uint32_t)(d << 6)) + step * 16 * RB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)a);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(a + 8 * RB));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2.x, l2.y, h2.x, h2.y};
  };
  // Matrix-core block: O^T += V^T P^T of tile t-1, then S^T of tile t (two 32-key blocks,
  // k-step chains alternating).  For P.V, MFMA k index 8*hl + j of step (kb, s2) is key
  // 32kb + 16s2 + 8(j/4) + 4hl + j%4: exactly the keys this lane's P registers hold.
  // P.V comes first so that the weights are dead before the scores are written: with the
  // fragment addresses formed by XOR the kernel fits 168 registers (three wavefronts per
  // SIMD) without spilling.  LDS reads run a fixed distance ahead of the MFMAs that use
  // them (one V^T fragment, one K k-step); scheduling fences keep the compiler from
  // hoisting them further, which would only cost registers.
  auto mblock = [&](int32_t t, auto do_qk, auto do_pv) {
    constexpr bool QK = decltype(do_qk)::value, PV = decltype(do_pv)::value;
    __builtin_amdgcn_s_setprio(1);
    const uint32_t kbase = lds_addr(Ks[t % STAGES]) + kA;
    const uint32_t vt = lds_addr(Vs[(t + STAGES - 1) % STAGES]) + vB;
    auto kfrag = [&](int s, int half) {
      const uint32_t a = (kbase ^ (uint32_t)(s << 5)) + half * 32 * RB;
      return *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)a;
    };
    constexpr int NV = 4 * DB;      // P.V MFMAs: step st = i / DB, dim block d = i % DB
    constexpr int VA = 1;           // V fragments read ahead of their MFMA
    u32x4 k0[2], k1[2];
    if constexpr (PV) {
      u32x4 vr[VA + 1];
#pragma unroll
      for (int i = 0; i < VA; ++i) vr[i] = vfrag(vt, i / DB, i % DB);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        if (i + VA < NV) vr[(i + VA) % (VA + 1)] = vfrag(vt, (i + VA) / DB, (i + VA) % DB);
        else if (QK && i + VA == NV) { k0[0] = kfrag(0, 0); k1[0] = kfrag(0, 1); }
        __builtin_amdgcn_sched_barrier(0);
        oacc[i % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(vr[i % (VA + 1)]), as_bf16x8(pb[i / DB]), oacc[i % DB], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      k0[0] = kfrag(0, 0);
      k1[0] = kfrag(0, 1);
    }
    if constexpr (QK) {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        if (s + 1 < KSTEPS) {
          k0[(s + 1) & 1] = kfrag(s + 1, 0);
          k1[(s + 1) & 1] = kfrag(s + 1, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(k0[s & 1]), as_bf16x8(qb[s]), s == 0 ? f32x16{} : sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(k1[s & 1]), as_bf16x8(qb[s]), s == 0 ? f32x16{} : sacc[1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // Causal mask (bottom-right): register r of block kb holds key t*64 + 32kb + 8(r/4) +
  // 4hl + r%4, which this lane's query (position rpos) sees iff it is <= rpos.
  auto mask_tile = [&](int32_t t) {
    const int32_t lim = rpos - t * 64 - 4 * hl;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) sacc[kb][r] = -INFINITY;
  };
  // Tiles t < t_free are visible to every query of the item (t*64 + 63 <= seen + q0).
  const int32_t t_free = (seen + q0 + 1) >> 6;
  // Online softmax of tile t: mask, running maximum, weights 2^(s*scale - m), their sum
  // and bf16 packing.  The running maximum m moves only when some row's maximum exceeds
  // it by more than RESCALE_SLACK (log2 units): weights then stay below 2^RESCALE_SLACK
  // and O and l are rescaled rarely.  The result is the same softmax; only the common
  // factor that the partial sums carry differs.  The first tile always moves m (from
  // -inf: key 0 is visible to every row, so its maximum is finite).
  constexpr float RESCALE_SLACK = 8.f;
  auto softmax = [&](int32_t t) {
    if (t >= t_free) mask_tile(t);
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
    mt = pair_max(mt);  // the other half of this row's keys lives 32 lanes away
    const float mn = fmaxf(m_run, mt * scale_log2);
    if (__any(mn > m_run + RESCALE_SLACK)) {
      const float alpha = fast_exp2(m_run - mn);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
      m_run = mn;
    }
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = fast_exp2(fmaf(sacc[kb][8 * s2 + j], scale_log2, -m_run));
          psum += p[j];
        }
        pb[2 * kb + s2] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
      }
    l_run += psum;
  };

  // Every wave runs the same sequence of blocks, a barrier after each:
  //   M_0, V_0, M_1, V_1, ..., M_{n-1}, V_{n-1}, M_n        (n = ntile)
  // with M_k = S^T of tile k (k < n) and P.V of tile k-1 (k >= 1) on the matrix core,
  // and V_k = softmax of tile k on the VALU.  Group 1 takes one extra barrier before M_0
  // and group 0 one after M_n, so group 1 runs one block behind: on every SIMD one wave
  // feeds the matrix core while the other does the softmax.  In the barrier-delimited
  // phases p = 0 .. 2n+1, group 0 runs M_k in phase 2k and group 1 in phase 2k+1.
  //
  // Tile loads, all by group 1 (by the loader waves when LW, in the same phases): tiles 0,
  // 1 and 2 in the prologue, tile k+3 at the start of its V_k (phase 2k+2) into the stage
  // of tile k-1, whose last reader (group 1's M_k) ran in phase 2k+1.  After its M_k
  // (phase 2k+1) group 1 waits for tile k+1, which group 0 reads first in phase 2k+2;
  // tile k+2 (issued in phase 2k) may still be in flight.
  int32_t ids[MAXNB];
  if (!LW) fetch_ids(0, ids);
  if (!LW && grp == 1) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      if (j < ntile) issue_loads(j, ids, j);
      fetch_ids(j + 1, ids);
    }
  }
  {
    const uint16_t* qr = qkv + ((size_t)(tok0 + rtok) * (Hq + 2 * Hkv) + rhead) * D;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qb[s] = ld16(qr + 16 * s + 8 * hl);
  }
  // Tiles 0 and 1 and the Q^T operand resident; tile 2 may stay in flight.  Afterwards
  // no register load is outstanding: every vector-memory operation in the loop is a
  // tile load whose completion these waits track.
  if (!LW && grp == 1 && ntile > 2) wait_vmcnt<LPT>();
  else wait_vmcnt<0>();
  __syncthreads();
  if (grp == 1) __syncthreads();  // group 1 starts one phase behind

  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  auto after_m = [&](int32_t kk) {  // group 1, end of M_kk: tile kk+1 resident
    if (!LW && grp == 1) {
      if (kk + 2 < ntile) wait_vmcnt<LPT>();
      else wait_vmcnt<0>();
    }
    __syncthreads();
  };
  auto before_v = [&](int32_t kk) {  // group 1, start of V_kk: tile kk+3 into flight
    if (!LW && grp == 1 && kk + 3 < ntile) {
      issue_loads(kk + 3, ids, (kk + 3) % STAGES);
      fetch_ids(kk + 4, ids);
    }
  };
  mblock(0, yes{}, no{});
  after_m(0);
  before_v(0);
  softmax(0);
  __syncthreads();
  for (int32_t kk = 1; kk < ntile; ++kk) {
    mblock(kk, yes{}, yes{});
    after_m(kk);
    before_v(kk);
    softmax(kk);
    __syncthreads();
  }
  mblock(ntile, no{}, yes{});
  if (grp == 0) __syncthreads();  // matches group 1's extra barrier

  if (!row_valid) return;
  const float l_tot = pair_sum(l_run);
  const float inv = 1.f / l_tot;
  uint16_t* orow = out + ((size_t)(tok0 + rtok) * Hq + rhead) * D;
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int dim = 32 * d + 8 * g4 + 4 * hl;
      u32x2 v;
      v.x = pack_bf16x2(oacc[d][4 * g4 + 0] * inv, oacc[d][4 * g4 + 1] * inv);
      v.y = pack_bf16x2(oacc[d][4 * g4 + 2] * inv, oacc[d][4 * g4 + 3] * inv);
      *(u32x2*)(orow + dim) = v;
    }
}

// Work placement.  Block b runs on XCD b % 8.  The (sequence, kv head) groups, in the
// order of the ranked chunk sequences (longest first), are dealt round-robin over the
// XCDs, so each XCD gets an even share; the query tiles of one group run back to back on
// one XCD (longest tile first) and share its L2.  Slots past a group's tiles exit.
// BIG: blocks of 64 keys or more.
template <int D, bool BIG>
__global__ __launch_bounds__(PF_LW_THREADS, 1) void prefill_attn_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ pool,
    uint16_t* __restrict__ out, const int4* __restrict__ work, int32_t n_groups, int32_t nq_max,
    int32_t qtt, const int32_t* __restrict__ cu, const int32_t* __restrict__ seen_arr,
    const int32_t* __restrict__ block_off, const int32_t* __restrict__ block_ids, int32_t Hq,
    int32_t Hkv, int32_t G, int32_t bs, float scale_log2) {
  __shared__ __attribute__((aligned(1024))) uint16_t Ks[STAGES][64 * D];
  __shared__ __attribute__((aligned(1024))) uint16_t Vs[STAGES][64 * D];
  const int32_t xcd = (int32_t)(blockIdx.x % N_XCD);
  const int32_t k = (int32_t)(blockIdx.x / N_XCD);
  const int32_t gidx = (k / nq_max) * N_XCD + xcd;
  if (gidx >= n_groups) return;  // whole workgroup leaves together
  const int4 rec = work[gidx / Hkv];
  const int32_t seq = rec.x, nqt = rec.y;
  const int32_t jq = k % nq_max;
  if (jq >= nqt) return;
  prefill_item<D, true, BIG>(qkv, pool, out, qtt, cu, seen_arr, block_off, block_ids, Hq,
                             Hkv, G, bs, scale_log2, Ks, Vs, gidx, seq, nqt, jq);
}

// Mixed batches (bf16, head dim 128, groups of 2-16 heads, blocks of 64+ keys): one
// persistent workgroup per CU takes items from both work lists, so the two phases share
// the chip by CUs inside one launch.  A workgroup starts on the decode list if it is one of
// the first dec_first of its XCD (block b runs on XCD b % 8), on the prefill list
// otherwise, and moves to the other list when its own is exhausted; it leaves when both
// are.  Prefill items come from per-XCD lists (the placement of prefill_attn_kernel, with
// a counter per XCD in claims[1 + xcd]; a workgroup whose list is exhausted moves to the
// list with the most slots left), decode items from one list (claims[0]), eight
// wavefronts per item (mfma_decode::run_item, two stages).  The ring of the prefill and the
// stages of the decode share the LDS.  claims[0..8] must be zero at launch.
__global__ __launch_bounds__(PF_THREADS, 1) void mixed_attn_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ pool,
    uint16_t* __restrict__ out, float* __restrict__ ws, const int4* __restrict__ pwork,
    int32_t n_groups, int32_t nq_max, int32_t qtt, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ seen_arr, const int4* __restrict__ dwork,
    const int32_t* __restrict__ tok2seq, const int32_t* __restrict__ pos, int32_t n_dec,
    int32_t split_tiles, const int32_t* __restrict__ block_off,
    const int32_t* __restrict__ block_ids, int32_t Hq, int32_t Hkv, int32_t G, int32_t bs,
    float scale_log2, int32_t* __restrict__ claims, int32_t dec_first) {
  constexpr int D = 128;
  constexpr int RING = STAGES * 64 * D;  // elements of the prefill's K (or V) ring
  static_assert(mfma_decode::buf_elems<2, PF_WAVES>() <= 2 * RING, "decode stages fit the ring");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * RING];
  __shared__ float ml[mfma_decode::ml_floats<PF_WAVES>()];
  __shared__ int32_t claimed, chosen;
  uint16_t(*Ks)[64 * D] = (uint16_t(*)[64 * D])lds;
  uint16_t(*Vs)[64 * D] = (uint16_t(*)[64 * D])(lds + RING);
  // XCD this workgroup runs on (hardware register XCC_ID, bits 0-3).
  const int32_t home = (int32_t)(__builtin_amdgcn_s_getreg(20 | (3 << 11)) & (N_XCD - 1));
  bool dec = (int32_t)(blockIdx.x / N_XCD) < dec_first;
  bool pre_left = n_groups > 0, dec_left = n_dec > 0;
  int32_t xcd = home;  // prefill list being drained
  const int32_t groups_per_list = (n_groups + N_XCD - 1) / N_XCD;
  while (pre_left || dec_left) {
    if (!pre_left) dec = true;
    if (!dec_left) dec = false;
    __syncthreads();  // the previous item is done with the LDS and the claim word
    if (threadIdx.x == 0) claimed = atomicAdd(dec ? &claims[0] : &claims[1 + xcd], 1);
    __syncthreads();
    const int32_t c = __builtin_amdgcn_readfirstlane(claimed);
    if (dec) {
      if (c >= n_dec) {
        dec_left = false;
        continue;
      }
      mfma_decode::run_item<2, PF_WAVES>(qkv, pool, out, ws, dwork, tok2seq, pos, block_off,
                                         block_ids, Hq, Hkv, G, bs, split_tiles, scale_log2, c,
                                         lds, ml);
    } else {
      const int32_t gidx = (c / nq_max) * N_XCD + xcd;
      if (gidx >= n_groups) {
        // This list is exhausted: move to the one with the most slots left, or leave the
        // prefill lists when none has any.  (Slots: list x holds the query tiles of
        // groups x, x + 8, ...; its counter may run past them.)
        if (threadIdx.x < 64) {
          const int x = threadIdx.x & (N_XCD - 1);
          const int32_t groups_x =
              x < n_groups % N_XCD || n_groups % N_XCD == 0 ? groups_per_list : groups_per_list - 1;
          const int32_t left =
              threadIdx.x < N_XCD
                  ? groups_x * nq_max -
                        __hip_atomic_load(&claims[1 + x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                  : -1;
          int32_t best = left > 0 ? (left << 3) | x : -1;
#pragma unroll
          for (int o = 1; o < N_XCD; o <<= 1) best = max(best, __shfl_xor(best, o, 64));
          if (threadIdx.x == 0) chosen = best < 0 ? -1 : (best & (N_XCD - 1));
        }
        __syncthreads();
        const int32_t next = __builtin_amdgcn_readfirstlane(chosen);
        if (next < 0) pre_left = false;
        else xcd = next;
        continue;
      }
      const int4 rec = pwork[gidx / Hkv];
      const int32_t jq = c % nq_max;
      if (jq >= rec.y) continue;
      prefill_item<D, false, true>(qkv, pool, out, qtt, cu, seen_arr, block_off, block_ids, Hq,
                                   Hkv, G, bs, scale_log2, Ks, Vs, gidx, rec.x, rec.y, jq);
    }
  }
}

template <int D, bool BIG>
hipError_t launch_t(const rbkv_shape& s, const rbkv_batch& b, const void* qkv, const void* pool,
                    void* out, hipStream_t stream) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  const int32_t n_groups = b.n_prefill_seqs * s.n_kv_heads;
  const int32_t grid = ((n_groups + N_XCD - 1) / N_XCD) * b.prefill_qtiles_max * N_XCD;
  const int32_t qtt = q_tile_tokens(s.n_q_heads / s.n_kv_heads);
  hipLaunchKernelGGL((prefill_attn_kernel<D, BIG>), dim3(grid), dim3(PF_LW_THREADS), 0, stream,
                     (const uint16_t*)qkv, (const uint16_t*)pool, (uint16_t*)out,
                     (const int4*)b.prefill_work, n_groups, b.prefill_qtiles_max, qtt,
                     b.cu_seqlens, b.seen, b.block_offsets,
                     b.block_ids, s.n_q_heads, s.n_kv_heads, s.n_q_heads / s.n_kv_heads,
                     s.block_size, scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mixed(const rbkv_shape& s, const rbkv_batch& b, const void* qkv,
                        const void* pool, void* out, float* ws, int32_t* claims,
                        int32_t workgroups, int32_t dec_first, hipStream_t stream) {
  if (!decode_mfma_ok(s)) return hipErrorInvalidValue;
  const float scale_log2 = 1.4426950408889634f / sqrtf(128.f);
  const int32_t G = s.n_q_heads / s.n_kv_heads;
  hipLaunchKernelGGL(mixed_attn_kernel, dim3(workgroups), dim3(PF_THREADS), 0, stream,
                     (const uint16_t*)qkv, (const uint16_t*)pool, (uint16_t*)out, ws,
                     (const int4*)b.prefill_work, b.n_prefill_seqs * s.n_kv_heads,
                     b.prefill_qtiles_max, q_tile_tokens(G), b.cu_seqlens, b.seen,
                     (const int4*)b.decode_work, b.token_to_seq, b.pos, b.n_decode_items,
                     b.split_tiles, b.block_offsets, b.block_ids, s.n_q_heads, s.n_kv_heads, G,
                     s.block_size, scale_log2, claims, dec_first);
  return hipGetLastError();
}

hipError_t launch_prefill(const rbkv_shape& s, const rbkv_batch& b, const void* qkv,
                          const void* pool, void* out, hipStream_t stream) {
  if (s.dtype != RBKV_DTYPE_BF16) return hipErrorInvalidValue;  // float32 chunks use the VALU path
  const bool big = s.block_size >= 64;
  if (s.head_dim == 128)
    return big ? launch_t<128, true>(s, b, qkv, pool, out, stream)
               : launch_t<128, false>(s, b, qkv, pool, out, stream);
  return big ? launch_t<64, true>(s, b, qkv, pool, out, stream)
             : launch_t<64, false>(s, b, qkv, pool, out, stream);
}

}  // namespace rbkv
