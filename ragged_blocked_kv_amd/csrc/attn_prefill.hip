// Causal attention of bf16 prefill chunks on the gfx950 matrix cores.
//
// A work item is (sequence, kv head, a run of the chunk's tokens).  Its 128 query rows
// are (token, head-in-group) pairs, so every K/V tile loaded into LDS serves all G query
// heads of the kv group.  Each of the 4 wavefronts owns 32 rows and runs
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16, keys x rows, K from LDS, Q held in registers)
//   online softmax down each column (the lane owns one row: a column max is 16 register
//                 maxima plus one exchange with the partner lane 32 away),
//   O^T += V^T P^T (same instruction; P comes straight from the S^T accumulators, the
//                 V^T fragments from transposing LDS reads, ds_read_b64_tr_b16),
// over 64-key tiles, with the causal mask applied bottom-right (query at position p sees
// keys 0..p, p = seen + offset in the chunk) and only on the tiles that need it.
//
// Data movement: K and V tiles go from HBM straight into LDS (global_load_lds_dwordx4,
// no staging registers), double-buffered with one barrier per tile; the next tile is
// in flight while the current one is computed, and block ids are fetched one tile
// further ahead.  Each lane's source address is chosen so that the LDS image carries an
// XOR swizzle: K fragments (16 consecutive rows, one 16-byte chunk each) and transposed
// V reads (8 keys x 32 dims per instruction) are both free of bank conflicts.  Work
// items are mapped onto block indices so that the query tiles of one (sequence,
// kv head) run on the same XCD and share its L2.
//
// Dynamic SplitFuse chunks continuing a sequence with seen cached tokens:
// "DeepSpeed-Inference and DeepSpeed-MII", sections 10.3 and 10.10; query-tile sizing per
// head and blocked attention over work atoms: "DeepSpeed Inference v2 source tour",
// section "Ragged batches: packing a whole server into four tensors".
#include "rbkv_device.h"
#include "rbkv_internal.h"

namespace rbkv {
namespace {

constexpr int PF_WAVES = PF_ROWS / 32;
constexpr int PF_THREADS = 64 * PF_WAVES;
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

// Max / sum of a value and its copy 32 lanes away (one v_permlane32_swap, no LDS).
__device__ __forceinline__ float pair_max(float v) { return fmaxf(v, __shfl_xor(v, 32, 64)); }
__device__ __forceinline__ float pair_sum(float v) { return v + __shfl_xor(v, 32, 64); }

__device__ __forceinline__ u32x2 ds_read_tr(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Wait until at most n vector-memory operations of this wave are outstanding (the LDS
// DMA loads of later tiles stay in flight); expcnt and lgkmcnt are left alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int D>
__global__ __launch_bounds__(PF_THREADS, 1) void prefill_attn_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ pool,
    uint16_t* __restrict__ out, const int4* __restrict__ work, int32_t n_groups, int32_t nq_max,
    int32_t qtt, const int32_t* __restrict__ cu, const int32_t* __restrict__ seen_arr,
    const int32_t* __restrict__ block_off, const int32_t* __restrict__ block_ids, int32_t Hq,
    int32_t Hkv, int32_t G, int32_t bs, float scale_log2) {
  constexpr int CPR = D / 8;               // 16-byte chunks per key row
  constexpr int TILE_CHUNKS = 64 * CPR;    // chunks per K (or V) tile
  constexpr int NLD = TILE_CHUNKS / PF_THREADS;  // direct loads per thread per K (or V) tile
  constexpr int LPT = 2 * NLD;             // vector-memory operations per thread per tile
  constexpr int KSTEPS = D / 16;           // MFMA k-steps over the head dim
  constexpr int DB = D / 32;               // 32-wide dim blocks of the output
  constexpr int MAXNB = 4;                 // blocks a 64-key tile can span (block size 16)
  static_assert(NLD >= 1, "tile smaller than the workgroup");
  __shared__ __attribute__((aligned(16))) uint16_t Ks[STAGES][64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[STAGES][64 * D];

  // Work placement.  Block b runs on XCD b % 8.  The (sequence, kv head) groups, in the
  // order of the ranked chunk sequences (longest first), are dealt round-robin over the
  // XCDs, so each XCD gets an even share; the query tiles of one group run back to back
  // on one XCD (longest tile first) and share its L2.  Slots past a group's tiles exit.
  const int32_t xcd = (int32_t)(blockIdx.x % N_XCD);
  const int32_t k = (int32_t)(blockIdx.x / N_XCD);
  const int32_t gidx = (k / nq_max) * N_XCD + xcd;
  if (gidx >= n_groups) return;  // whole workgroup leaves together
  const int4 rec = work[gidx / Hkv];
  const int32_t seq = rec.x, nqt = rec.y;
  const int32_t jq = k % nq_max;
  if (jq >= nqt) return;
  const int32_t kvh = gidx % Hkv;
  const int32_t qt = nqt - 1 - jq;
  const int32_t q0 = qt * qtt;
  const int32_t q1 = min(cu[seq + 1] - cu[seq], q0 + qtt);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hl = lane >> 5;     // half of the wave
  const int col = lane & 31;    // query row within the wave's 32

  const int32_t n_tok = q1 - q0;
  const int32_t rows = n_tok * G;
  const int32_t seen = seen_arr[seq];
  const int32_t tok0 = cu[seq] + q0;           // packed index of the item's first token
  const int32_t n_keys = seen + q1;            // keys visible to the last token
  const int32_t ntile = (n_keys + 63) >> 6;
  const int32_t* bids = block_ids + block_off[seq];
  const int32_t last_blk = (n_keys - 1) / bs;
  const size_t head_stride = (size_t)bs * D;
  const size_t v_off = (size_t)Hkv * head_stride;
  const uint16_t* pool_g = pool + (size_t)kvh * head_stride;

  // This lane's query row (clamped into range for the padding rows of the last item).
  const int32_t row = wave * 32 + col;
  const bool row_valid = row < rows;
  const int32_t rr = row_valid ? row : rows - 1;
  const int32_t rtok = rr / G, rhead = kvh * G + rr % G;
  const int32_t rpos = seen + q0 + rtok;
  // Rows spanned by this wave, for tile skipping and mask-free tiles.
  const int32_t w_lo = wave * 32;
  const bool wave_active = w_lo < rows;
  const int32_t w_hi = min(rows, w_lo + 32) - 1;
  const int32_t pmin = seen + q0 + (wave_active ? w_lo / G : 0);
  const int32_t pmax = seen + q0 + (wave_active ? w_hi / G : 0);


  // Loader role: direct load i of this thread fills LDS chunk i*PF_THREADS + tid of a
  // tile, which holds row (i*PF_THREADS + tid) / CPR and, after the swizzle, a chunk of
  // that row.
  int krow[NLD], kchk[NLD], vchk[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int pos = i * PF_THREADS + tid;
    krow[i] = pos / CPR;
    kchk[i] = (pos % CPR) ^ kswz<CPR>(krow[i]);
    vchk[i] = (pos % CPR) ^ vswz<CPR>(krow[i]);
  }
  // Block ids of a tile: uniform across the workgroup, so they come through the scalar
  // cache and never hold up the vector-memory queue that carries the tile data.
  auto fetch_ids = [&](int32_t t, int32_t* ids) {
    const int32_t b0 = min((t * 64) / bs, last_blk);
#pragma unroll
    for (int j = 0; j < MAXNB; ++j) ids[j] = bids[min(b0 + j, last_blk)];
  };
  const size_t blk_stride = (size_t)2 * Hkv * head_stride;  // elements per pool block
  // LDS byte address where this wave's first direct load of a K tile lands (stage 0); a
  // V tile's sits STAGES tiles further.  Stage buf adds buf * TILE_BYTES, load i adds
  // i * PF_THREADS * 16.
  constexpr uint32_t TILE_BYTES = 64 * D * 2;
  const uint32_t k_dst0 = __builtin_amdgcn_readfirstlane(lds_addr(&Ks[0][0]) + wave * 64 * 16);
  const uint32_t v_dst0 = __builtin_amdgcn_readfirstlane(lds_addr(&Vs[0][0]) + wave * 64 * 16);
  auto issue_loads = [&](int32_t t, const int32_t* ids, int buf) {
    const uint32_t kd = k_dst0 + buf * TILE_BYTES, vd = v_dst0 + buf * TILE_BYTES;
    if (bs >= 64 && t * 64 + 63 < n_keys) {
      // The whole tile sits in one block: one uniform base, fixed per-thread offsets.
      const uint16_t* base = pool_g + (size_t)ids[0] * blk_stride + (size_t)((t * 64) % bs) * D;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const uint16_t* src = base + krow[i] * D;
        load_lds16(src + kchk[i] * 8, kd + i * PF_THREADS * 16);
        load_lds16(src + v_off + vchk[i] * 8, vd + i * PF_THREADS * 16);
      }
      return;
    }
    const int32_t b0 = (t * 64) / bs;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int32_t key = min(t * 64 + krow[i], n_keys - 1);  // rows past the end: last key
      const int jb = key / bs - b0;
      const int32_t id = jb == 0 ? ids[0] : jb == 1 ? ids[1] : jb == 2 ? ids[2] : ids[3];
      const uint16_t* src = pool_g + (size_t)id * blk_stride + (size_t)(key % bs) * D;
      load_lds16(src + kchk[i] * 8, kd + i * PF_THREADS * 16);
      load_lds16(src + v_off + vchk[i] * 8, vd + i * PF_THREADS * 16);
    }
  };

  u32x4 qb[KSTEPS];  // Q^T operand, loaded in the prologue
  f32x16 oacc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Transposing-read addresses of the V^T fragments (element offsets into a V tile):
  // source lane 16g + 4j + r reads key kbase + 4(g/2) + j, dims 32d + 16(g%2) + 4r .. +4.
  const int tg = lane >> 4, tj = (lane >> 2) & 3, trr = lane & 3;
  const int vkey_in = 4 * (tg >> 1) + tj;                  // + kbase (multiple of 8)
  const int vdim_in = 16 * (tg & 1) + 4 * trr;             // + 32d

  // QK of one tile into S^T (two 32-key blocks, chains interleaved; K fragments are
  // streamed one k-step ahead of the MFMAs that use them).
  auto qk = [&](int32_t t, f32x16* sacc) {
    const int buf = t % STAGES;
    const uint16_t* kt = Ks[buf];
    const int r0 = col, r1 = 32 + col;
    auto frag = [&](int row, int s) {
      return *(const u32x4*)(kt + (row * CPR + ((2 * s + hl) ^ kswz<CPR>(row))) * 8);
    };
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
    u32x4 a0 = frag(r0, 0), a1 = frag(r1, 0);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      u32x4 n0 = a0, n1 = a1;
      if (s + 1 < KSTEPS) {
        n0 = frag(r0, s + 1);
        n1 = frag(r1, s + 1);
      }
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0), as_bf16x8(qb[s]), sacc[0],
                                                        0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a1), as_bf16x8(qb[s]), sacc[1],
                                                        0, 0, 0);
      a0 = n0;
      a1 = n1;
    }
  };
  // The two transposing reads that form the V^T fragment of step (kb, s2), dim block d.
  auto vfrag = [&](const uint16_t* vt, int step, int d) {
    const int kbase = 16 * step;  // step = 2 kb + s2: keys 32kb + 16s2
    const int r0 = kbase + vkey_in, r1 = r0 + 8;
    const int dim = 32 * d + vdim_in;
    const int u = dim >> 3, half = dim & 7;
    const u32x2 lo = ds_read_tr(vt + (r0 * CPR + (u ^ vswz<CPR>(r0))) * 8 + half);
    const u32x2 hi = ds_read_tr(vt + (r1 * CPR + (u ^ vswz<CPR>(r1))) * 8 + half);
    return u32x4{lo.x, lo.y, hi.x, hi.y};
  };
  // Mask, online softmax and P.V of one tile whose scores are in sacc.
  auto softmax_pv = [&](int32_t t, f32x16* sacc) {
    const int buf = t % STAGES;
    const uint16_t* vt = Vs[buf];
    const int32_t key0 = t * 64;
    // V fragments of the first P.V step go into flight before the softmax arithmetic.
    u32x4 va[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) va[d] = vfrag(vt, 0, d);
    // Causal mask where the tile reaches past the wave's first position; running
    // max.  Register r of block kb holds key 32kb + 8(r/4) + 4hl + r%4.
    if (key0 + 63 > pmin) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int32_t key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key > rpos) sacc[kb][r] = -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
    mt = pair_max(mt);  // the other half of this row's keys lives 32 lanes away
    const float mn = fmaxf(m_run, mt * scale_log2);
    if (__any(mn != m_run)) {  // rescale only when some running max moved
      const float alpha = fast_exp2(m_run - mn);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
      m_run = mn;
    }
    float psum = 0.f;
    u32x4 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(fmaf(sacc[kb][r], scale_log2, -m_run));
        psum += p[r];
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        pb[2 * kb + s2].x = pack_bf16x2(p[8 * s2 + 0], p[8 * s2 + 1]);
        pb[2 * kb + s2].y = pack_bf16x2(p[8 * s2 + 2], p[8 * s2 + 3]);
        pb[2 * kb + s2].z = pack_bf16x2(p[8 * s2 + 4], p[8 * s2 + 5]);
        pb[2 * kb + s2].w = pack_bf16x2(p[8 * s2 + 6], p[8 * s2 + 7]);
      }
    }
    l_run += psum;
    // O^T += V^T P^T over the four 16-key steps; MFMA k index 8*hl + j maps to key
    // 32kb + 16s2 + 8(j/4) + 4hl + j%4, the keys this lane's P registers hold.  The next
    // step's V fragments are read while this step's MFMAs run.
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      u32x4 vn[DB];
      if (step + 1 < 4) {
#pragma unroll
        for (int d = 0; d < DB; ++d) vn[d] = vfrag(vt, step + 1, d);
      }
#pragma unroll
      for (int d = 0; d < DB; ++d)
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[d]), as_bf16x8(pb[step]),
                                                         oacc[d], 0, 0, 0);
      if (step + 1 < 4) {
#pragma unroll
        for (int d = 0; d < DB; ++d) va[d] = vn[d];
      }
    }
  };
  auto active = [&](int32_t t) { return wave_active && t < ntile && t * 64 <= pmax; };

  // Prologue: tiles 0 .. STAGES-2 in flight; QK of tile 0 once it has landed.
  int32_t ids[MAXNB];
  fetch_ids(0, ids);
#pragma unroll
  for (int j = 0; j < STAGES - 1; ++j) {
    if (j < ntile) issue_loads(j, ids, j);
    fetch_ids(j + 1, ids);
  }
  // Q^T operand: k-step s holds dims 16s + 8*hl .. +8 of this lane's row.  Loaded after
  // the first tiles so that one full wait covers both: afterwards no register load is
  // outstanding, and every vector-memory operation in the loop is a tile load whose
  // completion the loop tracks with its own vmcnt waits.
  {
    const uint16_t* qr = qkv + ((size_t)(tok0 + rtok) * (Hq + 2 * Hkv) + rhead) * D;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qb[s] = ld16(qr + 16 * s + 8 * hl);
  }
  wait_vmcnt<0>();
  __syncthreads();
  f32x16 s_cur[2], s_next[2];
  if (active(0)) qk(0, s_cur);

  for (int32_t t = 0; t < ntile; ++t) {
    // Tiles t and t+1 resident: at most the tile issued last (t + STAGES - 2) pending.
    if (t + STAGES - 2 < ntile) wait_vmcnt<LPT>();
    else wait_vmcnt<0>();
    __syncthreads();  // buffer (t - 1) % STAGES is free for tile t + STAGES - 1
    if (t + STAGES - 1 < ntile) {
      issue_loads(t + STAGES - 1, ids, (t + STAGES - 1) % STAGES);
      fetch_ids(t + STAGES, ids);
    }
    // QK of the next tile goes to the matrix cores while this tile's softmax runs.
    if (active(t + 1)) qk(t + 1, s_next);
    if (active(t)) softmax_pv(t, s_cur);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s_cur[kb] = s_next[kb];
  }

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

template <int D>
hipError_t launch_t(const rbkv_shape& s, const rbkv_batch& b, const void* qkv, const void* pool,
                    void* out, hipStream_t stream) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  const int32_t n_groups = b.n_prefill_seqs * s.n_kv_heads;
  const int32_t grid = ((n_groups + N_XCD - 1) / N_XCD) * b.prefill_qtiles_max * N_XCD;
  const int32_t qtt = q_tile_tokens(s.n_q_heads / s.n_kv_heads);
  hipLaunchKernelGGL((prefill_attn_kernel<D>), dim3(grid), dim3(PF_THREADS), 0, stream,
                     (const uint16_t*)qkv, (const uint16_t*)pool, (uint16_t*)out,
                     (const int4*)b.prefill_work, n_groups, b.prefill_qtiles_max, qtt,
                     b.cu_seqlens, b.seen, b.block_offsets,
                     b.block_ids, s.n_q_heads, s.n_kv_heads, s.n_q_heads / s.n_kv_heads,
                     s.block_size, scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const rbkv_shape& s, const rbkv_batch& b, const void* qkv,
                          const void* pool, void* out, hipStream_t stream) {
  if (s.dtype != RBKV_DTYPE_BF16) return hipErrorInvalidValue;  // float32 chunks use the VALU path
  if (s.head_dim == 128) return launch_t<128>(s, b, qkv, pool, out, stream);
  return launch_t<64>(s, b, qkv, pool, out, stream);
}

}  // namespace rbkv
