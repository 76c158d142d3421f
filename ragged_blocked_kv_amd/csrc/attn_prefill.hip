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

// HBM -> LDS without registers: lane l writes its 16 bytes at dst + 16*l (dst must be
// wave-uniform).  Kept in a device function: used directly in a kernel template, the
// builtin makes the host pass drop that kernel's launch stub.
__device__ __forceinline__ void load_lds16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

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

  // Q^T operand: k-step s holds dims 16s + 8*hl .. +8 of this lane's row.
  u32x4 qb[KSTEPS];
  {
    const uint16_t* qr = qkv + ((size_t)(tok0 + rtok) * (Hq + 2 * Hkv) + rhead) * D;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qb[s] = ld16(qr + 16 * s + 8 * hl);
  }

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
  auto issue_loads = [&](int32_t t, const int32_t* ids, int buf) {
    if (bs >= 64 && t * 64 + 63 < n_keys) {
      // The whole tile sits in one block: one uniform base, fixed per-thread offsets.
      const uint16_t* base = pool_g + (size_t)ids[0] * blk_stride + (size_t)((t * 64) % bs) * D;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const uint16_t* src = base + krow[i] * D;
        load_lds16(src + kchk[i] * 8, Ks[buf] + (i * PF_THREADS + wave * 64) * 8);
        load_lds16(src + v_off + vchk[i] * 8, Vs[buf] + (i * PF_THREADS + wave * 64) * 8);
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
      load_lds16(src + kchk[i] * 8, Ks[buf] + (i * PF_THREADS + wave * 64) * 8);
      load_lds16(src + v_off + vchk[i] * 8, Vs[buf] + (i * PF_THREADS + wave * 64) * 8);
    }
  };

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

  // Prologue: tiles 0 .. STAGES-2 in flight, ids of tile STAGES-1 fetched.
  int32_t ids[MAXNB];
  fetch_ids(0, ids);
#pragma unroll
  for (int j = 0; j < STAGES - 1; ++j) {
    if (j < ntile) issue_loads(j, ids, j);
    fetch_ids(j + 1, ids);
  }

  for (int32_t t = 0; t < ntile; ++t) {
    const int buf = t % STAGES;
    // Tile t has landed once at most (tiles issued after it) * LPT loads are pending.
    const int32_t later = min(STAGES - 2, ntile - 1 - t);
    if (later >= 2) wait_vmcnt<2 * LPT>();
    else if (later == 1) wait_vmcnt<LPT>();
    else wait_vmcnt<0>();
    __syncthreads();  // everyone's part of tile t is in; buffer (t - 1) % STAGES is free
    if (t + STAGES - 1 < ntile) {
      issue_loads(t + STAGES - 1, ids, (t + STAGES - 1) % STAGES);
      fetch_ids(t + STAGES, ids);
    }
    const int32_t key0 = t * 64;
    if (!wave_active || key0 > pmax) continue;  // nothing of this tile is visible
    // S^T = K Q^T for keys key0 .. key0+63 (two 32-key blocks, their accumulation
    // chains interleaved so consecutive MFMAs are independent).
    f32x16 sacc[2];
    {
      u32x4 a[2][KSTEPS];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int krow_r = 32 * kb + col;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
          a[kb][s] = *(const u32x4*)(Ks[buf] +
                                     (krow_r * CPR + ((2 * s + hl) ^ kswz<CPR>(krow_r))) * 8);
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
      }
      __builtin_amdgcn_s_setprio(1);  // let the other wave's softmax fill the MFMA shadow
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[kb][s]),
                                                            as_bf16x8(qb[s]), sacc[kb], 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
    }
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
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
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
    u32x4 pb[2][2];
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
        pb[kb][s2].x = pack_bf16x2(p[8 * s2 + 0], p[8 * s2 + 1]);
        pb[kb][s2].y = pack_bf16x2(p[8 * s2 + 2], p[8 * s2 + 3]);
        pb[kb][s2].z = pack_bf16x2(p[8 * s2 + 4], p[8 * s2 + 5]);
        pb[kb][s2].w = pack_bf16x2(p[8 * s2 + 6], p[8 * s2 + 7]);
      }
    }
    l_run += psum;

    // O^T += V^T P^T.  MFMA k index 8*hl + j maps to key 32kb + 16s2 + 8(j/4) + 4hl + j%4,
    // the same keys this lane's P registers 8s2 .. 8s2+7 hold; the two transposing reads
    // fetch those keys (kbase + 4hl + 0..3 and kbase + 8 + 4hl + 0..3) at dim 32d + col.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int kbase = 32 * kb + 16 * s2;
        const int r0 = kbase + vkey_in, r1 = r0 + 8;
        u32x4 a[DB];
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          const int dim = 32 * d + vdim_in;
          const int u = dim >> 3, half = dim & 7;
          const u32x2 lo = ds_read_tr(Vs[buf] + (r0 * CPR + (u ^ vswz<CPR>(r0))) * 8 + half);
          const u32x2 hi = ds_read_tr(Vs[buf] + (r1 * CPR + (u ^ vswz<CPR>(r1))) * 8 + half);
          a[d] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int d = 0; d < DB; ++d)
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[d]),
                                                           as_bf16x8(pb[kb][s2]), oacc[d],
                                                           0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
      }
  }

  if (!row_valid) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
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
  static_assert(STAGES - 2 <= 2, "wait_vmcnt cases cover up to two later tiles");
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
