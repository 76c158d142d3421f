// Causal attention of bf16 prefill chunks on the gfx950 matrix cores.
//
// A work item is (sequence, kv head, a run of the chunk's tokens).  Its 128 query rows
// are (token, head-in-group) pairs, so every K/V tile loaded into LDS serves all G query
// heads of the kv group.  Each of the 4 wavefronts owns 32 rows and runs
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16, keys x rows, K from LDS, Q held in registers)
//   online softmax down each column (the lane owns one row: a column max is 16 register
//                 maxima plus one exchange with the partner lane 32 away),
//   O^T += V^T P^T (same instruction; P comes straight from the S^T accumulators, V from
//                 a transposed LDS copy),
// over 64-key tiles, with the causal mask applied bottom-right (query at position p sees
// keys 0..p, p = seen + offset in the chunk) and only on the tiles that need it.
//
// Pipeline: K/V tiles are double-buffered in LDS with one barrier per tile.  While a
// tile is computed, the next tile sits in registers waiting to be stored and the one
// after it is in flight from HBM; block ids are fetched one tile further ahead, so the
// id -> address -> data chain never stalls a tile.  Work items are mapped onto block
// indices so that the query tiles of one (sequence, kv head) run on the same XCD and
// share its L2.
//
// Dynamic SplitFuse chunks continuing a sequence with seen cached tokens:
// "DeepSpeed-Inference and DeepSpeed-MII", sections 10.3 and 10.10; query-tile sizing per
// head and blocked attention over work atoms: "DeepSpeed Inference v2 source tour",
// section "Ragged batches: packing a whole server into four tensors".
#include "rbkv_device.h"
#include "rbkv_internal.h"

namespace rbkv {
namespace {

constexpr int PF_THREADS = 256;
constexpr int N_XCD = 8;
constexpr int VTS = 68;  // transposed-V row stride in bf16 elements (64 keys + pad, 8-byte aligned)

template <int CPR>
__device__ __forceinline__ int kslot(int row, int c) {
  constexpr int SH = CPR >= 16 ? 0 : 1;
  const int swz = CPR >= 16 ? (row & 15) : ((row >> SH) & (CPR - 1));
  return row * CPR + (c ^ swz);
}

__device__ __forceinline__ bf16x8v as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8v, v); }

template <int D>
__global__ __launch_bounds__(PF_THREADS, 2) void prefill_attn_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ pool,
    uint16_t* __restrict__ out, const int4* __restrict__ work, int32_t n_items,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ seen_arr,
    const int32_t* __restrict__ block_off, const int32_t* __restrict__ block_ids, int32_t Hq,
    int32_t Hkv, int32_t G, int32_t bs, float scale_log2) {
  constexpr int CPR = D / 8;                // 16-byte chunks per key row
  constexpr int RPI = PF_THREADS / CPR;     // key rows covered by one pass of the WG
  constexpr int NP = 32 / RPI;              // adjacent key pairs per thread per tile
  constexpr int KSTEPS = D / 16;            // MFMA k-steps over the head dim
  constexpr int DB = D / 32;                // 32-wide dim blocks of the output
  __shared__ u32x4 Ks[2][64 * CPR];
  __shared__ uint32_t Vt[2][D * VTS / 2];

  // XCD-aware mapping: block b runs on XCD b % 8; give each XCD a contiguous run of
  // items so that the query tiles of one (sequence, kv head) share an L2.
  const int32_t per_xcd = (n_items + N_XCD - 1) / N_XCD;
  const int32_t item = (int32_t)(blockIdx.x % N_XCD) * per_xcd + (int32_t)(blockIdx.x / N_XCD);
  if (item >= n_items) return;  // whole workgroup leaves together

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hl = lane >> 5;     // half of the wave
  const int col = lane & 31;    // query row within the wave's 32

  const int4 w = work[item];
  const int32_t seq = w.x, kvh = w.y, q0 = w.z, q1 = w.w;
  const int32_t n_tok = q1 - q0;
  const int32_t rows = n_tok * G;
  const int32_t seen = seen_arr[seq];
  const int32_t tok0 = cu[seq] + q0;           // packed index of the item's first token
  const int32_t n_keys = seen + q1;            // keys visible to the last token
  const int32_t ntile = (n_keys + 63) >> 6;
  const int32_t* bids = block_ids + block_off[seq];
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

  // Loader role: pair p of this thread covers keys 2*kp and 2*kp+1 of a tile, chunk c.
  const int c_ld = tid % CPR;
  int kp_ld[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) kp_ld[p] = p * RPI + tid / CPR;

  // Block id of each pair's keys for a tile (-1 past the end of the sequence).
  auto fetch_ids = [&](int32_t t, int64_t* ids) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int32_t key = t * 64 + 2 * kp_ld[p];
      ids[p] = (t < ntile && key < n_keys) ? (int64_t)bids[key / bs] : -1;
    }
  };
  u32x4 st_k[NP][2], st_v[NP][2];  // staged tile (registers)
  auto issue_loads = [&](int32_t t, const int64_t* ids) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int32_t key = t * 64 + 2 * kp_ld[p] + j;
        st_k[p][j] = u32x4{0, 0, 0, 0};
        st_v[p][j] = u32x4{0, 0, 0, 0};
        if (ids[p] >= 0 && key < n_keys) {
          const uint16_t* src = pool_g + (size_t)(ids[p] * 2 * Hkv) * head_stride +
                                (size_t)(key % bs) * D + c_ld * 8;
          st_k[p][j] = ld16(src);
          st_v[p][j] = ld16(src + v_off);
        }
      }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int kp = kp_ld[p];
      Ks[buf][kslot<CPR>(2 * kp, c_ld)] = st_k[p][0];
      Ks[buf][kslot<CPR>(2 * kp + 1, c_ld)] = st_k[p][1];
      const u32x4 a = st_v[p][0], b = st_v[p][1];
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t lo = (j & 1) ? (aw[j >> 1] >> 16) : (aw[j >> 1] & 0xffffu);
        const uint32_t hi = (j & 1) ? (bw[j >> 1] & 0xffff0000u) : (bw[j >> 1] << 16);
        Vt[buf][((8 * c_ld + j) * VTS + 2 * kp) >> 1] = lo | hi;
      }
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Prologue: tile 0 into LDS, tile 1 in flight, ids of tile 2 in flight.
  int64_t ids_a[NP], ids_b[NP];
  fetch_ids(0, ids_a);
  fetch_ids(1, ids_b);
  issue_loads(0, ids_a);
  store_stage(0);
  issue_loads(1, ids_b);
  fetch_ids(2, ids_a);
  __syncthreads();

  for (int32_t t = 0; t < ntile; ++t) {
    const int buf = t & 1;
    const int32_t key0 = t * 64;
    if (wave_active && key0 <= pmax) {
      // S^T = K Q^T for keys key0 .. key0+63 (two 32-key blocks).
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const u32x4 a = Ks[buf][kslot<CPR>(32 * kb + col, 2 * s + hl)];
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qb[s]),
                                                            sacc[kb], 0, 0, 0);
        }
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
        const float alpha = exp2f(m_run - mn);
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
          p[r] = exp2f(fmaf(sacc[kb][r], scale_log2, -m_run));
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
      // the same keys this lane's P registers 8s2 .. 8s2+7 hold.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int kbase = 32 * kb + 16 * s2 + 4 * hl;
#pragma unroll
          for (int d = 0; d < DB; ++d) {
            const int dim = 32 * d + col;
            const uint32_t* vr = Vt[buf] + ((dim * VTS + kbase) >> 1);
            const u32x2 lo = *(const u32x2*)vr;
            const u32x2 hi = *(const u32x2*)(vr + 4);
            const u32x4 a = u32x4{lo.x, lo.y, hi.x, hi.y};
            oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a),
                                                             as_bf16x8(pb[kb][s2]), oacc[d],
                                                             0, 0, 0);
          }
        }
    }
    // Tile t+1 (staged in registers since the last iteration) into the other buffer,
    // tile t+2 into flight, ids of tile t+3 into flight.
    if (t + 1 < ntile) {
      store_stage(buf ^ 1);
      if (t + 2 < ntile) {
        issue_loads(t + 2, ids_a);
        fetch_ids(t + 3, ids_a);
      }
    }
    __syncthreads();
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
  const int32_t n = b.n_prefill_items;
  const int32_t grid = ((n + N_XCD - 1) / N_XCD) * N_XCD;
  hipLaunchKernelGGL((prefill_attn_kernel<D>), dim3(grid), dim3(PF_THREADS), 0, stream,
                     (const uint16_t*)qkv, (const uint16_t*)pool, (uint16_t*)out,
                     (const int4*)b.prefill_work, n, b.cu_seqlens, b.seen, b.block_offsets,
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
