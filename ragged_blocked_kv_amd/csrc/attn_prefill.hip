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
// Dynamic SplitFuse chunks continuing a sequence with seen cached tokens:
// "DeepSpeed-Inference and DeepSpeed-MII", sections 10.3 and 10.10; query-tile sizing per
// head and blocked attention over work atoms: "DeepSpeed Inference v2 source tour",
// section "Ragged batches: packing a whole server into four tensors".
#include "rbkv_device.h"
#include "rbkv_internal.h"

namespace rbkv {
namespace {

constexpr int PF_THREADS = 256;
constexpr int VTS = 68;  // transposed-V row stride in bf16 elements (64 keys + pad, 8-byte aligned)

template <int CPR>
__device__ __forceinline__ int kslot(int row, int c) {
  constexpr int SH = CPR >= 16 ? 0 : 1;
  const int swz = CPR >= 16 ? (row & 15) : ((row >> SH) & (CPR - 1));
  return row * CPR + (c ^ swz);
}

__device__ __forceinline__ bf16x8v as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8v, v); }

template <int D>
__global__ __launch_bounds__(PF_THREADS) void prefill_attn_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ pool,
    uint16_t* __restrict__ out, const int4* __restrict__ work, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ seen_arr, const int32_t* __restrict__ block_off,
    const int32_t* __restrict__ block_ids, int32_t Hq, int32_t Hkv, int32_t G, int32_t bs,
    float scale_log2) {
  constexpr int CPR = D / 8;           // 16-byte chunks per key row
  constexpr int NKI = CPR / 4;         // K load instructions per thread per tile
  constexpr int NVP = CPR / 8;         // V key-pair loads per thread per tile
  constexpr int KSTEPS = D / 16;       // MFMA k-steps over the head dim
  constexpr int DB = D / 32;           // 32-wide dim blocks of the output
  __shared__ u32x4 Ks[64 * CPR];
  __shared__ uint32_t Vt[D * VTS / 2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hl = lane >> 5;     // half of the wave
  const int col = lane & 31;    // query row within the wave's 32

  const int4 w = work[blockIdx.x];
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

  f32x16 oacc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Global -> register staging of one 64-key tile.
  u32x4 kreg[NKI], vreg[NVP][2];
  auto load_tile = [&](int32_t t) {
    const int32_t key0 = t * 64;
#pragma unroll
    for (int i = 0; i < NKI; ++i) {
      const int id = i * PF_THREADS + tid;
      const int32_t key = key0 + id / CPR;
      kreg[i] = u32x4{0, 0, 0, 0};
      if (key < n_keys) {
        const int64_t blk = bids[key / bs];
        kreg[i] = ld16(pool + (size_t)(blk * 2 * Hkv + kvh) * head_stride +
                       (size_t)(key % bs) * D + (id % CPR) * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < NVP; ++i) {
      const int kp = i * (PF_THREADS / CPR) + tid / CPR;  // key pair within the tile
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int32_t key = key0 + 2 * kp + j;
        vreg[i][j] = u32x4{0, 0, 0, 0};
        if (key < n_keys) {
          const int64_t blk = bids[key / bs];
          vreg[i][j] = ld16(pool + (size_t)(blk * 2 * Hkv + kvh) * head_stride + v_off +
                            (size_t)(key % bs) * D + (tid % CPR) * 8);
        }
      }
    }
  };

  load_tile(0);
  for (int32_t t = 0; t < ntile; ++t) {
    __syncthreads();  // every wave is done reading the previous tile
#pragma unroll
    for (int i = 0; i < NKI; ++i) {
      const int id = i * PF_THREADS + tid;
      Ks[kslot<CPR>(id / CPR, id % CPR)] = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < NVP; ++i) {
      const int kp = i * (PF_THREADS / CPR) + tid / CPR;
      const int c = tid % CPR;
      const u32x4 a = vreg[i][0], b = vreg[i][1];
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t lo = (j & 1) ? (aw[j >> 1] >> 16) : (aw[j >> 1] & 0xffffu);
        const uint32_t hi = (j & 1) ? (bw[j >> 1] & 0xffff0000u) : (bw[j >> 1] << 16);
        Vt[((8 * c + j) * VTS + 2 * kp) >> 1] = lo | hi;
      }
    }
    __syncthreads();
    if (t + 1 < ntile) load_tile(t + 1);

    const int32_t key0 = t * 64;
    if (!wave_active || key0 > pmax) continue;  // nothing of this tile is visible

    // S^T = K Q^T for keys key0 .. key0+63 (two 32-key blocks).
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const u32x4 a = Ks[kslot<CPR>(32 * kb + col, 2 * s + hl)];
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qb[s]),
                                                          sacc[kb], 0, 0, 0);
      }
    }
    // Scale, causal mask (only where the tile reaches past the wave's first position),
    // running max.  Register r of block kb holds key 32kb + 8(r/4) + 4hl + r%4.
    const bool need_mask = key0 + 63 > pmin;
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = sacc[kb][r] * scale_log2;
        if (need_mask) {
          const int32_t key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
          v = key <= rpos ? v : -INFINITY;
        }
        sacc[kb][r] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mn = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - mn);
    m_run = mn;
    float psum = 0.f;
    u32x4 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = exp2f(sacc[kb][r] - mn);
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
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;

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
          const uint32_t* vr = Vt + ((dim * VTS + kbase) >> 1);
          const u32x2 lo = *(const u32x2*)vr;
          const u32x2 hi = *(const u32x2*)(vr + 4);
          const u32x4 a = u32x4{lo.x, lo.y, hi.x, hi.y};
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pb[kb][s2]),
                                                           oacc[d], 0, 0, 0);
        }
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
  hipLaunchKernelGGL((prefill_attn_kernel<D>), dim3(b.n_prefill_items), dim3(PF_THREADS), 0,
                     stream, (const uint16_t*)qkv, (const uint16_t*)pool, (uint16_t*)out,
                     (const int4*)b.prefill_work, b.cu_seqlens, b.seen, b.block_offsets,
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
