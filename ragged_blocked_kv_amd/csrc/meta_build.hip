// Device metadata of one ragged batch, built from the staged per-sequence counts:
// cu_seqlens, kv_len, block_offsets, per-token owner and absolute position, and the three
// attention work lists (decode items with every whole split ahead of the shorter ones).  Every 1024-thread workgroup plans all sequences and scans the
// counts itself (a few microseconds, cheaper than a second launch or a grid-wide wait),
// then writes the records of its own share of the sequences.  ("DeepSpeed Inference v2
// source tour", section "Ragged batches: packing a whole server into four tensors":
// token start/stop offsets, a tokens-to-sequence map and per-sequence block tables.)
#include "rbkv_internal.h"

namespace rbkv {
namespace {

constexpr int MB_THREADS = 1024;
// n_new, blocks, decode items, prefill items, partials, combines, short decode items
constexpr int N_SCANS = 7;

// Exclusive prefix sum of vals[0..S) into out[0..S] (out[S] = total) by one wavefront:
// each lane sums a contiguous run, the 64 run totals are scanned across the wave, then
// each lane writes its run.
__device__ void wave_exclusive_scan(const int32_t* vals, int32_t* out, int S, int lane) {
  const int per = (S + 63) / 64;
  const int b = lane * per;
  const int e = min(S, b + per);
  int32_t sum = 0;
  for (int i = b; i < e; ++i) sum += vals[i];
  int32_t incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int32_t v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  int32_t run = incl - sum;
  for (int i = b; i < e; ++i) {
    out[i] = run;
    run += vals[i];
  }
  if (lane == 63) out[S] = incl;
}

__global__ __launch_bounds__(MB_THREADS) void meta_build_kernel(
    const int32_t* __restrict__ staging, int32_t* __restrict__ cu, int32_t* __restrict__ kv_len,
    int32_t* __restrict__ block_off, int32_t* __restrict__ tok2seq, int32_t* __restrict__ pos,
    int4* __restrict__ dec, int4* __restrict__ pre, int4* __restrict__ comb, int32_t block_size,
    int32_t max_seqs) {
  __shared__ int32_t vals[N_SCANS][MAX_SEQS_LIMIT];
  __shared__ int32_t offs[N_SCANS][MAX_SEQS_LIMIT + 1];
  __shared__ int32_t s_seen[MAX_SEQS_LIMIT];
  __shared__ int32_t s_nsplit[MAX_SEQS_LIMIT];
  __shared__ long long s_pwork[MAX_SEQS_LIMIT];  // chunk work proxy, -1 if not a chunk
  __shared__ int32_t s_rem[MAX_SEQS_LIMIT];      // tiles of a short decode item, -1 if none

  const int tid = threadIdx.x;
  const int32_t S = staging[H_S];
  const int32_t split = staging[H_SPLIT];
  const int32_t Hkv = staging[H_HKV];
  const bool mfma = staging[H_MFMA] != 0;
  const int32_t qtt = staging[H_QTT];
  const int32_t* n_new = staging + HDR_INTS;
  const int32_t* seen = n_new + max_seqs;

  for (int i = tid; i < S; i += MB_THREADS) {
    const int32_t n = n_new[i], s = seen[i];
    const SeqPlan p = plan_sequence(n, s, Hkv, split, mfma, qtt);
    vals[0][i] = n;
    vals[1][i] = (int32_t)cdiv64((int64_t)s + n, block_size);
    vals[2][i] = p.dec_items;
    vals[3][i] = p.pre_items;
    vals[4][i] = p.partials;
    vals[5][i] = p.comb_items;
    // A decode sequence's items shorter than a whole split: its last split when that is
    // partial (which is the whole sequence when it has one split).
    const int32_t rem = (int32_t)cdiv64((int64_t)s + 1, KT) - (p.nsplit - 1) * split;
    const bool has_short = n == 1 && rem < split;
    vals[6][i] = has_short ? Hkv : 0;
    s_rem[i] = has_short ? rem : -1;
    s_seen[i] = s;
    s_nsplit[i] = p.nsplit;
    s_pwork[i] = p.pre_items > 0 ? (long long)prefill_work_proxy(n, s, qtt) : -1;
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  if (wave < N_SCANS) wave_exclusive_scan(vals[wave], offs[wave], S, lane);
  __syncthreads();

  const int32_t* s_cu = offs[0];
  const int32_t* s_bo = offs[1];
  const int32_t* s_dec = offs[2];
  const int32_t* s_part = offs[4];
  const int32_t* s_comb = offs[5];
  const int32_t* s_short = offs[6];
  // Decode items: every whole split first, in sequence order, then the shorter items,
  // longest first (ties by sequence), so that workgroups taking items in list order (one
  // per item, or persistent ones from a counter) end on the shortest ones and finish
  // together.  Partial slots do not move.
  const int32_t full_total = s_dec[S] - s_short[S];

  for (int i = blockIdx.x * MB_THREADS + tid; i <= S; i += gridDim.x * MB_THREADS) {
    cu[i] = s_cu[i];
    block_off[i] = s_bo[i];
    if (i < S) kv_len[i] = s_seen[i] + vals[0][i];
  }
  // Per-token and per-item records.  Global wavefront w (of GW) takes sequences w, w + GW,
  // w + 2 GW, ...; lane k first reads everything about the wavefront's k-th sequence from
  // LDS in one go, then the wavefront walks its sequences with those values broadcast from
  // their lane and its lanes write each sequence's consecutive entries, so no entry has to
  // search for its sequence.
  constexpr int N_WAVES = MB_THREADS / 64;
  const int GW = gridDim.x * N_WAVES;
  for (int i0 = blockIdx.x * N_WAVES + wave; i0 < S; i0 += GW * 64) {
    const int il = i0 + GW * lane;
    const bool have = il < S;
    const int32_t l_n = have ? vals[0][il] : 0, l_base = have ? s_cu[il] : 0;
    const int32_t l_seen = have ? s_seen[il] : 0, l_nd = have ? vals[2][il] : 0;
    const int32_t l_dbase = have ? s_dec[il] : 0, l_nc = have ? vals[5][il] : 0;
    const int32_t l_cbase = have ? s_comb[il] : 0, l_ns = have ? s_nsplit[il] : 1;
    const int32_t l_part = have ? s_part[il] : 0;
    const int32_t l_sbase = have ? s_short[il] : 0, l_nsh = have ? vals[6][il] : 0;
    const long long l_work = have ? s_pwork[il] : -1;
    const int count = min(64, (S - i0 + GW - 1) / GW);
    for (int k = 0; k < count; ++k) {
      const int i = i0 + GW * k;
      const int32_t n = __builtin_amdgcn_readlane(l_n, k);
      const int32_t base = __builtin_amdgcn_readlane(l_base, k);
      const int32_t sn = __builtin_amdgcn_readlane(l_seen, k);
      for (int t = lane; t < n; t += 64) {
        tok2seq[base + t] = i;
        pos[base + t] = sn + t;
      }
      const int32_t nd = __builtin_amdgcn_readlane(l_nd, k);
      const int32_t dbase = __builtin_amdgcn_readlane(l_dbase, k);
      const int32_t ns = __builtin_amdgcn_readlane(l_ns, k);
      const int32_t part = __builtin_amdgcn_readlane(l_part, k);
      if (n == 1) {
        const int32_t sbase = __builtin_amdgcn_readlane(l_sbase, k);
        const int32_t hs = __builtin_amdgcn_readlane(l_nsh, k) > 0 ? 1 : 0;
        const int32_t nfull = ns - hs;  // whole splits per kv head
        // Rank of this sequence's short items among all short items: a ballot count of
        // the sequences ranked ahead (more tiles, or as many and earlier).
        int32_t srank = 0;
        if (hs) {
          const int32_t ri = s_rem[i];
          for (int j0 = 0; j0 < S; j0 += 64) {
            const int j = j0 + lane;
            const int32_t rj = j < S ? s_rem[j] : -1;
            srank += __popcll(__ballot(rj > ri || (rj == ri && j < i)));
          }
        }
        for (int local = lane; local < nd; local += 64) {
          int4 r;
          const int32_t kvh = local / ns, sp = local % ns;
          r.x = base;
          r.y = kvh;
          r.z = sp;
          r.w = ns > 1 ? part + local : -1;
          const int32_t at = (hs && sp == ns - 1) ? full_total + srank * Hkv + kvh
                                                   : dbase - sbase + kvh * nfull + sp;
          dec[at] = r;
        }
      } else {  // one vector-ALU item per token of a float32 chunk, never split
        const int32_t sbase = __builtin_amdgcn_readlane(l_sbase, k);
        for (int local = lane; local < nd; local += 64) {
          int4 r;
          r.x = base + local % n;
          r.y = local / n;
          r.z = 0;
          r.w = -1;
          dec[dbase - sbase + local] = r;
        }
      }
      const int32_t nc = __builtin_amdgcn_readlane(l_nc, k);
      const int32_t cbase = __builtin_amdgcn_readlane(l_cbase, k);
      for (int kvh = lane; kvh < nc; kvh += 64) {
        int4 r;
        r.x = base;
        r.y = kvh;
        r.z = part + kvh * ns;
        r.w = ns;
        comb[cbase + kvh] = r;
      }
      // Chunk sequences ranked by work, longest first (ties by batch order): the prefill
      // kernel deals their (sequence, kv head) groups round-robin over the XCDs.  Each
      // lane tests one sequence per step; a ballot counts those ranked ahead.
      const long long wi = (long long)(
          (unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(l_work >> 32), k) << 32 |
          (uint32_t)__builtin_amdgcn_readlane((int)l_work, k));
      if (wi >= 0) {
        int32_t ahead = 0;
        for (int j0 = 0; j0 < S; j0 += 64) {
          const int j = j0 + lane;
          const long long wj = j < S ? s_pwork[j] : -1;
          ahead += __popcll(__ballot(wj > wi || (wj == wi && j < i)));
        }
        if (lane == 0) {
          int4 r;
          r.x = i;
          r.y = (int32_t)cdiv64(n, qtt);
          r.z = 0;
          r.w = 0;
          pre[ahead] = r;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_meta_build(const int32_t* staging, int32_t* cu, int32_t* kv_len,
                             int32_t* block_off, int32_t* tok2seq, int32_t* pos,
                             int32_t* dec, int32_t* pre, int32_t* comb, int32_t block_size,
                             int32_t max_seqs, int32_t S, hipStream_t stream) {
  // About one sequence per wavefront: each wavefront's walk is then a short chain.
  const int groups = (int)std::min<int64_t>(std::max<int64_t>(cdiv64(S, 16), 1), 128);
  hipLaunchKernelGGL(meta_build_kernel, dim3(groups), dim3(MB_THREADS), 0, stream, staging, cu,
                     kv_len, block_off, tok2seq, pos, (int4*)dec, (int4*)pre, (int4*)comb,
                     block_size, max_seqs);
  return hipGetLastError();
}

}  // namespace rbkv
