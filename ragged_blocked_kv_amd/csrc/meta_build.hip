// Device metadata of one ragged batch, built by a single 1024-thread workgroup from the
// staged per-sequence counts: cu_seqlens, kv_len, block_offsets, per-token owner and
// absolute position, and the three attention work lists.  ("DeepSpeed Inference v2
// source tour", section "Ragged batches: packing a whole server into four tensors":
// token start/stop offsets, a tokens-to-sequence map and per-sequence block tables.)
#include "rbkv_internal.h"

namespace rbkv {
namespace {

constexpr int MB_THREADS = 1024;
constexpr int N_SCANS = 6;  // n_new, blocks, decode items, prefill items, partials, combines

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

// Largest i in [0, S) with off[i] <= x (off ascending, off[0] = 0 <= x).
__device__ int upper_index(const int32_t* off, int S, int32_t x) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
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

  const int tid = threadIdx.x;
  const int32_t S = staging[H_S];
  const int32_t T = staging[H_T];
  const int32_t split = staging[H_SPLIT];
  const int32_t Hkv = staging[H_HKV];
  const bool mfma = staging[H_MFMA] != 0;
  const int32_t qtt = staging[H_QTT];
  const int32_t n_dec = staging[H_NDEC];
  const int32_t n_comb = staging[H_NCOMB];
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
  const int32_t* s_pre = offs[3];
  const int32_t* s_part = offs[4];
  const int32_t* s_comb = offs[5];

  for (int i = tid; i <= S; i += MB_THREADS) {
    cu[i] = s_cu[i];
    block_off[i] = s_bo[i];
    if (i < S) kv_len[i] = s_seen[i] + vals[0][i];
  }
  for (int t = tid; t < T; t += MB_THREADS) {
    const int i = upper_index(s_cu, S, t);
    tok2seq[t] = i;
    pos[t] = s_seen[i] + (t - s_cu[i]);
  }
  for (int w = tid; w < n_dec; w += MB_THREADS) {
    const int i = upper_index(s_dec, S, w);
    const int32_t local = w - s_dec[i];
    const int32_t n = vals[0][i];
    int4 r;
    if (n == 1) {
      const int32_t ns = s_nsplit[i];
      r.x = s_cu[i];
      r.y = local / ns;
      r.z = local % ns;
      r.w = ns > 1 ? s_part[i] + local : -1;
    } else {  // one vector-ALU item per token of a float32 chunk, never split
      r.x = s_cu[i] + local % n;
      r.y = local / n;
      r.z = 0;
      r.w = -1;
    }
    dec[w] = r;
  }
  // Chunk sequences ranked by work, longest first (ties by batch order): the prefill
  // kernel deals their (sequence, kv head) groups round-robin over the XCDs.
  for (int i = tid; i < S; i += MB_THREADS) {
    const long long wi = s_pwork[i];
    if (wi < 0) continue;
    int32_t rank = 0;
    for (int j = 0; j < S; ++j) {
      const long long wj = s_pwork[j];
      rank += (wj > wi || (wj == wi && j < i)) ? 1 : 0;
    }
    int4 r;
    r.x = i;
    r.y = (int32_t)cdiv64(vals[0][i], qtt);
    r.z = 0;
    r.w = 0;
    pre[rank] = r;
  }
  for (int w = tid; w < n_comb; w += MB_THREADS) {
    const int i = upper_index(s_comb, S, w);
    const int32_t kvh = w - s_comb[i];
    const int32_t ns = s_nsplit[i];
    int4 r;
    r.x = s_cu[i];
    r.y = kvh;
    r.z = s_part[i] + kvh * ns;
    r.w = ns;
    comb[w] = r;
  }
}

}  // namespace

hipError_t launch_meta_build(const int32_t* staging, int32_t* cu, int32_t* kv_len,
                             int32_t* block_off, int32_t* tok2seq, int32_t* pos,
                             int32_t* dec, int32_t* pre, int32_t* comb, int32_t block_size,
                             int32_t max_seqs, hipStream_t stream) {
  hipLaunchKernelGGL(meta_build_kernel, dim3(1), dim3(MB_THREADS), 0, stream, staging, cu,
                     kv_len, block_off, tok2seq, pos, (int4*)dec, (int4*)pre, (int4*)comb,
                     block_size, max_seqs);
  return hipGetLastError();
}

}  // namespace rbkv
