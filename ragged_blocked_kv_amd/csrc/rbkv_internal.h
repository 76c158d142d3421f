// Internal definitions shared by the host side of librbkv and its gfx950 kernels:
// work decomposition, metadata-buffer layout and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rbkv.h"

namespace rbkv {

// Keys per decode tile: one key per lane of a 64-wide wavefront.
constexpr int KT = 64;
// Query rows (tokens x heads of one kv group) per prefill workgroup: 8 waves x 32.
constexpr int PF_ROWS = 256;
constexpr int MAX_GROUP = 16;
constexpr int MAX_SEQS_LIMIT = 2048;
constexpr int MAX_TOKENS_LIMIT = 1 << 20;
constexpr int MAX_BLOCKS_LIMIT = 1 << 26;
// Decode split-K sizing: aim for about this many decode work items per batch (one
// wavefront each), or DECODE_TARGET_ITEMS_GROUPED for the one-wave-per-head kernel
// (a workgroup each, two resident per CU; finer items trim its tail).  The lean and
// matrix-core kernels take fewer, longer items (fewer item starts; the list ends on its
// shortest items): DECODE_TARGET_ITEMS_LEAN for groups of up to four heads, _LEAN2 for
// larger groups.
constexpr int64_t DECODE_TARGET_ITEMS = 6144;
constexpr int64_t DECODE_TARGET_ITEMS_GROUPED = 12288;
constexpr int64_t DECODE_TARGET_ITEMS_LEAN = 3072;
constexpr int64_t DECODE_TARGET_ITEMS_LEAN2 = 6144;
constexpr int MIN_SPLIT_TILES = 4;
constexpr int MAX_SPLIT_TILES = 64;
// The matrix-core decode (persistent workgroups, each wave streaming its own slices) wins
// with still fewer, longer items: groups of up to four heads ~512 items, larger groups
// ~2k with splits of up to 256 tiles (measured: full-budget decode 601 -> 594 us and
// mixed launch 958 -> 943 us from 3072 items to 1024; long decode 2181 -> 2082 us from
// 6144 items capped at 64 tiles; SplitFuse mixed launch 353 -> 342 us with 1024 items,
// 333 -> 329 us with 512, the full-budget batch equal at 512 and 256).  The register-only
// kernel (single-head groups) takes the same target (MHA decode 154 -> 153 us at 1k; its
// pairs are never long enough to split at 512).
constexpr int64_t DECODE_TARGET_ITEMS_MFMA = 512;
constexpr int64_t DECODE_TARGET_ITEMS_MFMA_WIDE = 2048;
constexpr int MAX_SPLIT_TILES_MFMA = 256;

// Header of the staged batch (int32 words at the start of the staging area).
enum HeaderWord {
  H_S = 0, H_T, H_NBLK, H_SPLIT, H_HKV, H_MFMA, H_QTT, H_NDEC, H_NPRE, H_NPART, H_NCOMB,
  H_NPSEQ, HDR_INTS = 16
};

__host__ __device__ inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Single-token decodes of bf16 groups of five or more query heads that no kernel below
// takes (head dim 64 over blocks of fewer than 64 keys, or groups of 9-16 heads at head dim
// 64; groups of 5-16 over blocks of fewer than 64 keys at head dim 128) run on the
// one-wave-per-head kernel (shared LDS tiles); everything else on one wave per item.
inline bool decode_grouped(const rbkv_shape& s) {
  return s.dtype == RBKV_DTYPE_BF16 && s.n_q_heads / s.n_kv_heads > 4;
}

// Single-token decodes of bf16 groups of at most eight query heads over blocks of 64 or
// more keys: at head dim 64 the lean kernels (one K/V tile per workgroup), at head dim 128
// the register-only kernel for single-head groups (larger groups: decode_mfma_ok below).
inline bool decode_lean_ok(const rbkv_shape& s) {
  return s.dtype == RBKV_DTYPE_BF16 && s.n_q_heads / s.n_kv_heads <= 8 && s.block_size >= 64;
}

// Single-token decodes of bf16 groups of 2-16 query heads at head dim 128 over blocks of
// 64 or more keys run on the matrix-core kernel (each wave a 16-key slice of every tile).
inline bool decode_mfma_ok(const rbkv_shape& s) {
  const int32_t G = s.n_q_heads / s.n_kv_heads;
  return s.dtype == RBKV_DTYPE_BF16 && s.head_dim == 128 && s.block_size >= 64 && G >= 2 &&
         G <= MAX_GROUP;
}

// Single-token decodes of bf16 single-head groups at head dim 128 over blocks of 64 or
// more keys run on the register-only kernel.
inline bool decode_reg_ok(const rbkv_shape& s) {
  return s.dtype == RBKV_DTYPE_BF16 && s.head_dim == 128 && s.block_size >= 64 &&
         s.n_q_heads == s.n_kv_heads;
}

// Shapes whose decodes can run as persistent workgroups draining the decode list through
// a device counter (launch_decode_persistent).
inline bool decode_persistent_ok(const rbkv_shape& s) {
  return decode_lean_ok(s) || decode_mfma_ok(s);
}

// Tokens of one sequence per prefill workgroup: as many as fit PF_ROWS rows of G heads.
__host__ __device__ inline int32_t q_tile_tokens(int32_t G) {
  int32_t q = PF_ROWS / G;
  return q < 1 ? 1 : q;
}

struct SeqPlan {
  int32_t dec_items;   // decode work items (token, kv head, split)
  int32_t pre_items;   // prefill work items (q tile, kv head)
  int32_t partials;    // split-K partial slots
  int32_t comb_items;  // combine items (token, kv head)
  int32_t nsplit;      // splits per (token, kv head) for a single-token decode
};

// Work decomposition of one sequence.  Single-token decodes stream their keys in
// splits of split_tiles 64-key tiles; chunks of several tokens either go to MFMA
// tiles (bf16) or become one vector-ALU item per token and kv head (float32).
__host__ __device__ inline SeqPlan plan_sequence(int32_t n, int32_t seen, int32_t Hkv,
                                                 int32_t split_tiles, bool mfma_prefill,
                                                 int32_t qtt) {
  SeqPlan p{0, 0, 0, 0, 1};
  if (n == 1) {
    int32_t tiles = (int32_t)cdiv64((int64_t)seen + 1, KT);
    int32_t ns = (int32_t)cdiv64(tiles, split_tiles);
    p.nsplit = ns;
    p.dec_items = Hkv * ns;
    if (ns > 1) {
      p.partials = Hkv * ns;
      p.comb_items = Hkv;
    }
  } else if (mfma_prefill) {
    p.pre_items = Hkv * (int32_t)cdiv64(n, qtt);
  } else {
    p.dec_items = Hkv * n;
  }
  return p;
}

// Work proxy used to order chunk sequences longest first on the matrix cores: query
// tiles times the keys an average tile sees (monotone in the 64-key tiles it streams).
__host__ __device__ inline int64_t prefill_work_proxy(int32_t n, int32_t seen, int32_t qtt) {
  return cdiv64(n, qtt) * (2 * (int64_t)seen + n);
}

// Capacities of the work lists for a shape (upper bounds over every valid batch).
struct Caps {
  int64_t dec, pre, comb;
};
inline Caps work_caps(const rbkv_shape& s) {
  Caps c;
  const int64_t tiles = cdiv64((int64_t)s.num_blocks * s.block_size, KT) + s.max_seqs;
  c.dec = (int64_t)s.n_kv_heads * (tiles + s.max_tokens);
  c.pre = (int64_t)s.n_kv_heads * (s.max_tokens + s.max_seqs);
  c.comb = (int64_t)s.n_kv_heads * s.max_seqs;
  return c;
}

// Device metadata buffer layout (byte offsets, each 256-byte aligned).  The staging
// region (header, n_new, seen, flat block ids) is the image of the pinned host buffer.
struct MetaLayout {
  size_t staging, n_new, seen, block_ids, staging_bytes;
  size_t cu, kv_len, block_off, tok2seq, pos, dec, pre, comb, total;
};
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline MetaLayout meta_layout(const rbkv_shape& s) {
  MetaLayout L;
  size_t at = 0;
  L.staging = 0;
  L.n_new = HDR_INTS * 4;
  L.seen = L.n_new + (size_t)s.max_seqs * 4;
  L.block_ids = L.seen + (size_t)s.max_seqs * 4;
  L.staging_bytes = L.block_ids + (size_t)s.num_blocks * 4;
  at = align256(L.staging_bytes);
  Caps c = work_caps(s);
  L.cu = at;        at = align256(at + (size_t)(s.max_seqs + 1) * 4);
  L.kv_len = at;    at = align256(at + (size_t)s.max_seqs * 4);
  L.block_off = at; at = align256(at + (size_t)(s.max_seqs + 1) * 4);
  L.tok2seq = at;   at = align256(at + (size_t)s.max_tokens * 4);
  L.pos = at;       at = align256(at + (size_t)s.max_tokens * 4);
  L.dec = at;       at = align256(at + (size_t)c.dec * 16);
  L.pre = at;       at = align256(at + (size_t)c.pre * 16);
  L.comb = at;      at = align256(at + (size_t)c.comb * 16);
  L.total = at;
  return L;
}

// Floats per split-K partial slot: m[G], l[G], acc[G][d].
inline size_t partial_floats(int32_t G, int32_t d) { return (size_t)G * (d + 2); }

// ---- kernel launchers (defined in the .hip files) ----

hipError_t launch_meta_build(const int32_t* staging, int32_t* cu, int32_t* kv_len,
                             int32_t* block_off, int32_t* tok2seq, int32_t* pos,
                             int32_t* dec, int32_t* pre, int32_t* comb, int32_t block_size,
                             int32_t max_seqs, int32_t S, hipStream_t stream);

hipError_t launch_append_rotary(const rbkv_shape& s, const rbkv_batch& b, void* qkv,
                                void* pool, double rope_base, hipStream_t stream);

hipError_t launch_decode(const rbkv_shape& s, const rbkv_batch& b, const void* qkv,
                         const void* pool, void* out, float* ws, hipStream_t stream);

// The decode as persistent workgroups draining the decode list through a device counter
// (decode_persistent_ok shapes only); the counter must be zero when the first of the
// launches sharing it starts (launch_claims_reset).  stages: tile stages per wave
// of the matrix-core kernel (3, or 2 for anything less); the other kernels have one form.
hipError_t launch_decode_persistent(const rbkv_shape& s, const rbkv_batch& b, const void* qkv,
                                    const void* pool, void* out, float* ws, int32_t* claim,
                                    int32_t workgroups, hipStream_t stream, int stages);

hipError_t launch_prefill(const rbkv_shape& s, const rbkv_batch& b, const void* qkv,
                          const void* pool, void* out, hipStream_t stream);

// Prefill and decode items of a mixed batch in one launch of `workgroups` persistent
// workgroups (decode_mfma_ok shapes; one workgroup fits a CU), dec_first of every XCD's
// starting on the decode list; claims[0..8] zero at launch (launch_claims_reset).
hipError_t launch_mixed(const rbkv_shape& s, const rbkv_batch& b, const void* qkv,
                        const void* pool, void* out, float* ws, int32_t* claims,
                        int32_t workgroups, int32_t dec_first, hipStream_t stream);
// Zeroes n (<= 64) item counters.
hipError_t launch_claims_reset(int32_t* claims, int n, hipStream_t stream);

hipError_t launch_combine(const rbkv_shape& s, const rbkv_batch& b, const float* ws,
                          void* out, hipStream_t stream);

// Address of the library's static scratch array (RBKV_STATIC_SCRATCH_BYTES) on the current
// device, resolved once per device (static_scratch.hip).
hipError_t static_scratch(void** ptr);

// Row gather: mode 0 takes source row idx[r] (zero row outside [0, n_src)), mode 1 takes
// idx[r + 1] - 1.  row_bytes is a multiple of 16; rows * row_bytes / 16 < 2^31.
hipError_t launch_gather_rows(int mode, const void* src, void* dst, const int32_t* idx,
                              int32_t n_src, int32_t rows, size_t row_bytes,
                              hipStream_t stream);

// Copies n pool blocks of block_bytes each between the pool and a host buffer mapped at
// host_dev (dir 0: pool -> host, dir 1: host -> pool); ids_dev is the device view of the
// staged block ids.  n * ceil(block_bytes / 16 KiB) * 256 < 2^32.
hipError_t launch_kv_block_copy(int dir, void* pool, void* host_dev, const int32_t* ids_dev,
                                int32_t n, size_t block_bytes, hipStream_t stream);

}  // namespace rbkv
