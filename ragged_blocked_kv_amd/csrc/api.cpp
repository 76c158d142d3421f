// Host side of librbkv: argument validation, batch planning, staging and launches.
// Every check runs before any HIP call, so each error path is testable without a GPU.
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "rbkv_internal.h"

using namespace rbkv;

namespace {

bool shape_supported(const rbkv_shape& s, rbkv_status* st) {
  if (s.max_tokens < 1 || s.max_seqs < 1 || s.num_blocks < 1 || s.n_q_heads < 1 ||
      s.n_kv_heads < 1 || s.block_size < 1 || s.head_dim < 1) {
    *st = RBKV_ERR_INVALID_ARG;
    return false;
  }
  const bool ok_d = s.head_dim == 64 || s.head_dim == 128;
  const bool ok_bs = s.block_size == 16 || s.block_size == 32 || s.block_size == 64 ||
                     s.block_size == 128;
  const bool ok_dt = s.dtype == RBKV_DTYPE_F32 || s.dtype == RBKV_DTYPE_BF16;
  const bool ok_g = s.n_q_heads % s.n_kv_heads == 0 &&
                    s.n_q_heads / s.n_kv_heads <= MAX_GROUP;
  const bool ok_lim = s.max_seqs <= MAX_SEQS_LIMIT && s.max_tokens <= MAX_TOKENS_LIMIT &&
                      s.num_blocks <= MAX_BLOCKS_LIMIT && s.n_q_heads <= 1024;
  if (!(ok_d && ok_bs && ok_dt && ok_g && ok_lim)) {
    *st = RBKV_ERR_UNSUPPORTED;
    return false;
  }
  return true;
}

rbkv_status check_shape(const rbkv_shape* s) {
  if (!s) return RBKV_ERR_INVALID_ARG;
  rbkv_status st = RBKV_OK;
  return shape_supported(*s, &st) ? RBKV_OK : st;
}

size_t elem_bytes(const rbkv_shape& s) { return s.dtype == RBKV_DTYPE_F32 ? 4 : 2; }

// A device buffer must be device (or managed) memory of the current device, and its
// allocation must extend at least `bytes` past `p`.
rbkv_status check_device(const void* p, size_t bytes) {
  if (!p) return RBKV_ERR_INVALID_ARG;
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return RBKV_ERR_DEVICE_PTR;
  }
  if (a.type != hipMemoryTypeDevice && a.type != hipMemoryTypeManaged)
    return RBKV_ERR_DEVICE_PTR;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return RBKV_ERR_HIP;
  if (a.device != dev) return RBKV_ERR_DEVICE_PTR;
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p) != hipSuccess) {
    (void)hipGetLastError();
    return RBKV_ERR_DEVICE_PTR;
  }
  if ((const char*)p + bytes > (const char*)base + size) return RBKV_ERR_DEVICE_PTR;
  return RBKV_OK;
}

rbkv_status check_pinned(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return RBKV_ERR_DEVICE_PTR;
  }
  return a.type == hipMemoryTypeHost ? RBKV_OK : RBKV_ERR_DEVICE_PTR;
}

rbkv_status launch_build(const rbkv_shape& s, char* dm, int32_t S, hipStream_t stream) {
  const MetaLayout L = meta_layout(s);
  if (launch_meta_build((const int32_t*)dm, (int32_t*)(dm + L.cu), (int32_t*)(dm + L.kv_len),
                        (int32_t*)(dm + L.block_off), (int32_t*)(dm + L.tok2seq),
                        (int32_t*)(dm + L.pos), (int32_t*)(dm + L.dec), (int32_t*)(dm + L.pre),
                        (int32_t*)(dm + L.comb), s.block_size, s.max_seqs, S, stream) !=
      hipSuccess) {
    (void)hipGetLastError();
    return RBKV_ERR_HIP;
  }
  return RBKV_OK;
}

// Decodes on the matrix-core kernel run as persistent workgroups in the serial call too:
// one per CU with three tile stages per wave (97 KB of LDS), taking items from a counter,
// instead of one workgroup per item (long decode 2262 -> 2177 us; with two stages and two
// workgroups per CU 2190 us, full-budget 614 against 605 us).  Single-head groups keep
// one workgroup per item on the register-only kernel.
constexpr int SERIAL_PERSISTENT_WG_PER_CU = 1;
constexpr int SERIAL_PERSISTENT_STAGES = 3;
bool serial_persistent(const rbkv_shape& s) { return decode_mfma_ok(s); }

// Workspace: the split-K partials, then (when decodes run as persistent workgroups: in
// the two-stream call, and in the serial call for the shapes above) the 256-byte-aligned
// counter they claim items from.
constexpr size_t CLAIM_BYTES = 256;
bool uses_claim(const rbkv_shape& s, const rbkv_batch& b) {
  return decode_persistent_ok(s) && b.n_decode_items > 0 &&
         (b.n_prefill_items > 0 || serial_persistent(s));
}

// Compute units of the current device.
hipError_t cu_count(int* n_cu) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess && *n_cu < 1) e = hipErrorInvalidDevice;
  return e;
}
size_t claim_offset(const rbkv_shape& s, const rbkv_batch& b) {
  const int32_t G = s.n_q_heads / s.n_kv_heads;
  const size_t partials = (size_t)b.n_partials * partial_floats(G, s.head_dim) * sizeof(float);
  return uses_claim(s, b) ? (partials + CLAIM_BYTES - 1) / CLAIM_BYTES * CLAIM_BYTES : partials;
}

bool same_shape(const rbkv_shape& a, const rbkv_shape& b) {
  return memcmp(&a, &b, sizeof(rbkv_shape)) == 0;
}

// Split size for single-token decodes: about the kernel's target number of items overall.
int32_t choose_split_tiles(const rbkv_shape& s, int64_t decode_tiles_total) {
  const bool small_group = s.n_q_heads / s.n_kv_heads <= 4;
  const int64_t target =
      decode_mfma_ok(s) || decode_reg_ok(s)
          ? (small_group ? DECODE_TARGET_ITEMS_MFMA : DECODE_TARGET_ITEMS_MFMA_WIDE)
      : decode_persistent_ok(s) ? (small_group ? DECODE_TARGET_ITEMS_LEAN : DECODE_TARGET_ITEMS_LEAN2)
      : decode_grouped(s)     ? DECODE_TARGET_ITEMS_GROUPED
                              : DECODE_TARGET_ITEMS;
  const int64_t cap = decode_mfma_ok(s) ? MAX_SPLIT_TILES_MFMA : MAX_SPLIT_TILES;
  int64_t st = cdiv64(decode_tiles_total, target);
  if (st < MIN_SPLIT_TILES) st = MIN_SPLIT_TILES;
  if (st > cap) st = cap;
  return (int32_t)st;
}

}  // namespace

extern "C" {

const char* rbkv_status_string(rbkv_status status) {
  switch (status) {
    case RBKV_OK: return "ok";
    case RBKV_ERR_INVALID_ARG: return "invalid argument";
    case RBKV_ERR_CAPACITY: return "batch exceeds max_tokens or max_seqs";
    case RBKV_ERR_BLOCKS: return "block list too short, id out of range or id used twice";
    case RBKV_ERR_UNSUPPORTED: return "unsupported shape (head_dim, block_size, dtype, group)";
    case RBKV_ERR_WORKSPACE: return "buffer smaller than the size query requires";
    case RBKV_ERR_DEVICE_PTR: return "buffer is not memory of the expected kind on this device";
    case RBKV_ERR_HIP: return "HIP call or kernel launch failed";
    case RBKV_ERR_HOST_MEMORY: return "host memory allocation failed";
    default: return "unknown status";
  }
}

rbkv_status rbkv_metadata_bytes(const rbkv_shape* shape, size_t* dev_bytes,
                                size_t* host_pinned_bytes) {
  rbkv_status st = check_shape(shape);
  if (st != RBKV_OK) return st;
  MetaLayout L = meta_layout(*shape);
  if (dev_bytes) *dev_bytes = L.total;
  if (host_pinned_bytes) *host_pinned_bytes = L.staging_bytes;
  return RBKV_OK;
}

rbkv_status rbkv_workspace_bytes(const rbkv_shape* shape, const rbkv_batch* batch,
                                 size_t* bytes) {
  rbkv_status st = check_shape(shape);
  if (st != RBKV_OK) return st;
  if (!batch || !bytes) return RBKV_ERR_INVALID_ARG;
  if (!same_shape(batch->shape, *shape)) return RBKV_ERR_INVALID_ARG;
  *bytes = claim_offset(*shape, *batch) + (uses_claim(*shape, *batch) ? CLAIM_BYTES : 0);
  return RBKV_OK;
}

rbkv_status ragged_batch_finalize(const rbkv_shape* shape, int32_t S, const int32_t* n_new,
                                  const int32_t* seen, const int32_t* const* block_ids,
                                  const int32_t* n_block_ids, void* host_pinned,
                                  size_t host_pinned_bytes, void* dev_meta,
                                  size_t dev_meta_bytes, void* stream, rbkv_batch* out) {
  rbkv_status st = check_shape(shape);
  if (st != RBKV_OK) return st;
  const rbkv_shape& s = *shape;
  if (!out || S < 0) return RBKV_ERR_INVALID_ARG;
  if (S > s.max_seqs) return RBKV_ERR_CAPACITY;
  if (S > 0 && (!n_new || !seen || !block_ids || !n_block_ids)) return RBKV_ERR_INVALID_ARG;
  if (!host_pinned || !dev_meta) return RBKV_ERR_INVALID_ARG;
  const MetaLayout L = meta_layout(s);
  if (host_pinned_bytes < L.staging_bytes || dev_meta_bytes < L.total)
    return RBKV_ERR_WORKSPACE;

  const int32_t Hkv = s.n_kv_heads;
  const int32_t G = s.n_q_heads / Hkv;
  const bool mfma = s.dtype == RBKV_DTYPE_BF16;
  const int32_t qtt = q_tile_tokens(G);

  // Per-sequence checks, totals and the decode tile count.
  int64_t T = 0, nblk = 0, dec_tiles = 0;
  for (int32_t i = 0; i < S; ++i) {
    if (n_new[i] < 1 || seen[i] < 0) return RBKV_ERR_INVALID_ARG;
    T += n_new[i];
    if (T > s.max_tokens) return RBKV_ERR_CAPACITY;
    const int64_t L_i = (int64_t)seen[i] + n_new[i];
    const int64_t B_i = cdiv64(L_i, s.block_size);
    if (B_i > s.num_blocks) return RBKV_ERR_BLOCKS;
    if (!block_ids[i] || n_block_ids[i] < B_i) return RBKV_ERR_BLOCKS;
    nblk += B_i;
    if (nblk > s.num_blocks) return RBKV_ERR_BLOCKS;  // ids are distinct, so they cannot fit
    if (n_new[i] == 1) dec_tiles += (int64_t)Hkv * cdiv64(L_i, KT);
  }
  // Block ids: in range and distinct across the batch.
  if (S > 0) {
    std::vector<uint8_t> used;
    try {
      used.assign((size_t)s.num_blocks, 0);
    } catch (const std::bad_alloc&) {
      return RBKV_ERR_HOST_MEMORY;
    }
    for (int32_t i = 0; i < S; ++i) {
      const int64_t B_i = cdiv64((int64_t)seen[i] + n_new[i], s.block_size);
      for (int64_t k = 0; k < B_i; ++k) {
        const int32_t id = block_ids[i][k];
        if (id < 0 || id >= s.num_blocks) return RBKV_ERR_BLOCKS;
        if (used[(size_t)id]) return RBKV_ERR_BLOCKS;
        used[(size_t)id] = 1;
      }
    }
  }

  const int32_t split = choose_split_tiles(s, dec_tiles);
  int64_t ndec = 0, npre = 0, npart = 0, ncomb = 0;
  int32_t npseq = 0, nqt_max = 0;
  for (int32_t i = 0; i < S; ++i) {
    SeqPlan p = plan_sequence(n_new[i], seen[i], Hkv, split, mfma, qtt);
    ndec += p.dec_items;
    npre += p.pre_items;
    npart += p.partials;
    ncomb += p.comb_items;
    if (p.pre_items > 0) {
      ++npseq;
      nqt_max = std::max(nqt_max, (int32_t)cdiv64(n_new[i], qtt));
    }
  }
  const Caps caps = work_caps(s);  // bounds every valid batch; checked to fail loudly
  if (ndec > caps.dec || npre > caps.pre || ncomb > caps.comb || npart > caps.dec ||
      ndec > INT32_MAX)
    return RBKV_ERR_CAPACITY;

  char* dm = (char*)dev_meta;
  rbkv_batch b;
  memset(&b, 0, sizeof(b));
  b.shape = s;
  b.S = S;
  b.T = (int32_t)T;
  b.n_blocks_used = (int32_t)nblk;
  b.split_tiles = split;
  b.n_decode_items = (int32_t)ndec;
  b.n_prefill_items = (int32_t)npre;
  b.n_partials = (int32_t)npart;
  b.n_combine_items = (int32_t)ncomb;
  b.n_prefill_seqs = npseq;
  b.prefill_qtiles_max = nqt_max;
  b.cu_seqlens = (const int32_t*)(dm + L.cu);
  b.seen = (const int32_t*)(dm + L.seen);
  b.kv_len = (const int32_t*)(dm + L.kv_len);
  b.block_offsets = (const int32_t*)(dm + L.block_off);
  b.block_ids = (const int32_t*)(dm + L.block_ids);
  b.token_to_seq = (const int32_t*)(dm + L.tok2seq);
  b.pos = (const int32_t*)(dm + L.pos);
  b.decode_work = (const int32_t*)(dm + L.dec);
  b.prefill_work = (const int32_t*)(dm + L.pre);
  b.combine_work = (const int32_t*)(dm + L.comb);
  if (S == 0) {  // nothing to build or launch
    *out = b;
    return RBKV_OK;
  }

  // Pointer kinds (the first HIP calls).
  if ((st = check_pinned(host_pinned)) != RBKV_OK) return st;
  if ((st = check_device(dev_meta, L.total)) != RBKV_OK) return st;

  // Pack header, n_new, seen and the flat block tables into the staging area.
  int32_t* hp = (int32_t*)host_pinned;
  memset(hp, 0, HDR_INTS * 4);
  hp[H_S] = S;
  hp[H_T] = (int32_t)T;
  hp[H_NBLK] = (int32_t)nblk;
  hp[H_SPLIT] = split;
  hp[H_HKV] = Hkv;
  hp[H_MFMA] = mfma ? 1 : 0;
  hp[H_QTT] = qtt;
  hp[H_NDEC] = (int32_t)ndec;
  hp[H_NPRE] = (int32_t)npre;
  hp[H_NPART] = (int32_t)npart;
  hp[H_NCOMB] = (int32_t)ncomb;
  hp[H_NPSEQ] = npseq;
  int32_t* hn = (int32_t*)((char*)host_pinned + L.n_new);
  int32_t* hs = (int32_t*)((char*)host_pinned + L.seen);
  int32_t* hb = (int32_t*)((char*)host_pinned + L.block_ids);
  memcpy(hn, n_new, (size_t)S * 4);
  memcpy(hs, seen, (size_t)S * 4);
  int64_t at = 0;
  for (int32_t i = 0; i < S; ++i) {
    const int64_t B_i = cdiv64((int64_t)seen[i] + n_new[i], s.block_size);
    memcpy(hb + at, block_ids[i], (size_t)B_i * 4);
    at += B_i;
  }

  hipStream_t hs_stream = (hipStream_t)stream;
  // One copy covers header, n_new, seen (capacity-sized) and the used block ids.
  const size_t copy_bytes = L.block_ids + (size_t)nblk * 4;
  if (hipMemcpyAsync(dm, host_pinned, copy_bytes, hipMemcpyHostToDevice, hs_stream) !=
      hipSuccess) {
    (void)hipGetLastError();
    return RBKV_ERR_HIP;
  }
  if ((st = launch_build(s, dm, S, hs_stream)) != RBKV_OK) return st;
  *out = b;
  return RBKV_OK;
}

rbkv_status ragged_batch_rebuild(const rbkv_shape* shape, const rbkv_batch* batch,
                                 void* stream) {
  rbkv_status st = check_shape(shape);
  if (st != RBKV_OK) return st;
  if (!batch || !same_shape(batch->shape, *shape)) return RBKV_ERR_INVALID_ARG;
  if (batch->S == 0) return RBKV_OK;
  // The staging image sits at the start of the metadata buffer, just before n_new.
  const MetaLayout L = meta_layout(*shape);
  char* dm = (char*)batch->seen - L.seen;
  if ((const char*)batch->cu_seqlens != dm + L.cu) return RBKV_ERR_INVALID_ARG;
  if ((st = check_device(dm, L.total)) != RBKV_OK) return st;
  return launch_build(*shape, dm, batch->S, (hipStream_t)stream);
}

rbkv_status blocked_kv_append_rotary(const rbkv_shape* shape, const rbkv_batch* batch,
                                     void* qkv, void* kv_pool, double rope_base,
                                     void* stream) {
  rbkv_status st = check_shape(shape);
  if (st != RBKV_OK) return st;
  if (!batch || !qkv || !kv_pool) return RBKV_ERR_INVALID_ARG;
  const rbkv_shape& s = *shape;
  if (!same_shape(batch->shape, s)) return RBKV_ERR_INVALID_ARG;
  if (batch->T < 0 || batch->T > s.max_tokens) return RBKV_ERR_INVALID_ARG;
  if (batch->T == 0) return RBKV_OK;
  const size_t e = elem_bytes(s);
  const size_t qkv_bytes = (size_t)batch->T * (s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim * e;
  const size_t pool_bytes = (size_t)s.num_blocks * 2 * s.n_kv_heads * s.block_size * s.head_dim * e;
  if ((st = check_device(qkv, qkv_bytes)) != RBKV_OK) return st;
  if ((st = check_device(kv_pool, pool_bytes)) != RBKV_OK) return st;
  if (launch_append_rotary(s, *batch, qkv, kv_pool, rope_base, (hipStream_t)stream) !=
      hipSuccess) {
    (void)hipGetLastError();
    return RBKV_ERR_HIP;
  }
  return RBKV_OK;
}

namespace {

// Argument checks of an attention call (phases pre / dec / comb requested and non-empty).
// *launch is false when there is nothing to launch (then no buffer is inspected).
// Checks shared by the attention calls.  workspace_owned: the workspace is the library's
// static scratch (its size is checked by the caller, and it is not a caller allocation
// that the pointer queries could describe), so only the caller's buffers are queried.
rbkv_status check_attention(const rbkv_shape* shape, const rbkv_batch* batch, bool pre,
                            bool dec, bool comb, const void* qkv, const void* kv_pool,
                            const void* out, const void* workspace, size_t workspace_bytes,
                            bool* launch, bool workspace_owned = false) {
  *launch = false;
  rbkv_status st = check_shape(shape);
  if (st != RBKV_OK) return st;
  if (!batch || !qkv || !kv_pool || !out) return RBKV_ERR_INVALID_ARG;
  const rbkv_shape& s = *shape;
  if (!same_shape(batch->shape, s)) return RBKV_ERR_INVALID_ARG;
  if (batch->T < 0 || batch->T > s.max_tokens) return RBKV_ERR_INVALID_ARG;
  size_t need = 0;
  if ((st = rbkv_workspace_bytes(shape, batch, &need)) != RBKV_OK) return st;
  if (workspace_bytes < need || (need > 0 && !workspace)) return RBKV_ERR_WORKSPACE;
  if (batch->T == 0 || (!pre && !dec && !comb)) return RBKV_OK;
  const size_t e = elem_bytes(s);
  const size_t qkv_bytes = (size_t)batch->T * (s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim * e;
  const size_t pool_bytes = (size_t)s.num_blocks * 2 * s.n_kv_heads * s.block_size * s.head_dim * e;
  const size_t out_bytes = (size_t)batch->T * s.n_q_heads * s.head_dim * e;
  if ((st = check_device(qkv, qkv_bytes)) != RBKV_OK) return st;
  if ((st = check_device(kv_pool, pool_bytes)) != RBKV_OK) return st;
  if ((st = check_device(out, out_bytes)) != RBKV_OK) return st;
  if (need > 0 && !workspace_owned && (st = check_device(workspace, need)) != RBKV_OK)
    return st;
  *launch = true;
  return RBKV_OK;
}

// Mixed batches whose decodes run on the matrix cores take one persistent launch for both
// phases (launch_mixed): one workgroup per CU, MIXED_DEC_FIRST of every XCD's 32 starting
// on the decode list.
constexpr int32_t MIXED_DEC_FIRST = 16;
bool mixed_launch(const rbkv_shape& s, bool pre, bool dec) {
  return pre && dec && decode_mfma_ok(s);
}

// The launches of one attention call on one stream (checks already done).
rbkv_status launch_attention(const rbkv_shape& s, const rbkv_batch& b, bool pre, bool dec,
                             bool comb, const void* qkv, const void* kv_pool, void* out,
                             void* workspace, hipStream_t hs) {
  hipError_t err = hipSuccess;
  if (mixed_launch(s, pre, dec)) {
    int n_cu = 0;
    int32_t* claims = (int32_t*)((char*)workspace + claim_offset(s, b));
    err = cu_count(&n_cu);
    if (err == hipSuccess) err = launch_claims_reset(claims, 9, hs);
    if (err == hipSuccess)
      err = launch_mixed(s, b, qkv, kv_pool, out, (float*)workspace, claims, n_cu,
                         MIXED_DEC_FIRST, hs);
    pre = dec = false;
  }
  if (err == hipSuccess && pre) err = launch_prefill(s, b, qkv, kv_pool, out, hs);
  if (err == hipSuccess && dec) {
    if (serial_persistent(s)) {
      int n_cu = 0;
      int32_t* claim = (int32_t*)((char*)workspace + claim_offset(s, b));
      err = cu_count(&n_cu);
      if (err == hipSuccess) err = launch_claims_reset(claim, 1, hs);
      if (err == hipSuccess)
        err = launch_decode_persistent(s, b, qkv, kv_pool, out, (float*)workspace, claim,
                                       SERIAL_PERSISTENT_WG_PER_CU * n_cu, hs,
                                       SERIAL_PERSISTENT_STAGES);
    } else {
      err = launch_decode(s, b, qkv, kv_pool, out, (float*)workspace, hs);
    }
  }
  if (err == hipSuccess && comb) err = launch_combine(s, b, (const float*)workspace, out, hs);
  if (err != hipSuccess) {
    (void)hipGetLastError();
    return RBKV_ERR_HIP;
  }
  return RBKV_OK;
}

}  // namespace

rbkv_status ragged_blocked_attention_phase(const rbkv_shape* shape, const rbkv_batch* batch,
                                           int32_t phase, const void* qkv, const void* kv_pool,
                                           void* out, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  if (phase < RBKV_PHASE_ALL || phase > RBKV_PHASE_ATTEND) return RBKV_ERR_INVALID_ARG;
  const bool both = phase == RBKV_PHASE_ALL || phase == RBKV_PHASE_ATTEND;
  const bool pre = (both || phase == RBKV_PHASE_PREFILL) && batch && batch->n_prefill_items > 0;
  const bool dec = (both || phase == RBKV_PHASE_DECODE) && batch && batch->n_decode_items > 0;
  const bool comb = (phase == RBKV_PHASE_ALL || phase == RBKV_PHASE_COMBINE) && batch &&
                    batch->n_combine_items > 0;
  bool launch = false;
  rbkv_status st = check_attention(shape, batch, pre, dec, comb, qkv, kv_pool, out, workspace,
                                   workspace_bytes, &launch);
  if (st != RBKV_OK || !launch) return st;
  return launch_attention(*shape, *batch, pre, dec, comb, qkv, kv_pool, out, workspace,
                          (hipStream_t)stream);
}

rbkv_status ragged_blocked_attention_noalloc(const rbkv_shape* shape, const rbkv_batch* batch,
                                             const void* qkv, const void* kv_pool, void* out,
                                             void* stream) {
  rbkv_status st = check_shape(shape);
  if (st != RBKV_OK) return st;
  if (!batch) return RBKV_ERR_INVALID_ARG;
  if (!same_shape(batch->shape, *shape)) return RBKV_ERR_INVALID_ARG;
  size_t need = 0;
  if ((st = rbkv_workspace_bytes(shape, batch, &need)) != RBKV_OK) return st;
  if (need > (size_t)RBKV_STATIC_SCRATCH_BYTES) return RBKV_ERR_WORKSPACE;
  const bool pre = batch->n_prefill_items > 0;
  const bool dec = batch->n_decode_items > 0;
  const bool comb = batch->n_combine_items > 0;
  // A non-null stand-in lets the shared checks run; the real address is resolved only
  // when there is something to launch.
  bool launch = false;
  st = check_attention(shape, batch, pre, dec, comb, qkv, kv_pool, out,
                       need > 0 ? (const void*)1 : nullptr, need, &launch, true);
  if (st != RBKV_OK || !launch) return st;
  void* ws = nullptr;
  if (need > 0 && static_scratch(&ws) != hipSuccess) {
    (void)hipGetLastError();
    return RBKV_ERR_HIP;
  }
  return launch_attention(*shape, *batch, pre, dec, comb, qkv, kv_pool, out, ws,
                          (hipStream_t)stream);
}

namespace {

// Shared checks of the two gathers; *row_bytes receives width * element size.
rbkv_status check_gather(const rbkv_batch* batch, int32_t width, int32_t dtype,
                         int64_t rows, size_t* row_bytes) {
  if (!batch || width < 1) return RBKV_ERR_INVALID_ARG;
  if (dtype != RBKV_DTYPE_F32 && dtype != RBKV_DTYPE_BF16) return RBKV_ERR_INVALID_ARG;
  const rbkv_shape& s = batch->shape;
  if (batch->T < 0 || batch->T > s.max_tokens || batch->S < 0 || batch->S > s.max_seqs ||
      batch->S > batch->T)
    return RBKV_ERR_INVALID_ARG;
  const size_t rb = (size_t)width * (dtype == RBKV_DTYPE_F32 ? 4 : 2);
  if (rb % 16 != 0) return RBKV_ERR_UNSUPPORTED;
  if ((uint64_t)rows * (rb / 16) >= (1ull << 31)) return RBKV_ERR_UNSUPPORTED;
  *row_bytes = rb;
  return RBKV_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

rbkv_status ragged_embedding_gather(const rbkv_batch* batch, const int32_t* token_ids,
                                    const void* table, int32_t vocab, int32_t width,
                                    int32_t dtype, void* out, void* stream) {
  size_t rb = 0;
  rbkv_status st = check_gather(batch, width, dtype, batch ? batch->T : 0, &rb);
  if (st != RBKV_OK) return st;
  if (!token_ids || !table || !out || vocab < 1) return RBKV_ERR_INVALID_ARG;
  if (!aligned16(table) || !aligned16(out)) return RBKV_ERR_INVALID_ARG;
  const int32_t T = batch->T;
  if (T == 0) return RBKV_OK;
  if ((st = check_device(token_ids, (size_t)T * 4)) != RBKV_OK) return st;
  if ((st = check_device(table, (size_t)vocab * rb)) != RBKV_OK) return st;
  if ((st = check_device(out, (size_t)T * rb)) != RBKV_OK) return st;
  if (launch_gather_rows(0, table, out, token_ids, vocab, T, rb, (hipStream_t)stream) !=
      hipSuccess) {
    (void)hipGetLastError();
    return RBKV_ERR_HIP;
  }
  return RBKV_OK;
}

rbkv_status ragged_logits_gather(const rbkv_batch* batch, const void* rows, int32_t width,
                                 int32_t dtype, void* out, void* stream) {
  size_t rb = 0;
  rbkv_status st = check_gather(batch, width, dtype, batch ? batch->S : 0, &rb);
  if (st != RBKV_OK) return st;
  if (!rows || !out) return RBKV_ERR_INVALID_ARG;
  if (!aligned16(rows) || !aligned16(out)) return RBKV_ERR_INVALID_ARG;
  const int32_t S = batch->S;
  if (S == 0) return RBKV_OK;
  if (!batch->cu_seqlens) return RBKV_ERR_INVALID_ARG;
  if ((st = check_device(batch->cu_seqlens, (size_t)(S + 1) * 4)) != RBKV_OK) return st;
  if ((st = check_device(rows, (size_t)batch->T * rb)) != RBKV_OK) return st;
  if ((st = check_device(out, (size_t)S * rb)) != RBKV_OK) return st;
  if (launch_gather_rows(1, rows, out, batch->cu_seqlens, batch->T, S, rb,
                         (hipStream_t)stream) != hipSuccess) {
    (void)hipGetLastError();
    return RBKV_ERR_HIP;
  }
  return RBKV_OK;
}

namespace {

size_t kv_block_bytes(const rbkv_shape& s) {
  return (size_t)2 * s.n_kv_heads * s.block_size * s.head_dim * elem_bytes(s);
}

// Device view of a page-locked host range [p, p + bytes): both ends must be page-locked
// host memory mapped at consecutive device addresses.
rbkv_status pinned_range(void* p, size_t bytes, char** dev) {
  hipPointerAttribute_t a, b;
  if (hipPointerGetAttributes(&a, p) != hipSuccess ||
      hipPointerGetAttributes(&b, (char*)p + bytes - 1) != hipSuccess) {
    (void)hipGetLastError();
    return RBKV_ERR_DEVICE_PTR;
  }
  if (a.type != hipMemoryTypeHost || b.type != hipMemoryTypeHost || !a.devicePointer ||
      (char*)b.devicePointer - (char*)a.devicePointer != (ptrdiff_t)(bytes - 1))
    return RBKV_ERR_DEVICE_PTR;
  *dev = (char*)a.devicePointer;
  return RBKV_OK;
}

rbkv_status kv_transfer(int dir, const rbkv_shape* shape, void* pool, int32_t n,
                        const int32_t* ids, void* host, size_t host_bytes, void* stream) {
  rbkv_status st = check_shape(shape);
  if (st != RBKV_OK) return st;
  if (n < 0 || !pool || !host || (n > 0 && !ids)) return RBKV_ERR_INVALID_ARG;
  if (n == 0) return RBKV_OK;
  const rbkv_shape& s = *shape;
  size_t need = 0;
  if ((st = rbkv_kv_host_bytes(shape, n, &need)) != RBKV_OK) return st;
  if (host_bytes < need) return RBKV_ERR_INVALID_ARG;
  const size_t bb = kv_block_bytes(s);
  if ((uint64_t)n * ((bb + 16383) / 16384) * 256 >= (1ull << 32)) return RBKV_ERR_UNSUPPORTED;
  for (int32_t k = 0; k < n; ++k)
    if (ids[k] < 0 || ids[k] >= s.num_blocks) return RBKV_ERR_BLOCKS;
  if (dir == 1) {  // destinations must be distinct
    std::vector<uint8_t> used;
    try {
      used.assign((size_t)s.num_blocks, 0);
    } catch (const std::bad_alloc&) {
      return RBKV_ERR_HOST_MEMORY;
    }
    for (int32_t k = 0; k < n; ++k) {
      if (used[(size_t)ids[k]]) return RBKV_ERR_BLOCKS;
      used[(size_t)ids[k]] = 1;
    }
  }
  if ((st = check_device(pool, (size_t)s.num_blocks * bb)) != RBKV_OK) return st;
  char* hdev = nullptr;
  if ((st = pinned_range(host, need, &hdev)) != RBKV_OK) return st;
  // Stage the ids behind the slabs; the kernel reads them through the mapping.
  const size_t ids_off = (size_t)n * bb;
  memcpy((char*)host + ids_off, ids, (size_t)n * 4);
  if (launch_kv_block_copy(dir, pool, hdev, (const int32_t*)(hdev + ids_off), n, bb,
                           (hipStream_t)stream) != hipSuccess) {
    (void)hipGetLastError();
    return RBKV_ERR_HIP;
  }
  return RBKV_OK;
}

}  // namespace

rbkv_status rbkv_kv_host_bytes(const rbkv_shape* shape, int32_t n, size_t* bytes) {
  rbkv_status st = check_shape(shape);
  if (st != RBKV_OK) return st;
  if (n < 0 || !bytes) return RBKV_ERR_INVALID_ARG;
  *bytes = (size_t)n * kv_block_bytes(*shape) + (size_t)n * 4;
  return RBKV_OK;
}

rbkv_status blocked_kv_offload(const rbkv_shape* shape, const void* kv_pool, int32_t n,
                               const int32_t* block_ids, void* host, size_t host_bytes,
                               void* stream) {
  return kv_transfer(0, shape, const_cast<void*>(kv_pool), n, block_ids, host, host_bytes,
                     stream);
}

rbkv_status blocked_kv_restore(const rbkv_shape* shape, void* kv_pool, int32_t n,
                               const int32_t* block_ids, void* host, size_t host_bytes,
                               void* stream) {
  return kv_transfer(1, shape, kv_pool, n, block_ids, host, host_bytes, stream);
}

rbkv_status ragged_blocked_attention(const rbkv_shape* shape, const rbkv_batch* batch,
                                     const void* qkv, const void* kv_pool, void* out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return ragged_blocked_attention_phase(shape, batch, RBKV_PHASE_ALL, qkv, kv_pool, out,
                                        workspace, workspace_bytes, stream);
}

namespace {

// The two-stream call for the persistent-decode shapes that do not take the mixed launch
// (head dim 64 with groups of up to eight heads, single-head groups at head dim 128):
// decode workgroups, two per CU, start beside the prefill on the side stream and take
// the CUs it leaves; once the prefill is done a second launch on the main stream joins
// them, four per CU.  Both take items from one counter, so they finish together whatever
// the split of the work.  (Sizes measured on the full-budget and SplitFuse batches when
// they ran this way: one per CU beside the prefill, or more than three, was slower; the
// second launch's size matters within 1-2%.)
constexpr int OVERLAP_SIDE_WG_PER_CU = 2;
constexpr int OVERLAP_MAIN_WG_PER_CU = 4;
rbkv_status attention_overlapped(const rbkv_shape& s, const rbkv_batch& b, const void* qkv,
                                 const void* kv_pool, void* out, char* ws, hipStream_t hs,
                                 hipStream_t hside, hipEvent_t fork, hipEvent_t join) {
  int n_cu = 0;
  if (cu_count(&n_cu) != hipSuccess) {
    (void)hipGetLastError();
    return RBKV_ERR_HIP;
  }
  int32_t* claim = (int32_t*)(ws + claim_offset(s, b));
  float* partials = (float*)ws;
  // The counter reset runs on the side stream ahead of the side decodes, so the prefill
  // starts on the main stream at once; the join event is recorded right after the reset
  // and the main stream waits for that record before its own decode launch (long done by
  // the time the prefill ends), then recorded again at the end for the final join.
  bool ok = hipEventRecord(fork, hs) == hipSuccess &&
            hipStreamWaitEvent(hside, fork, 0) == hipSuccess &&
            launch_claims_reset(claim, 1, hside) == hipSuccess &&
            hipEventRecord(join, hside) == hipSuccess &&
            launch_prefill(s, b, qkv, kv_pool, out, hs) == hipSuccess &&
            launch_decode_persistent(s, b, qkv, kv_pool, out, partials, claim,
                                     OVERLAP_SIDE_WG_PER_CU * n_cu, hside, 1) == hipSuccess &&
            hipStreamWaitEvent(hs, join, 0) == hipSuccess &&
            launch_decode_persistent(s, b, qkv, kv_pool, out, partials, claim,
                                     OVERLAP_MAIN_WG_PER_CU * n_cu, hs, 1) == hipSuccess;
  // Join whatever was launched, so the caller's stream never runs ahead of the side work.
  const bool joined = hipEventRecord(join, hside) == hipSuccess &&
                      hipStreamWaitEvent(hs, join, 0) == hipSuccess;
  ok = ok && joined && (b.n_combine_items == 0 ||
                        launch_combine(s, b, partials, out, hs) == hipSuccess);
  if (!ok) {
    (void)hipGetLastError();
    return RBKV_ERR_HIP;
  }
  return RBKV_OK;
}

}  // namespace

rbkv_status ragged_blocked_attention_concurrent(const rbkv_shape* shape, const rbkv_batch* batch,
                                                const void* qkv, const void* kv_pool, void* out,
                                                void* workspace, size_t workspace_bytes,
                                                void* stream, void* side_stream,
                                                void* fork_event, void* join_event) {
  if (!side_stream || !fork_event || !join_event || side_stream == stream)
    return RBKV_ERR_INVALID_ARG;
  const bool pre = batch && batch->n_prefill_items > 0;
  const bool dec = batch && batch->n_decode_items > 0;
  if (!pre || !dec)
    return ragged_blocked_attention(shape, batch, qkv, kv_pool, out, workspace,
                                    workspace_bytes, stream);
  // Every check (buffers included) before the fork, so an error launches nothing.
  bool launch = false;
  rbkv_status st = check_attention(shape, batch, pre, dec, batch->n_combine_items > 0, qkv,
                                   kv_pool, out, workspace, workspace_bytes, &launch);
  if (st != RBKV_OK || !launch) return st;
  hipStream_t hs = (hipStream_t)stream, hside = (hipStream_t)side_stream;
  hipEvent_t fork = (hipEvent_t)fork_event, join = (hipEvent_t)join_event;
  // Batches that take the mixed launch run it on the caller's stream (the two phases
  // already share the chip inside it).
  if (mixed_launch(*shape, pre, dec))
    return launch_attention(*shape, *batch, pre, dec, batch->n_combine_items > 0, qkv, kv_pool,
                            out, workspace, hs);
  if (uses_claim(*shape, *batch))
    return attention_overlapped(*shape, *batch, qkv, kv_pool, out, (char*)workspace, hs, hside,
                                fork, join);
  if (hipEventRecord(fork, hs) != hipSuccess || hipStreamWaitEvent(hside, fork, 0) != hipSuccess) {
    (void)hipGetLastError();
    return RBKV_ERR_HIP;
  }
  rbkv_status st2 = ragged_blocked_attention_phase(shape, batch, RBKV_PHASE_PREFILL, qkv,
                                                   kv_pool, out, workspace, workspace_bytes,
                                                   stream);
  st = ragged_blocked_attention_phase(shape, batch, RBKV_PHASE_DECODE, qkv, kv_pool, out,
                                      workspace, workspace_bytes, side_stream);
  // Join whatever was launched, so the caller's stream never runs ahead of the side work.
  if (hipEventRecord(join, hside) != hipSuccess || hipStreamWaitEvent(hs, join, 0) != hipSuccess) {
    (void)hipGetLastError();
    return RBKV_ERR_HIP;
  }
  if (st != RBKV_OK) return st;
  if (st2 != RBKV_OK) return st2;
  return ragged_blocked_attention_phase(shape, batch, RBKV_PHASE_COMBINE, qkv, kv_pool, out,
                                        workspace, workspace_bytes, stream);
}

}  // extern "C"
