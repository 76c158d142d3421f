/*
 * rbkv.h -- C ABI of librbkv: ragged-batch attention over a blocked (paged) KV cache
 * on AMD Instinct MI355X (gfx950).
 *
 * Three operations make up one forward pass of attention over a ragged batch:
 *
 *   ragged_batch_finalize     once per forward pass: validate the batch on the host and
 *                             build its device metadata (token offsets / cu_seqlens,
 *                             seen tokens, block tables, per-token sequence and
 *                             position, and the list of work items).
 *   blocked_kv_append_rotary  once per layer: rotate the new Q and K rows at their
 *                             absolute positions and store rotated K and raw V into the
 *                             sequence's KV blocks.
 *   ragged_blocked_attention  once per layer: causal softmax(Q K^T / sqrt(d)) V per
 *                             sequence over its blocks, with grouped-query heads.
 *
 * The ragged layout follows "DeepSpeed Inference v2 source tour" (pyshine.com), section
 * "Ragged batches: packing a whole server into four tensors": the live tokens of all
 * sequences sit edge to edge in one stream with no padding, a metadata buffer records
 * where each sequence's tokens start and stop, a tokens-to-sequence map rides beside
 * it, and kernels read per-sequence integer block ids to address the KV pool
 * directly.  The blocked pool (flat, block-indexed, with key and value views) follows
 * section "The front desk: put, query, can_schedule" of the same page.  Prefill chunks
 * and single-token decodes share one batch (Dynamic SplitFuse, "DeepSpeed-Inference
 * and DeepSpeed-MII" tutorial, sections 10.3 and 10.10).
 *
 * Conventions
 * -----------
 * - Every call returns an rbkv_status and never throws or aborts.  All argument checks
 *   run on the host before anything is launched or written; on error nothing is
 *   launched.  (Non-throwing verdicts follow can_schedule's SchedulingResult, same
 *   page, "The front desk" section; catching a buffer in the wrong place at call time
 *   rather than as a kernel fault follows InferenceParameter, section "Policies,
 *   containers, and a metaclass that checks your weights".)
 * - The caller owns all memory.  The library allocates no device memory, keeps no
 *   mutable global state and never synchronises the stream; every call only enqueues
 *   work on the given stream.  (One exception, for callers that cannot allocate:
 *   ragged_blocked_attention_noalloc uses a static scratch array the library holds per
 *   GPU.)
 * - `stream` is a hipStream_t passed as void*; NULL means the default stream.  Device
 *   buffers must belong to the current HIP device.
 * - Element types: RBKV_DTYPE_F32 (float) or RBKV_DTYPE_BF16 (bfloat16 bit patterns).
 *   Integers are int32.  All multi-dimensional arrays are dense, row-major.
 *
 * Layouts (d = head_dim, Hq = n_q_heads, Hkv = n_kv_heads, G = Hq / Hkv, bs = block_size)
 *   qkv      [T][Hq + 2*Hkv][d]   fused new rows: Q heads, then K heads, then V heads
 *   kv_pool  [num_blocks][2][Hkv][bs][d]   index 0 = keys, 1 = values; key p of a
 *            sequence lives in block block_ids[p / bs] at slot p % bs
 *   out      [T][Hq][d]           attention output, same dtype as qkv
 * Query head h reads kv head h / G.  Token k of a sequence with `seen` cached tokens
 * sits at position seen + k and attends to keys 0 .. seen + k of its own sequence.
 */
#ifndef RBKV_H
#define RBKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t rbkv_status;
enum {
  RBKV_OK = 0,
  RBKV_ERR_INVALID_ARG = 1, /* null pointer, negative count, n_new < 1, shape mismatch */
  RBKV_ERR_CAPACITY = 2,    /* T > max_tokens or S > max_seqs */
  RBKV_ERR_BLOCKS = 3,      /* block list too short, id out of range, id used twice */
  RBKV_ERR_UNSUPPORTED = 4, /* head_dim, block_size, dtype, group size or limits */
  RBKV_ERR_WORKSPACE = 5,   /* a caller buffer is smaller than the size query says */
  RBKV_ERR_DEVICE_PTR = 6,  /* buffer is not device (or pinned host) memory of the
                               current device, or its allocation is too small */
  RBKV_ERR_HIP = 7,         /* a HIP call or kernel launch failed */
  RBKV_ERR_HOST_MEMORY = 8  /* a host allocation of the library failed */
};

enum { RBKV_DTYPE_F32 = 0, RBKV_DTYPE_BF16 = 1 };

/* Phases of ragged_blocked_attention (see ragged_blocked_attention_phase). */
enum {
  RBKV_PHASE_ALL = 0,     /* ATTEND, then COMBINE */
  RBKV_PHASE_PREFILL = 1, /* multi-token chunks (bf16: matrix cores) */
  RBKV_PHASE_DECODE = 2,  /* single-token decodes, split-K (and float32 chunks) */
  RBKV_PHASE_COMBINE = 3, /* log-sum-exp merge of the split-K partials */
  RBKV_PHASE_ATTEND = 4   /* PREFILL and DECODE work items together (one launch for the
                             mixed batches of ragged_blocked_attention) */
};

/* Static shape of one attention layer and its KV pool, plus the batch capacities.
 * Supported: head_dim in {64, 128}; block_size in {16, 32, 64, 128};
 * n_q_heads = G * n_kv_heads with 1 <= G <= 16; 1 <= max_seqs <= 2048;
 * 1 <= max_tokens <= 1048576; 1 <= num_blocks <= 2^26.
 * The engine limits quoted on the pages are max_tokens = 8192 and max_seqs = 256
 * ("DeepSpeed-Inference and DeepSpeed-MII", section 10.3). */
typedef struct rbkv_shape {
  int32_t max_tokens;
  int32_t max_seqs;
  int32_t num_blocks;
  int32_t block_size;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;
} rbkv_shape;

/* A finalized batch: host-side counts plus device pointers into the caller's metadata
 * buffer.  Filled by ragged_batch_finalize; read-only for the caller; valid as long as
 * that buffer is (one batch serves every layer of the forward pass).  The device
 * arrays are int32:
 *   cu_seqlens[S+1]     start of each sequence's tokens in the packed stream
 *   seen[S]             tokens already cached before this pass
 *   kv_len[S]           seen + new tokens
 *   block_offsets[S+1]  start of each sequence's block table in block_ids
 *   block_ids[n_blocks_used]  the first ceil(kv_len / block_size) ids of each list
 *   token_to_seq[T]     owning sequence of each packed token
 *   pos[T]              absolute position of each packed token
 *   decode_work, prefill_work, combine_work: work-item records (4 int32 each) of the
 *                       three attention kernels; their format is internal (prefill_work
 *                       holds one record per chunk sequence, longest first). */
typedef struct rbkv_batch {
  rbkv_shape shape; /* the shape this batch was built for */
  int32_t S;
  int32_t T;
  int32_t n_blocks_used;
  int32_t split_tiles;   /* keys per decode split, in units of 64 keys */
  int32_t n_decode_items;
  int32_t n_prefill_items;
  int32_t n_partials;    /* split-K partial-result slots needed in the workspace */
  int32_t n_combine_items;
  int32_t n_prefill_seqs;      /* sequences whose chunk runs on the matrix cores */
  int32_t prefill_qtiles_max;  /* most query tiles of one such sequence */
  const int32_t* cu_seqlens;
  const int32_t* seen;
  const int32_t* kv_len;
  const int32_t* block_offsets;
  const int32_t* block_ids;
  const int32_t* token_to_seq;
  const int32_t* pos;
  const int32_t* decode_work;
  const int32_t* prefill_work;
  const int32_t* combine_work;
} rbkv_batch;

/* Static string naming a status code (never NULL). */
const char* rbkv_status_string(rbkv_status status);

/* Sizes of the two caller-owned buffers ragged_batch_finalize needs for `shape`:
 * device metadata (dev_bytes) and page-locked host staging (host_pinned_bytes, from
 * hipHostMalloc).  They play the part of the host buffers that the pages' batch wrapper
 * fills ahead of time and of its device tensors ("DeepSpeed Inference v2 source tour",
 * section "Ragged batches").
 * Either output pointer may be NULL.  Pure host computation. */
rbkv_status rbkv_metadata_bytes(const rbkv_shape* shape, size_t* dev_bytes,
                                size_t* host_pinned_bytes);

/* Device workspace ragged_blocked_attention needs for `batch` (split-K partial
 * results; the scratch output the blocked attention kernel is handed in the same
 * section), plus a 256-byte-aligned block of item counters for work that runs as
 * persistent workgroups: bf16 batches over blocks of 64+ keys with both prefill chunks
 * and decodes, at head dim 64 with groups of at most eight heads, at head dim 128 with
 * groups of up to 16; and, at head dim 128 with groups of 2-16 heads, any batch with
 * decodes.  The calls reset the counters themselves (a kernel, no memset).  0 when no
 * decode is split and no counter is needed.  Pure host computation. */
rbkv_status rbkv_workspace_bytes(const rbkv_shape* shape, const rbkv_batch* batch,
                                 size_t* bytes);

/* Build the device metadata of one ragged batch (the pages' insert_sequence then
 * finalize, "DeepSpeed Inference v2 source tour", section "Ragged batches").
 *
 *   S                  number of sequences, 0 <= S <= max_seqs (S = 0: no-op, OK)
 *   n_new[S]           new tokens per sequence (>= 1), host memory
 *   seen[S]            tokens already in the cache per sequence (>= 0), host memory
 *   block_ids[S]       host array of S host pointers: sequence i's block-id list
 *   n_block_ids[S]     length of each list; must be >= ceil((seen+n_new)/block_size);
 *                      only that many leading ids are used.  Used ids must lie in
 *                      [0, num_blocks) and be distinct across the whole batch.
 *   host_pinned        page-locked staging buffer (hipHostMalloc) of at least the
 *                      size rbkv_metadata_bytes gives; it must stay untouched until
 *                      the stream has passed this call (the upload is asynchronous).
 *   dev_meta           device buffer of at least the size rbkv_metadata_bytes gives.
 *   out                filled on success (host struct).
 * Errors: INVALID_ARG, CAPACITY (S > max_seqs, sum(n_new) > max_tokens), BLOCKS,
 * UNSUPPORTED, WORKSPACE (a buffer smaller than required), DEVICE_PTR, HIP.
 * Enqueues one host-to-device copy and one kernel on `stream`. */
rbkv_status ragged_batch_finalize(const rbkv_shape* shape, int32_t S, const int32_t* n_new,
                                  const int32_t* seen, const int32_t* const* block_ids,
                                  const int32_t* n_block_ids, void* host_pinned,
                                  size_t host_pinned_bytes, void* dev_meta,
                                  size_t dev_meta_bytes, void* stream, rbkv_batch* out);

/* Re-run the device half of ragged_batch_finalize: rebuild the batch's device metadata
 * from the staged copy already in its metadata buffer, with no host packing and no
 * transfer.  For a batch whose metadata buffer was reused or overwritten, or to time
 * the device work alone.  `batch` must come from a successful finalize with the same
 * shape and metadata buffer.  Errors: INVALID_ARG, HIP.  Enqueues one kernel. */
rbkv_status ragged_batch_rebuild(const rbkv_shape* shape, const rbkv_batch* batch,
                                 void* stream);

/* Rotary position embedding and KV append for one layer.
 *   qkv       device [T][Hq + 2*Hkv][d]; the Q heads are rotated IN PLACE, K and V rows
 *             are left as they are.
 *   kv_pool   device [num_blocks][2][Hkv][bs][d]; for each new token at position p the
 *             rotated K and the raw V are written to block block_ids[p / bs], slot
 *             p % bs, of its sequence.  No other pool element is touched.
 *   rope_base > 0: rotate each pair (x_j, x_{j + d/2}) by the angle p * base^(-2j/d)
 *             (angle, sine and cosine in float64, the rotation in float64, one
 *             round-to-nearest-even into the storage dtype); <= 0: no rotation.
 * Errors: INVALID_ARG (null, batch built for another shape), DEVICE_PTR, HIP. */
rbkv_status blocked_kv_append_rotary(const rbkv_shape* shape, const rbkv_batch* batch,
                                     void* qkv, void* kv_pool, double rope_base,
                                     void* stream);

/* Causal grouped-query attention of every new token over its sequence's blocks:
 * out[t][h] = sum_p softmax_p(q_t,h . K[p, h/G] / sqrt(d)) V[p, h/G], p = 0 .. pos[t].
 *   qkv       device [T][Hq + 2*Hkv][d] (read: the rotated Q heads)
 *   kv_pool   device pool already holding this pass's keys and values
 *   out       device [T][Hq][d], written entirely
 *   workspace device scratch of at least rbkv_workspace_bytes (may be NULL if 0)
 * Single-token decodes run as split-K streaming over 64-key tiles followed by a
 * log-sum-exp combine; bf16 prefill chunks run on MFMA tiles; float32 runs on the
 * vector ALUs throughout.  Accumulation is float32.  Batches with both chunks and
 * decodes in bf16 at head dim 128, groups of 2-16 heads and blocks of 64+ keys run both
 * kinds of work item in one launch of persistent workgroups (one per CU, each taking
 * chunk tiles and decode items from counters in the workspace), then the combine.
 * Errors: INVALID_ARG, WORKSPACE, DEVICE_PTR, HIP. */
rbkv_status ragged_blocked_attention(const rbkv_shape* shape, const rbkv_batch* batch,
                                     const void* qkv, const void* kv_pool, void* out,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* Size of the library's static scratch: the largest split-K workspace (as
 * rbkv_workspace_bytes reports it) that ragged_blocked_attention_noalloc accepts.
 * 64 MiB covers every measured batch (the 256-sequence long-context decode batch needs
 * about 32 MiB). */
#define RBKV_STATIC_SCRATCH_BYTES (64u << 20)

/* ragged_blocked_attention without a caller workspace and without any allocation: for
 * callers that cannot allocate device memory or pass one (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The split-K partials go to a
 * fixed array of RBKV_STATIC_SCRATCH_BYTES that the library holds in device memory, one
 * per GPU it runs on, until the process ends (its address is looked up once per device,
 * at the first call on that device).  Same kernels, same result (bit for bit) as
 * ragged_blocked_attention.  The call allocates nothing (no hipMalloc, no allocating
 * library routine) and never synchronises.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (two
 * streams, or two host threads) race and may corrupt each other's results, so order
 * them (one stream).  Nothing in the array needs to start at zero; it keeps the last
 * call's partials.
 * Errors: WORKSPACE (the batch needs more split-K scratch than
 * RBKV_STATIC_SCRATCH_BYTES: use ragged_blocked_attention with a workspace), and as
 * ragged_blocked_attention (INVALID_ARG, DEVICE_PTR, HIP).  All checks run before
 * anything is launched. */
rbkv_status ragged_blocked_attention_noalloc(const rbkv_shape* shape, const rbkv_batch* batch,
                                             const void* qkv, const void* kv_pool, void* out,
                                             void* stream);

/* One phase of ragged_blocked_attention (RBKV_PHASE_*), for callers that place other
 * work between the phases or time them separately.  Running ATTEND then COMBINE on one
 * stream is exactly ragged_blocked_attention (bit for bit).  PREFILL, DECODE, COMBINE in
 * this order compute the same attention with the chunks and the decodes in separate
 * launches; for the batches ragged_blocked_attention runs in one launch, the decodes then
 * split their keys over four instead of eight wavefronts, so results agree to rounding
 * (within the float32 accumulation), not bit for bit.  COMBINE reads what DECODE (or
 * ATTEND) wrote to the workspace.  A phase with no work items returns OK without
 * launching.  Errors: as ragged_blocked_attention, plus INVALID_ARG for an unknown
 * phase. */
rbkv_status ragged_blocked_attention_phase(const rbkv_shape* shape, const rbkv_batch* batch,
                                           int32_t phase, const void* qkv, const void* kv_pool,
                                           void* out, void* workspace, size_t workspace_bytes,
                                           void* stream);

/* ragged_blocked_attention with its two independent phases running at once.  Batches
 * that ragged_blocked_attention already runs in one launch (bf16, head dim 128, groups of
 * 2-16 heads, blocks of 64+ keys) run exactly that on `stream` and leave the side
 * stream and the events unused.  Otherwise the matrix-core prefill chunks run on
 * `stream`, the single-token decodes beside them on `side_stream`, then the split-K
 * combine on `stream` once both are done.  The phases read the same inputs and write
 * disjoint output rows, and every decode work item is computed by one workgroup in the
 * same order as in the serial call, so the result is identical (bit for bit) to
 * ragged_blocked_attention.  For bf16 over blocks of 64+ keys (head dim 64 with groups of
 * up to eight heads, head dim 128 with single-head groups) the decodes run as persistent
 * workgroups taking items from a counter in the workspace (reset by the call): two per CU
 * start beside the prefill, and more join on `stream` once the prefill is done, so the
 * chip is shared between the phases rather than split by kernel boundaries.  Other
 * shapes gain only where one phase leaves CUs idle.  Calls sharing a workspace must be
 * ordered (one stream).  The
 * fork and join use two caller-owned events (hipEvent_t as void*, created by the
 * caller, e.g. with hipEventDisableTiming): fork_event is recorded on `stream` and
 * waited on by `side_stream`; join_event is recorded on `side_stream` and waited on by
 * `stream` (on the persistent-decode path twice: after the counter reset, which runs on
 * `side_stream`, before the main stream's own decode launch, and at the end).  Both
 * streams must be of the current device and must differ.  With no
 * prefill or no decode work the call runs like ragged_blocked_attention on `stream`
 * alone and leaves the events unused.  Graph-capturable like the rest (the standard
 * event fork/join).  Errors: as ragged_blocked_attention, plus INVALID_ARG (NULL
 * side_stream or event, side_stream == stream). */
rbkv_status ragged_blocked_attention_concurrent(const rbkv_shape* shape, const rbkv_batch* batch,
                                                const void* qkv, const void* kv_pool, void* out,
                                                void* workspace, size_t workspace_bytes,
                                                void* stream, void* side_stream,
                                                void* fork_event, void* join_event);

/* The two row gathers that frame the layer stack over the same ragged batch ("DeepSpeed
 * Inference v2 source tour", section "Ragged batches: packing a whole server into four
 * tensors": the ragged embedding kernel gathers embedding rows for the packed token
 * stream, and the logits gather copies out only each sequence's last-token row for
 * sampling).  Both copy whole rows byte for byte; `dtype` (RBKV_DTYPE_*) only sets the
 * element size.  A row must be a multiple of 16 bytes and every buffer 16-byte aligned.
 * `batch` is a finalized batch (its T, S and device cu_seqlens are used); no shape is
 * needed.  Errors: INVALID_ARG (NULL, width or vocab < 1, bad dtype, misaligned buffer,
 * a batch outside its shape's limits), UNSUPPORTED (row bytes not a multiple of 16, or
 * more than 2^31 16-byte words to copy), DEVICE_PTR, HIP. */

/* out[t][:] = table[token_ids[t]][:] for t < batch->T.  token_ids: device int32 [T];
 * table: device [vocab][width]; out: device [T][width].  An id outside [0, vocab) gives a
 * zero row (device ids cannot be checked on the host without a synchronisation). */
rbkv_status ragged_embedding_gather(const rbkv_batch* batch, const int32_t* token_ids,
                                    const void* table, int32_t vocab, int32_t width,
                                    int32_t dtype, void* out, void* stream);

/* out[i][:] = rows[cu_seqlens[i + 1] - 1][:] for i < batch->S: the row of each
 * sequence's last new token.  rows: device [T][width]; out: device [S][width]. */
rbkv_status ragged_logits_gather(const rbkv_batch* batch, const void* rows, int32_t width,
                                 int32_t dtype, void* out, void* stream);

/* KV block offload and restore ("DeepSpeed Inference v2 source tour", section "The
 * front desk: put, query, can_schedule", and its overview list: besides the allocator's
 * bookkeeping, the blocked KV cache can copy chosen blocks out to host memory to make
 * room on the device and copy them back when their sequence runs again).
 *
 * The host buffer is page-locked memory (hipHostMalloc; torch pin_memory) of at least
 * rbkv_kv_host_bytes(shape, n) bytes laid out as
 *   [n][2][Hkv][bs][d]  the n blocks in list order (each exactly as in the pool)
 *   [n] int32           block ids
 * Both calls first write `block_ids` (a host array) into the id region, then enqueue one
 * kernel on `stream` that copies every listed block straight between the pool and the
 * host buffer; the buffer must stay untouched until the stream has passed that kernel.
 * offload: host slab k <- pool block block_ids[k] (the pool is not modified; the id
 *          region keeps the source ids as a manifest).
 * restore: pool block block_ids[k] <- host slab k (slabs written by an earlier offload of
 *          the same shape; the id region is overwritten with the destination ids, which
 *          must be distinct).  No other pool element is touched.
 * Errors: INVALID_ARG (NULL, n < 0, host buffer smaller than required), BLOCKS (an id
 * out of range, or repeated in a restore), UNSUPPORTED (n too large for one launch),
 * DEVICE_PTR (pool not device memory of this device, host buffer not page-locked across
 * its whole range), HIP.  n = 0 is OK and does nothing. */
rbkv_status rbkv_kv_host_bytes(const rbkv_shape* shape, int32_t n, size_t* bytes);

rbkv_status blocked_kv_offload(const rbkv_shape* shape, const void* kv_pool, int32_t n,
                               const int32_t* block_ids, void* host, size_t host_bytes,
                               void* stream);

rbkv_status blocked_kv_restore(const rbkv_shape* shape, void* kv_pool, int32_t n,
                               const int32_t* block_ids, void* host, size_t host_bytes,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RBKV_H */
