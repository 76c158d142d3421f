/*
 * rbkv_state.h -- host-side KV block allocator and sequence ledger of librbkv.
 *
 * These calls do the bookkeeping that comes before ragged_batch_finalize in every
 * forward pass: which sequences are alive, how many tokens each has in the cache, and
 * which KV blocks of the pool each one owns.  They run on the host only (no HIP call,
 * except inside rbkv_state_finalize, which forwards to ragged_batch_finalize).
 *
 * Sources, "DeepSpeed Inference v2 source tour" (pyshine.com):
 *   - section "The front desk: put, query, can_schedule": the ledger (DSStateManager)
 *     is configured with a cap on tracked sequences; each sequence remembers only
 *     integer block ids; a block allocator (BlockedAllocator) hands out free indices
 *     and takes them back and is the whole memory manager; can_schedule checks the
 *     candidates against the tracked-sequence cap and the free-block count and returns
 *     a verdict instead of failing; query reports, for a token and block budget,
 *     whether a sequence can run this pass; flush retires a sequence and returns its
 *     blocks;
 *   - overview list of the same page: the ledger creates sequences on first use and
 *     allocates blocks; a sequence descriptor's block list grows through
 *     extend_kv_cache;
 *   - section "Policies, containers, and a metaclass that checks your weights": blocks
 *     are requested before each forward pass from the sequence's KV requirements.
 * The free-block count as a queryable property is also in the tutorial chapter
 * "DeepSpeed-Inference and DeepSpeed-MII" (jwzheng96.github.io), section 10.10.
 *
 * Readings where the pages leave the rule open:
 *   - The allocator may return any free ids.  This one is a LIFO free list: the most
 *     recently freed ids come back first; a fresh pool hands out 0, 1, 2, ...
 *   - A request for more blocks than are free fails as a whole (nothing is handed out),
 *     and freeing an id that is not allocated fails as a whole (nothing is freed).
 *   - A sequence holds ceil(tokens / block_size) blocks for its cached plus in-flight
 *     tokens; blocks are taken when a batch is put, before the pass, and the sequence's
 *     seen count advances only when the pass is declared done (rbkv_state_post_forward).
 *   - can_schedule's verdict order is fixed below (RBKV_SCHED_*).
 *
 * Conventions: every call returns an rbkv_status (rbkv.h) and never throws or aborts;
 * on any non-OK status the object is unchanged.  Objects are not thread-safe: one
 * thread at a time per object.  Sequence ids (uid) are arbitrary int64 values chosen
 * by the caller.
 */
#ifndef RBKV_STATE_H
#define RBKV_STATE_H

#include <stddef.h>
#include <stdint.h>

#include "rbkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------------------------
 * Block allocator
 * --------------------------------------------------------------------------------- */

typedef struct rbkv_allocator rbkv_allocator; /* opaque */

/* Create an allocator over block ids 0 .. num_blocks - 1, all free.
 * Errors: INVALID_ARG (out NULL, num_blocks < 1), UNSUPPORTED (num_blocks > 2^26). */
rbkv_status rbkv_allocator_create(int32_t num_blocks, rbkv_allocator** out);

/* Destroy; NULL is accepted.  Always OK. */
rbkv_status rbkv_allocator_destroy(rbkv_allocator* a);

/* Take n free ids and write them to ids[0 .. n-1] (host array the caller owns).
 * n = 0 is OK and writes nothing.  Errors: INVALID_ARG (a NULL, n < 0, ids NULL with
 * n > 0), BLOCKS (fewer than n ids free; nothing is taken). */
rbkv_status rbkv_allocator_allocate(rbkv_allocator* a, int32_t n, int32_t* ids);

/* Give back n ids.  Errors: INVALID_ARG (a NULL, n < 0, ids NULL with n > 0), BLOCKS (an
 * id out of range, not currently allocated, or listed twice; nothing is freed). */
rbkv_status rbkv_allocator_free(rbkv_allocator* a, int32_t n, const int32_t* ids);

/* Number of free ids.  Errors: INVALID_ARG. */
rbkv_status rbkv_allocator_free_count(const rbkv_allocator* a, int32_t* n);

/* ---------------------------------------------------------------------------------
 * Sequence ledger
 * --------------------------------------------------------------------------------- */

typedef struct rbkv_state rbkv_state; /* opaque */

typedef struct rbkv_state_config {
  int32_t num_blocks;       /* blocks in the KV pool; the ledger owns ids 0..num_blocks-1 */
  int32_t block_size;       /* keys per block */
  int32_t max_tracked_seqs; /* sequences the ledger holds at once (created, not flushed) */
  int32_t max_seqs;         /* sequences in one batch */
  int32_t max_tokens;       /* new tokens in one batch */
  int32_t max_context;      /* tokens one sequence may hold (cached + new) */
} rbkv_state_config;

/* Verdicts of rbkv_state_can_schedule / rbkv_state_put (the pages' SchedulingResult).
 * When several limits are exceeded the first in this order is reported:
 *   1. BATCH_SEQ_LIMIT    more than max_seqs sequences in the batch
 *   2. BATCH_TOKEN_LIMIT  more than max_tokens new tokens in the batch
 *   3. walking the uids in batch order, the first of:
 *      ENGINE_SEQ_LIMIT   this uid is new and the ledger would exceed max_tracked_seqs
 *      SEQ_TOKEN_LIMIT    this sequence's cached + new tokens exceed max_context
 *      KV_LIMIT           the blocks needed so far exceed the free-block count */
enum {
  RBKV_SCHED_OK = 0,
  RBKV_SCHED_ENGINE_SEQ_LIMIT = 1,
  RBKV_SCHED_KV_LIMIT = 2,
  RBKV_SCHED_BATCH_SEQ_LIMIT = 3,
  RBKV_SCHED_BATCH_TOKEN_LIMIT = 4,
  RBKV_SCHED_SEQ_TOKEN_LIMIT = 5
};

/* Create an empty ledger with its own allocator over the pool's blocks.
 * Errors: INVALID_ARG (NULL, a field < 1), UNSUPPORTED (num_blocks > 2^26,
 * max_tracked_seqs or max_seqs > 65536, max_tokens > 2^20, block_size > 4096). */
rbkv_status rbkv_state_create(const rbkv_state_config* cfg, rbkv_state** out);

/* Destroy; NULL is accepted.  Always OK. */
rbkv_status rbkv_state_destroy(rbkv_state* s);

/* Free blocks of the pool, and sequences currently tracked.  Either pointer may be
 * NULL.  Errors: INVALID_ARG (s NULL). */
rbkv_status rbkv_state_counts(const rbkv_state* s, int32_t* free_blocks, int32_t* n_tracked);

/* One sequence: cached tokens (`seen`), tokens in the open batch (`in_flight`, 0 when
 * it is not in it) and blocks held.  Any output pointer may be NULL.
 * Errors: INVALID_ARG (s NULL, uid not tracked). */
rbkv_status rbkv_state_sequence(const rbkv_state* s, int64_t uid, int32_t* seen,
                                int32_t* in_flight, int32_t* n_blocks);

/* Copy the block ids a sequence holds, in key order (key p lives in ids[p / bs]), into
 * ids[0 .. cap-1]; *n receives the number held.  Errors: INVALID_ARG (NULL, unknown
 * uid, cap < number held). */
rbkv_status rbkv_state_block_ids(const rbkv_state* s, int64_t uid, int32_t* ids, int32_t cap,
                                 int32_t* n);

/* KV requirements of running `max_new_tokens` more tokens of sequence `uid` when at most
 * `max_new_blocks` more blocks can be given to it (the pages' query / get_kv_requirements).
 * An unknown uid is a sequence with nothing cached and no blocks.  With `held` blocks
 * and `seen` cached tokens:
 *   need = ceil((seen + max_new_tokens) / bs) - held, at least 0;
 *   if need <= max_new_blocks:  *tokens = max_new_tokens,                 *blocks = need
 *   else:                       *tokens = (held + max_new_blocks) * bs - seen,
 *                               *blocks = max_new_blocks
 * so *tokens is how many of the tokens fit and *blocks how many blocks they need.  A
 * sequence in the open batch counts its in-flight tokens as cached.
 * Errors: INVALID_ARG (NULL, max_new_tokens < 0, max_new_blocks < 0, uid offloaded). */
rbkv_status rbkv_state_query(const rbkv_state* s, int64_t uid, int32_t max_new_tokens,
                             int32_t max_new_blocks, int32_t* tokens, int32_t* blocks);

/* Verdict (RBKV_SCHED_*) of running n sequences with n_new[i] new tokens each as one
 * batch, without changing anything.  While a batch is open its in-flight tokens count
 * as cached.  Errors: INVALID_ARG (NULL, n < 0, n_new[i] < 1, a uid listed twice). */
rbkv_status rbkv_state_can_schedule(const rbkv_state* s, int32_t n, const int64_t* uids,
                                    const int32_t* n_new, int32_t* verdict);

/* Dynamic SplitFuse composition of the next batch from a queue of candidates, without
 * changing anything.  Candidate i is sequence uids[i] (tracked or new) with pending[i]
 * tokens waiting to be fed: 1 for a decode, the rest of its prompt for a prefill.  The
 * batch mixes single-token decodes and prefill chunks in one pass and fills the token
 * budget by cutting a prompt that does not fit into a chunk of what is left; the rest of
 * that prompt waits for later passes ("DeepSpeed-Inference and DeepSpeed-MII",
 * sections 10.3 and 10.10: prefill and decode requests of the queue are merged into one
 * forward pass before put).  Rule, with budget = min(token_budget, max_tokens):
 *   two walks over the queue in its order, first the candidates with pending = 1, then
 *   those with pending > 1; each candidate, while fewer than max_seqs are chosen and
 *   budget is left, is offered want = min(pending, budget left, max_context - cached)
 *   tokens, cut further to what the free blocks not yet promised can hold (the
 *   rbkv_state_query rule with max_new_blocks = those blocks); a new uid needs a free
 *   tracked slot.  A candidate offered nothing is skipped.  The chosen (uid, tokens)
 *   pairs are written in choice order (decodes first) to out_uids / out_n, which must
 *   hold min(n, max_seqs) entries; *S receives their count.  rbkv_state_put of that
 *   list returns RBKV_SCHED_OK.  While a batch is open its in-flight tokens count as
 *   cached.
 * Errors: INVALID_ARG (NULL, n < 0, token_budget < 1, pending[i] < 1, a uid listed
 * twice), CAPACITY (n > 65536). */
rbkv_status rbkv_state_compose(const rbkv_state* s, int32_t n, const int64_t* uids,
                               const int32_t* pending, int32_t token_budget, int32_t* S,
                               int64_t* out_uids, int32_t* out_n);

/* Open a batch: if can_schedule's verdict is OK, create the new sequences, extend each
 * sequence's block list to cover its cached + new tokens (blocks from the allocator) and
 * record n_new as in flight; otherwise change nothing.  *verdict receives the verdict
 * either way; the status is OK in both cases.  Errors: as rbkv_state_can_schedule, and
 * INVALID_ARG while a batch is already open. */
rbkv_status rbkv_state_put(rbkv_state* s, int32_t n, const int64_t* uids,
                           const int32_t* n_new, int32_t* verdict);

/* Views of the open batch in the form ragged_batch_finalize takes: S sequences in put
 * order, their new and cached token counts and block lists (pointers into the ledger,
 * valid until the next call that changes it).  Any output pointer may be NULL.
 * Errors: INVALID_ARG (s NULL, no open batch). */
rbkv_status rbkv_state_batch(const rbkv_state* s, int32_t* S, const int32_t** n_new,
                             const int32_t** seen, const int32_t* const** block_ids,
                             const int32_t** n_block_ids);

/* ragged_batch_finalize of the open batch (see rbkv.h for every argument after `s`).
 * `shape` must match the ledger's num_blocks and block_size.  Errors: INVALID_ARG (no
 * open batch, shape mismatch), and those of ragged_batch_finalize. */
rbkv_status rbkv_state_finalize(const rbkv_state* s, const rbkv_shape* shape,
                                void* host_pinned, size_t host_pinned_bytes, void* dev_meta,
                                size_t dev_meta_bytes, void* stream, rbkv_batch* out);

/* Close the open batch after its forward pass: each sequence's seen count grows by its
 * in-flight tokens.  Errors: INVALID_ARG (s NULL, no open batch). */
rbkv_status rbkv_state_post_forward(rbkv_state* s);

/* Retire a sequence: its blocks go back to the allocator and its slot is freed.
 * Errors: INVALID_ARG (s NULL, uid not tracked, uid in the open batch). */
rbkv_status rbkv_state_flush(rbkv_state* s, int64_t uid);

/* Offload a sequence's blocks ("DeepSpeed Inference v2 source tour", section "The front
 * desk": chosen blocks are copied to host memory to make room on the device, and copied
 * back when their sequence is scheduled again).  rbkv_state_offload writes the ids the
 * sequence holds, in key order, to ids[0 .. *n - 1] (cap >= that count) and gives them
 * back to the allocator; the sequence keeps its slot and cached count but holds no
 * blocks until rbkv_state_restore.  The caller copies the blocks out with
 * blocked_kv_offload on the stream that later reuses them, before anything that could
 * write them.  While offloaded a sequence may only be restored or flushed: naming it in
 * query, can_schedule, put or compose is INVALID_ARG, and rbkv_state_sequence reports 0
 * blocks.
 * Errors: INVALID_ARG (NULL, uid not tracked, in the open batch or already offloaded,
 * cap too small). */
rbkv_status rbkv_state_offload(rbkv_state* s, int64_t uid, int32_t* ids, int32_t cap,
                               int32_t* n);

/* Give an offloaded sequence ceil(cached / block_size) blocks again and write their ids,
 * in key order, to ids[0 .. *n - 1]; the caller copies the offloaded blocks back into
 * them with blocked_kv_restore.  Errors: INVALID_ARG (NULL, uid not tracked or not
 * offloaded, cap too small), BLOCKS (not enough free blocks; nothing changes),
 * HOST_MEMORY. */
rbkv_status rbkv_state_restore(rbkv_state* s, int64_t uid, int32_t* ids, int32_t cap,
                               int32_t* n);

#ifdef __cplusplus
}
#endif

#endif /* RBKV_STATE_H */
