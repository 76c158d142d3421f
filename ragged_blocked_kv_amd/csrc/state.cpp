// Host-side KV block allocator and sequence ledger (declared in rbkv_state.h).
//
// The ledger tracks, per live sequence, its cached token count and the ids of the pool
// blocks holding its keys and values; the allocator owns the free ids.  After creation
// the per-pass calls (can_schedule, put, batch, post_forward, flush) allocate host
// memory only when a sequence's block list outgrows its capacity, and every such
// allocation happens before any state changes, so a failed allocation leaves the
// object as it was.
#include <stdint.h>

#include <algorithm>
#include <new>
#include <vector>

#include "rbkv_state.h"

namespace {

constexpr int32_t kMaxBlocks = 1 << 26;
constexpr int32_t kMaxTracked = 65536;
constexpr int32_t kMaxBatchSeqs = 65536;
constexpr int32_t kMaxTokens = 1 << 20;
constexpr int32_t kMaxBlockSize = 4096;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// splitmix64 finaliser: spreads consecutive uids over the table.
uint64_t mix(uint64_t x) {
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}

// Open-addressing uid -> slot map with linear probing and backward-shift deletion, sized
// once (load factor <= 1/2), so lookups, inserts and erases never allocate.
class UidMap {
 public:
  void init(int32_t max_entries) {
    size_t cap = 16;
    while (cap < 2 * (size_t)max_entries) cap <<= 1;
    keys_.assign(cap, 0);
    vals_.assign(cap, -1);
    mask_ = cap - 1;
  }
  int32_t find(int64_t uid) const {
    for (size_t i = mix((uint64_t)uid) & mask_;; i = (i + 1) & mask_) {
      if (vals_[i] < 0) return -1;
      if (keys_[i] == uid) return vals_[i];
    }
  }
  void insert(int64_t uid, int32_t slot) {  // uid must be absent
    size_t i = mix((uint64_t)uid) & mask_;
    while (vals_[i] >= 0) i = (i + 1) & mask_;
    keys_[i] = uid;
    vals_[i] = slot;
  }
  void erase(int64_t uid) {  // uid must be present
    size_t i = mix((uint64_t)uid) & mask_;
    while (keys_[i] != uid || vals_[i] < 0) i = (i + 1) & mask_;
    // Shift later members of the probe run back into the hole when their home position
    // does not lie cyclically in (hole, j].
    size_t hole = i;
    for (size_t j = (hole + 1) & mask_; vals_[j] >= 0; j = (j + 1) & mask_) {
      const size_t home = mix((uint64_t)keys_[j]) & mask_;
      const bool stays = hole <= j ? (hole < home && home <= j) : (hole < home || home <= j);
      if (stays) continue;
      keys_[hole] = keys_[j];
      vals_[hole] = vals_[j];
      hole = j;
    }
    vals_[hole] = -1;
  }

 private:
  std::vector<int64_t> keys_;
  std::vector<int32_t> vals_;
  size_t mask_ = 0;
};

}  // namespace

// ---------------------------------------------------------------------------------------
// Allocator: a LIFO stack of free ids plus a per-id "allocated" flag for checking frees.
// ---------------------------------------------------------------------------------------

struct rbkv_allocator {
  int32_t num_blocks = 0;
  std::vector<int32_t> free_ids;  // top of the stack is the back
  std::vector<uint8_t> allocated;
  std::vector<uint32_t> seen_in_call;  // duplicate detection inside one free call
  uint32_t call = 0;

  void init(int32_t n) {
    num_blocks = n;
    free_ids.resize((size_t)n);
    for (int32_t i = 0; i < n; ++i) free_ids[(size_t)i] = n - 1 - i;  // pops 0, 1, 2, ...
    allocated.assign((size_t)n, 0);
    seen_in_call.assign((size_t)n, 0);
    call = 0;
  }
  int32_t n_free() const { return (int32_t)free_ids.size(); }
  // Caller has checked n <= n_free().
  void take(int32_t n, int32_t* out) {
    for (int32_t k = 0; k < n; ++k) {
      const int32_t id = free_ids.back();
      free_ids.pop_back();
      allocated[(size_t)id] = 1;
      out[k] = id;
    }
  }
  bool check_free(int32_t n, const int32_t* ids) {
    if (++call == 0) {  // wrapped: clear the stamps
      std::fill(seen_in_call.begin(), seen_in_call.end(), 0u);
      call = 1;
    }
    for (int32_t k = 0; k < n; ++k) {
      const int32_t id = ids[k];
      if (id < 0 || id >= num_blocks || !allocated[(size_t)id]) return false;
      if (seen_in_call[(size_t)id] == call) return false;
      seen_in_call[(size_t)id] = call;
    }
    return true;
  }
  // Caller has run check_free.  Pushed in reverse so a following take returns them in
  // the order they were given back.  free_ids has capacity num_blocks: never allocates.
  void give(int32_t n, const int32_t* ids) {
    for (int32_t k = n - 1; k >= 0; --k) {
      allocated[(size_t)ids[k]] = 0;
      free_ids.push_back(ids[k]);
    }
  }
};

// ---------------------------------------------------------------------------------------
// Ledger
// ---------------------------------------------------------------------------------------

namespace {

struct Seq {
  int64_t uid = 0;
  int32_t seen = 0;       // tokens cached in the pool
  int32_t in_flight = 0;  // tokens of the open batch (0 when not in it)
  bool offloaded = false;  // blocks given up; contents held by the caller on the host
  std::vector<int32_t> blocks;
};

}  // namespace

struct rbkv_state {
  rbkv_state_config cfg{};
  rbkv_allocator alloc;
  std::vector<Seq> slots;
  std::vector<int32_t> free_slots;  // stack
  UidMap index;
  bool open = false;
  // The open batch, in put order.
  std::vector<int32_t> b_slot, b_new, b_seen, b_len;
  std::vector<const int32_t*> b_ptr;
  // Scratch of the batch checks (sized at creation).
  std::vector<uint32_t> slot_stamp;
  uint32_t stamp = 0;
  std::vector<int64_t> new_uids;
  std::vector<int32_t> looked_up;  // slot of each candidate, -1 when new

  int32_t n_tracked() const { return cfg.max_tracked_seqs - (int32_t)free_slots.size(); }

  // Cached (seen + in-flight) and held blocks of the sequence in `slot` (-1: new).
  void cached_held(int32_t slot, int64_t* cached, int64_t* held) const {
    if (slot < 0) {
      *cached = 0;
      *held = 0;
    } else {
      const Seq& q = slots[(size_t)slot];
      *cached = (int64_t)q.seen + q.in_flight;
      *held = (int64_t)q.blocks.size();
    }
  }

  // Look up n (<= kMaxBatchSeqs) uids into looked_up[0..n-1]; false if one is listed
  // twice or a count is below 1.
  bool lookup(int32_t n, const int64_t* uids, const int32_t* counts) {
    if (++stamp == 0) {
      std::fill(slot_stamp.begin(), slot_stamp.end(), 0u);
      stamp = 1;
    }
    new_uids.clear();
    for (int32_t i = 0; i < n; ++i) {
      if (counts[i] < 1) return false;
      const int32_t slot = index.find(uids[i]);
      looked_up[(size_t)i] = slot;
      if (slot >= 0) {
        if (slots[(size_t)slot].offloaded) return false;  // must be restored first
        if (slot_stamp[(size_t)slot] == stamp) return false;  // listed twice
        slot_stamp[(size_t)slot] = stamp;
      } else {
        new_uids.push_back(uids[i]);  // capacity kMaxBatchSeqs: no allocation
      }
    }
    if (new_uids.size() > 1) {
      std::sort(new_uids.begin(), new_uids.end());
      if (std::adjacent_find(new_uids.begin(), new_uids.end()) != new_uids.end())
        return false;
    }
    return true;
  }

  // Validation and verdict shared by can_schedule and put.  Fills looked_up[0..n-1].
  rbkv_status evaluate(int32_t n, const int64_t* uids, const int32_t* n_new, int32_t* verdict) {
    if (n < 0 || !verdict) return RBKV_ERR_INVALID_ARG;
    if (n > 0 && (!uids || !n_new)) return RBKV_ERR_INVALID_ARG;
    if (n > kMaxBatchSeqs) {  // scratch is sized for this; such a batch is over max_seqs
      for (int32_t i = 0; i < n; ++i)
        if (n_new[i] < 1) return RBKV_ERR_INVALID_ARG;
      *verdict = RBKV_SCHED_BATCH_SEQ_LIMIT;
      return RBKV_OK;
    }
    if (!lookup(n, uids, n_new)) return RBKV_ERR_INVALID_ARG;
    int64_t tokens = 0;
    for (int32_t i = 0; i < n; ++i) tokens += n_new[i];
    if (n > cfg.max_seqs) {
      *verdict = RBKV_SCHED_BATCH_SEQ_LIMIT;
      return RBKV_OK;
    }
    if (tokens > cfg.max_tokens) {
      *verdict = RBKV_SCHED_BATCH_TOKEN_LIMIT;
      return RBKV_OK;
    }
    int64_t tracked = n_tracked(), need_total = 0;
    const int64_t free_blocks = alloc.n_free();
    for (int32_t i = 0; i < n; ++i) {
      const int32_t slot = looked_up[(size_t)i];
      int64_t cached, held;
      cached_held(slot, &cached, &held);
      if (slot < 0 && ++tracked > cfg.max_tracked_seqs) {
        *verdict = RBKV_SCHED_ENGINE_SEQ_LIMIT;
        return RBKV_OK;
      }
      const int64_t total = cached + n_new[i];
      if (total > cfg.max_context) {
        *verdict = RBKV_SCHED_SEQ_TOKEN_LIMIT;
        return RBKV_OK;
      }
      need_total += std::max<int64_t>(0, cdiv(total, cfg.block_size) - held);
      if (need_total > free_blocks) {
        *verdict = RBKV_SCHED_KV_LIMIT;
        return RBKV_OK;
      }
    }
    *verdict = RBKV_SCHED_OK;
    return RBKV_OK;
  }
};

extern "C" {

rbkv_status rbkv_allocator_create(int32_t num_blocks, rbkv_allocator** out) {
  if (!out || num_blocks < 1) return RBKV_ERR_INVALID_ARG;
  if (num_blocks > kMaxBlocks) return RBKV_ERR_UNSUPPORTED;
  try {
    rbkv_allocator* a = new rbkv_allocator();
    try {
      a->init(num_blocks);
    } catch (...) {
      delete a;
      throw;
    }
    *out = a;
  } catch (const std::bad_alloc&) {
    return RBKV_ERR_HOST_MEMORY;
  }
  return RBKV_OK;
}

rbkv_status rbkv_allocator_destroy(rbkv_allocator* a) {
  delete a;
  return RBKV_OK;
}

rbkv_status rbkv_allocator_allocate(rbkv_allocator* a, int32_t n, int32_t* ids) {
  if (!a || n < 0 || (n > 0 && !ids)) return RBKV_ERR_INVALID_ARG;
  if (n > a->n_free()) return RBKV_ERR_BLOCKS;
  a->take(n, ids);
  return RBKV_OK;
}

rbkv_status rbkv_allocator_free(rbkv_allocator* a, int32_t n, const int32_t* ids) {
  if (!a || n < 0 || (n > 0 && !ids)) return RBKV_ERR_INVALID_ARG;
  if (!a->check_free(n, ids)) return RBKV_ERR_BLOCKS;
  a->give(n, ids);
  return RBKV_OK;
}

rbkv_status rbkv_allocator_free_count(const rbkv_allocator* a, int32_t* n) {
  if (!a || !n) return RBKV_ERR_INVALID_ARG;
  *n = a->n_free();
  return RBKV_OK;
}

rbkv_status rbkv_state_create(const rbkv_state_config* cfg, rbkv_state** out) {
  if (!cfg || !out) return RBKV_ERR_INVALID_ARG;
  const rbkv_state_config& c = *cfg;
  if (c.num_blocks < 1 || c.block_size < 1 || c.max_tracked_seqs < 1 || c.max_seqs < 1 ||
      c.max_tokens < 1 || c.max_context < 1)
    return RBKV_ERR_INVALID_ARG;
  if (c.num_blocks > kMaxBlocks || c.max_tracked_seqs > kMaxTracked ||
      c.max_seqs > kMaxBatchSeqs || c.max_tokens > kMaxTokens || c.block_size > kMaxBlockSize)
    return RBKV_ERR_UNSUPPORTED;
  rbkv_state* s = nullptr;
  try {
    s = new rbkv_state();
    s->cfg = c;
    s->alloc.init(c.num_blocks);
    s->slots.resize((size_t)c.max_tracked_seqs);
    s->free_slots.resize((size_t)c.max_tracked_seqs);
    for (int32_t i = 0; i < c.max_tracked_seqs; ++i)
      s->free_slots[(size_t)i] = c.max_tracked_seqs - 1 - i;
    s->index.init(c.max_tracked_seqs);
    const size_t nb = (size_t)c.max_seqs;
    s->b_slot.reserve(nb);
    s->b_new.reserve(nb);
    s->b_seen.reserve(nb);
    s->b_len.reserve(nb);
    s->b_ptr.reserve(nb);
    s->slot_stamp.assign((size_t)c.max_tracked_seqs, 0u);
    s->new_uids.reserve((size_t)kMaxBatchSeqs);
    s->looked_up.resize((size_t)kMaxBatchSeqs);
  } catch (const std::bad_alloc&) {
    delete s;
    return RBKV_ERR_HOST_MEMORY;
  }
  *out = s;
  return RBKV_OK;
}

rbkv_status rbkv_state_destroy(rbkv_state* s) {
  delete s;
  return RBKV_OK;
}

rbkv_status rbkv_state_counts(const rbkv_state* s, int32_t* free_blocks, int32_t* n_tracked) {
  if (!s) return RBKV_ERR_INVALID_ARG;
  if (free_blocks) *free_blocks = s->alloc.n_free();
  if (n_tracked) *n_tracked = s->n_tracked();
  return RBKV_OK;
}

rbkv_status rbkv_state_sequence(const rbkv_state* s, int64_t uid, int32_t* seen,
                                int32_t* in_flight, int32_t* n_blocks) {
  if (!s) return RBKV_ERR_INVALID_ARG;
  const int32_t slot = s->index.find(uid);
  if (slot < 0) return RBKV_ERR_INVALID_ARG;
  const Seq& q = s->slots[(size_t)slot];
  if (seen) *seen = q.seen;
  if (in_flight) *in_flight = q.in_flight;
  if (n_blocks) *n_blocks = (int32_t)q.blocks.size();
  return RBKV_OK;
}

rbkv_status rbkv_state_block_ids(const rbkv_state* s, int64_t uid, int32_t* ids, int32_t cap,
                                 int32_t* n) {
  if (!s || !n || cap < 0 || (cap > 0 && !ids)) return RBKV_ERR_INVALID_ARG;
  const int32_t slot = s->index.find(uid);
  if (slot < 0) return RBKV_ERR_INVALID_ARG;
  const Seq& q = s->slots[(size_t)slot];
  const int32_t held = (int32_t)q.blocks.size();
  if (cap < held) return RBKV_ERR_INVALID_ARG;
  std::copy(q.blocks.begin(), q.blocks.end(), ids);
  *n = held;
  return RBKV_OK;
}

rbkv_status rbkv_state_query(const rbkv_state* s, int64_t uid, int32_t max_new_tokens,
                             int32_t max_new_blocks, int32_t* tokens, int32_t* blocks) {
  if (!s || !tokens || !blocks || max_new_tokens < 0 || max_new_blocks < 0)
    return RBKV_ERR_INVALID_ARG;
  const int32_t slot = s->index.find(uid);
  if (slot >= 0 && s->slots[(size_t)slot].offloaded) return RBKV_ERR_INVALID_ARG;
  int64_t cached, held;
  s->cached_held(slot, &cached, &held);
  const int64_t bs = s->cfg.block_size;
  const int64_t need = std::max<int64_t>(0, cdiv(cached + max_new_tokens, bs) - held);
  if (need <= max_new_blocks) {
    *tokens = max_new_tokens;
    *blocks = (int32_t)need;
  } else {
    *tokens = (int32_t)((held + max_new_blocks) * bs - cached);
    *blocks = max_new_blocks;
  }
  return RBKV_OK;
}

rbkv_status rbkv_state_compose(const rbkv_state* s, int32_t n, const int64_t* uids,
                               const int32_t* pending, int32_t token_budget, int32_t* S,
                               int64_t* out_uids, int32_t* out_n) {
  if (!s || !S || n < 0 || token_budget < 1) return RBKV_ERR_INVALID_ARG;
  if (n > 0 && (!uids || !pending || !out_uids || !out_n)) return RBKV_ERR_INVALID_ARG;
  if (n > kMaxBatchSeqs) return RBKV_ERR_CAPACITY;
  // Only scratch members change; the ledger itself is untouched.
  rbkv_state* m = const_cast<rbkv_state*>(s);
  if (!m->lookup(n, uids, pending)) return RBKV_ERR_INVALID_ARG;
  const rbkv_state_config& c = s->cfg;
  const int64_t bs = c.block_size;
  int64_t left = std::min(token_budget, c.max_tokens);
  int64_t free_left = s->alloc.n_free();
  int64_t tracked = s->n_tracked();
  int32_t count = 0;
  for (int pass = 0; pass < 2; ++pass) {
    for (int32_t i = 0; i < n && count < c.max_seqs && left > 0; ++i) {
      if ((pending[i] == 1) != (pass == 0)) continue;
      const int32_t slot = m->looked_up[(size_t)i];
      if (slot < 0 && tracked >= c.max_tracked_seqs) continue;
      int64_t cached, held;
      s->cached_held(slot, &cached, &held);
      const int64_t want = std::min<int64_t>({(int64_t)pending[i], left, c.max_context - cached});
      if (want <= 0) continue;
      int64_t tokens = want, blocks = std::max<int64_t>(0, cdiv(cached + want, bs) - held);
      if (blocks > free_left) {  // cut to what the unpromised free blocks can hold
        tokens = (held + free_left) * bs - cached;
        blocks = free_left;
      }
      if (tokens <= 0) continue;
      out_uids[count] = uids[i];
      out_n[count] = (int32_t)tokens;
      ++count;
      left -= tokens;
      free_left -= blocks;
      if (slot < 0) ++tracked;
    }
  }
  *S = count;
  return RBKV_OK;
}

rbkv_status rbkv_state_can_schedule(const rbkv_state* s, int32_t n, const int64_t* uids,
                                    const int32_t* n_new, int32_t* verdict) {
  if (!s) return RBKV_ERR_INVALID_ARG;
  // Only scratch members change; the ledger itself is untouched.
  return const_cast<rbkv_state*>(s)->evaluate(n, uids, n_new, verdict);
}

rbkv_status rbkv_state_put(rbkv_state* s, int32_t n, const int64_t* uids, const int32_t* n_new,
                           int32_t* verdict) {
  if (!s || s->open) return RBKV_ERR_INVALID_ARG;
  rbkv_status st = s->evaluate(n, uids, n_new, verdict);
  if (st != RBKV_OK || *verdict != RBKV_SCHED_OK) return st;
  const int32_t bs = s->cfg.block_size;
  // Phase 1 (may throw, changes no state): give each sequence's block list room for its
  // new blocks.  New sequences take free slots from the top of the stack in order.
  try {
    size_t next_new = 0;
    for (int32_t i = 0; i < n; ++i) {
      int32_t slot = s->looked_up[(size_t)i];
      int64_t cached = 0;
      if (slot < 0) {
        slot = s->free_slots[s->free_slots.size() - 1 - next_new++];
      } else {
        cached = s->slots[(size_t)slot].seen;
      }
      s->slots[(size_t)slot].blocks.reserve((size_t)cdiv(cached + n_new[i], bs));
    }
  } catch (const std::bad_alloc&) {
    return RBKV_ERR_HOST_MEMORY;
  }
  // Phase 2 (no allocation): create, extend, record.
  s->b_slot.clear();
  s->b_new.clear();
  s->b_seen.clear();
  s->b_len.clear();
  s->b_ptr.clear();
  for (int32_t i = 0; i < n; ++i) {
    int32_t slot = s->looked_up[(size_t)i];
    if (slot < 0) {
      slot = s->free_slots.back();
      s->free_slots.pop_back();
      Seq& q = s->slots[(size_t)slot];
      q.uid = uids[i];
      q.seen = 0;
      q.in_flight = 0;
      q.offloaded = false;
      q.blocks.clear();
      s->index.insert(uids[i], slot);
    }
    Seq& q = s->slots[(size_t)slot];
    const int32_t need = (int32_t)cdiv((int64_t)q.seen + n_new[i], bs) - (int32_t)q.blocks.size();
    if (need > 0) {
      const size_t old = q.blocks.size();
      q.blocks.resize(old + (size_t)need);  // within the reserved capacity
      s->alloc.take(need, q.blocks.data() + old);
    }
    q.in_flight = n_new[i];
    s->b_slot.push_back(slot);
    s->b_new.push_back(n_new[i]);
    s->b_seen.push_back(q.seen);
    s->b_len.push_back((int32_t)q.blocks.size());
    s->b_ptr.push_back(q.blocks.data());
  }
  s->open = true;
  return RBKV_OK;
}

rbkv_status rbkv_state_batch(const rbkv_state* s, int32_t* S, const int32_t** n_new,
                             const int32_t** seen, const int32_t* const** block_ids,
                             const int32_t** n_block_ids) {
  if (!s || !s->open) return RBKV_ERR_INVALID_ARG;
  if (S) *S = (int32_t)s->b_slot.size();
  if (n_new) *n_new = s->b_new.data();
  if (seen) *seen = s->b_seen.data();
  if (block_ids) *block_ids = s->b_ptr.data();
  if (n_block_ids) *n_block_ids = s->b_len.data();
  return RBKV_OK;
}

rbkv_status rbkv_state_finalize(const rbkv_state* s, const rbkv_shape* shape,
                                void* host_pinned, size_t host_pinned_bytes, void* dev_meta,
                                size_t dev_meta_bytes, void* stream, rbkv_batch* out) {
  if (!s || !s->open || !shape) return RBKV_ERR_INVALID_ARG;
  if (shape->num_blocks != s->cfg.num_blocks || shape->block_size != s->cfg.block_size)
    return RBKV_ERR_INVALID_ARG;
  return ragged_batch_finalize(shape, (int32_t)s->b_slot.size(), s->b_new.data(),
                               s->b_seen.data(), s->b_ptr.data(), s->b_len.data(), host_pinned,
                               host_pinned_bytes, dev_meta, dev_meta_bytes, stream, out);
}

rbkv_status rbkv_state_post_forward(rbkv_state* s) {
  if (!s || !s->open) return RBKV_ERR_INVALID_ARG;
  for (const int32_t slot : s->b_slot) {
    Seq& q = s->slots[(size_t)slot];
    q.seen += q.in_flight;
    q.in_flight = 0;
  }
  s->open = false;
  return RBKV_OK;
}

rbkv_status rbkv_state_flush(rbkv_state* s, int64_t uid) {
  if (!s) return RBKV_ERR_INVALID_ARG;
  const int32_t slot = s->index.find(uid);
  if (slot < 0) return RBKV_ERR_INVALID_ARG;
  Seq& q = s->slots[(size_t)slot];
  if (s->open && q.in_flight > 0) return RBKV_ERR_INVALID_ARG;
  s->alloc.give((int32_t)q.blocks.size(), q.blocks.data());
  if (q.blocks.capacity() > 4096) {
    std::vector<int32_t>().swap(q.blocks);
  } else {
    q.blocks.clear();
  }
  q.seen = 0;
  q.offloaded = false;
  s->index.erase(uid);
  s->free_slots.push_back(slot);  // capacity max_tracked_seqs: never allocates
  return RBKV_OK;
}

rbkv_status rbkv_state_offload(rbkv_state* s, int64_t uid, int32_t* ids, int32_t cap,
                               int32_t* n) {
  if (!s || !n || cap < 0 || (cap > 0 && !ids)) return RBKV_ERR_INVALID_ARG;
  const int32_t slot = s->index.find(uid);
  if (slot < 0) return RBKV_ERR_INVALID_ARG;
  Seq& q = s->slots[(size_t)slot];
  if (q.offloaded || (s->open && q.in_flight > 0)) return RBKV_ERR_INVALID_ARG;
  const int32_t held = (int32_t)q.blocks.size();
  if (cap < held) return RBKV_ERR_INVALID_ARG;
  std::copy(q.blocks.begin(), q.blocks.end(), ids);
  s->alloc.give(held, q.blocks.data());
  q.blocks.clear();
  q.offloaded = true;
  *n = held;
  return RBKV_OK;
}

rbkv_status rbkv_state_restore(rbkv_state* s, int64_t uid, int32_t* ids, int32_t cap,
                               int32_t* n) {
  if (!s || !n || cap < 0 || (cap > 0 && !ids)) return RBKV_ERR_INVALID_ARG;
  const int32_t slot = s->index.find(uid);
  if (slot < 0) return RBKV_ERR_INVALID_ARG;
  Seq& q = s->slots[(size_t)slot];
  if (!q.offloaded) return RBKV_ERR_INVALID_ARG;
  const int32_t need = (int32_t)cdiv(q.seen, s->cfg.block_size);
  if (cap < need) return RBKV_ERR_INVALID_ARG;
  if (need > s->alloc.n_free()) return RBKV_ERR_BLOCKS;
  try {
    q.blocks.reserve((size_t)need);
  } catch (const std::bad_alloc&) {
    return RBKV_ERR_HOST_MEMORY;
  }
  q.blocks.resize((size_t)need);
  s->alloc.take(need, q.blocks.data());
  std::copy(q.blocks.begin(), q.blocks.end(), ids);
  q.offloaded = false;
  *n = need;
  return RBKV_OK;
}

}  // extern "C"
