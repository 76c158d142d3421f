"""Plain CPU model of the KV block allocator, the sequence ledger and a multi-step
serving loop over a per-sequence KV history.

TEST INFRASTRUCTURE ONLY (see the package docstring): only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use it.  It
shares no code or constants with the library: verdicts are strings and argument
errors are exceptions here.

Sources, by page title and section:

* "DeepSpeed Inference v2 source tour" (pyshine.com/deepspeed-2), section "The front
  desk: put, query, can_schedule": the ledger fixes a cap on tracked sequences; a
  sequence keeps only integer block ids; the block allocator hands out free indices and
  takes them back and is the whole memory manager; can_schedule checks the candidates
  against the tracked-sequence cap and the free-block count and returns a verdict
  rather than raising; query answers, for a budget of new tokens and blocks, whether a
  sequence can run; flush retires a sequence and gives its blocks back.
* same page, overview list: sequences are created on first use; a descriptor's block
  list grows by extend_kv_cache; same page, section "Policies, containers, and a
  metaclass that checks your weights": blocks are requested before each forward pass
  from the sequence's KV requirements.
* "DeepSpeed-Inference and DeepSpeed-MII" (jwzheng96.github.io), section 10.10: the
  ledger records which sequence holds which blocks and exposes the free-block count.
* "DeepSpeed-MII source tour" (pyshine.com/deepspeed-mii), section "Inside the Ragged
  Batching Engine": each step of the serving loop flushes finished requests, feeds new
  tokens to the engine and schedules the next batch.

Readings (each a choice where the pages are silent; the library states the same ones):

1. A sequence holding ``seen`` cached and ``n`` in-flight tokens owns exactly
   ceil((seen + n) / bs) blocks; blocks are added before the pass, ``seen`` grows after.
2. Which free ids the allocator returns is not fixed by the pages.  This model hands
   out the smallest free ids; the library may choose others, so only counts and
   validity are comparable.
3. An over-large allocation or a bad free fails as a whole and changes nothing.
4. can_schedule's verdict order: batch sequence count, batch token count, then per
   candidate in batch order: tracked-sequence cap (new uids), per-sequence context
   cap, running block demand against the free-block count.
5. The per-sequence context cap (``max_context``) and the batch caps (``max_seqs``,
   ``max_tokens``) are the engine limits of the tutorial chapter, section 10.3.

Parity status: pinned by ``tests/golden/ledger_walk.txt`` (hand-derived from the
definitions above), brute-force KV requirements, and conservation invariants
(``tests/test_state_oracle_pins.py``).  The serving loop's attention is the plain
per-sequence definition over a contiguous history, pinned through the functions of
``oracle.ragged_attention`` it calls.
"""
from __future__ import annotations

import numpy as np

from .ragged_attention import f64_to_storage, rope_angles, rotate, sequence_attention, \
    storage_to_f64

VERDICTS = ("ok", "engine_seq_limit", "kv_limit", "batch_seq_limit", "batch_token_limit",
            "seq_token_limit")


class OracleBlocksError(Exception):
    """Allocation or free refused (too few free ids, id not allocated)."""


def ceil_div(a: int, b: int) -> int:
    return -(-int(a) // int(b))


def kv_requirements(seen: int, held: int, max_new_tokens: int, max_new_blocks: int,
                    block_size: int):
    """(tokens, blocks): how many of ``max_new_tokens`` fit when at most
    ``max_new_blocks`` blocks can be added to the ``held`` ones, and how many blocks
    those tokens need.  Plain definition: the blocks needed for seen + m tokens are
    ceil((seen + m) / bs) - held (never below 0); take the largest m <= max_new_tokens
    whose need fits the budget."""
    if max_new_tokens < 0 or max_new_blocks < 0:
        raise ValueError("negative budget")

    def need(m):
        return max(0, ceil_div(seen + m, block_size) - held)

    m = max_new_tokens
    while m > 0 and need(m) > max_new_blocks:  # need() never decreases as m grows
        m -= 1
    return m, need(m)


class BlockAllocator:
    """Set of free block ids; allocate hands out the smallest free ids."""

    def __init__(self, num_blocks: int):
        if num_blocks < 1:
            raise ValueError("num_blocks < 1")
        self.num_blocks = int(num_blocks)
        self.free = set(range(self.num_blocks))

    @property
    def free_blocks(self) -> int:
        return len(self.free)

    def allocate(self, n: int):
        if n < 0:
            raise ValueError("n < 0")
        if n > len(self.free):
            raise OracleBlocksError(f"{n} blocks asked, {len(self.free)} free")
        ids = sorted(self.free)[:n]
        self.free.difference_update(ids)
        return ids

    def release(self, ids):
        ids = [int(i) for i in ids]
        if len(set(ids)) != len(ids):
            raise OracleBlocksError("id listed twice")
        for i in ids:
            if i < 0 or i >= self.num_blocks or i in self.free:
                raise OracleBlocksError(f"id {i} is not allocated")
        self.free.update(ids)


class StateManager:
    """Ledger of live sequences: uid -> {seen, in_flight, blocks}."""

    def __init__(self, *, num_blocks, block_size, max_tracked_seqs, max_seqs, max_tokens,
                 max_context):
        self.block_size = int(block_size)
        self.max_tracked_seqs = int(max_tracked_seqs)
        self.max_seqs = int(max_seqs)
        self.max_tokens = int(max_tokens)
        self.max_context = int(max_context)
        self.alloc = BlockAllocator(num_blocks)
        self.seqs = {}
        self.open = None  # list of uids of the open batch, in put order

    # -- queries ------------------------------------------------------------------
    @property
    def free_blocks(self) -> int:
        return self.alloc.free_blocks

    @property
    def n_tracked(self) -> int:
        return len(self.seqs)

    def sequence(self, uid):
        q = self.seqs.get(uid)
        if q is None:
            return None
        return q["seen"], q["in_flight"], len(q["blocks"])

    def _cached_and_held(self, uid):
        q = self.seqs.get(uid)
        if q is None:
            return 0, 0
        return q["seen"] + q["in_flight"], len(q["blocks"])

    def query(self, uid, max_new_tokens, max_new_blocks):
        if self.seqs.get(uid, {}).get("offloaded"):
            raise ValueError("an offloaded sequence must be restored first")
        cached, held = self._cached_and_held(uid)
        return kv_requirements(cached, held, max_new_tokens, max_new_blocks, self.block_size)

    def can_schedule(self, uids, n_new) -> str:
        uids, n_new = [int(u) for u in uids], [int(n) for n in n_new]
        if len(uids) != len(n_new) or any(n < 1 for n in n_new):
            raise ValueError("bad token counts")
        if len(set(uids)) != len(uids):
            raise ValueError("uid listed twice")
        if any(self.seqs.get(u, {}).get("offloaded") for u in uids):
            raise ValueError("an offloaded sequence must be restored first")
        if len(uids) > self.max_seqs:
            return "batch_seq_limit"
        if sum(n_new) > self.max_tokens:
            return "batch_token_limit"
        tracked, demand = self.n_tracked, 0
        for u, n in zip(uids, n_new):
            if u not in self.seqs:
                tracked += 1
                if tracked > self.max_tracked_seqs:
                    return "engine_seq_limit"
            cached, held = self._cached_and_held(u)
            if cached + n > self.max_context:
                return "seq_token_limit"
            demand += max(0, ceil_div(cached + n, self.block_size) - held)
            if demand > self.free_blocks:
                return "kv_limit"
        return "ok"

    def compose(self, uids, pending, token_budget):
        """Dynamic SplitFuse: the next batch [(uid, tokens)] from a queue of candidates
        (uid, pending tokens), mixing decodes and prefill chunks and cutting a prompt
        that does not fit into a chunk of what is left.

        Steps (the reading of the pages' idea; nothing here is changed):
        1. budget = min(token_budget, max_tokens); the free blocks and tracked slots
           not yet promised start at the ledger's counts;
        2. walk the queue in order taking only single-token candidates (decodes), then
           walk it again taking the longer ones (prefills);
        3. stop a walk when max_seqs candidates are chosen or the budget is spent;
        4. a new uid needs an unpromised tracked slot, else it is skipped;
        5. offer min(pending, budget left, max_context - cached) tokens and cut the offer
           to what the unpromised free blocks can hold (``kv_requirements``); skip the
           candidate if nothing is left, else choose it and promise its tokens, blocks
           and (if new) its slot.
        """
        uids, pending = [int(u) for u in uids], [int(p) for p in pending]
        if int(token_budget) < 1 or any(p < 1 for p in pending):
            raise ValueError("bad budget or pending count")
        if len(set(uids)) != len(uids):
            raise ValueError("uid listed twice")
        if any(self.seqs.get(u, {}).get("offloaded") for u in uids):
            raise ValueError("an offloaded sequence must be restored first")
        left = min(int(token_budget), self.max_tokens)
        free_left = self.free_blocks
        tracked = self.n_tracked
        chosen = []
        for decodes in (True, False):
            for u, p in zip(uids, pending):
                if len(chosen) == self.max_seqs or left == 0:
                    break
                if (p == 1) != decodes:
                    continue
                is_new = u not in self.seqs
                if is_new and tracked >= self.max_tracked_seqs:
                    continue
                cached, held = self._cached_and_held(u)
                want = min(p, left, self.max_context - cached)
                if want <= 0:
                    continue
                tokens, blocks = kv_requirements(cached, held, want, free_left,
                                                 self.block_size)
                if tokens == 0:
                    continue
                chosen.append((u, tokens))
                left -= tokens
                free_left -= blocks
                tracked += is_new
        return chosen

    # -- mutations ----------------------------------------------------------------
    def put(self, uids, n_new) -> str:
        if self.open is not None:
            raise ValueError("a batch is already open")
        verdict = self.can_schedule(uids, n_new)
        if verdict != "ok":
            return verdict
        for u, n in zip(uids, n_new):
            u, n = int(u), int(n)
            q = self.seqs.setdefault(u, {"seen": 0, "in_flight": 0, "blocks": []})
            extra = ceil_div(q["seen"] + n, self.block_size) - len(q["blocks"])
            if extra > 0:
                q["blocks"].extend(self.alloc.allocate(extra))
            q["in_flight"] = n
        self.open = [int(u) for u in uids]
        return "ok"

    def batch(self):
        """(n_new, seen, block lists) of the open batch in put order."""
        if self.open is None:
            raise ValueError("no open batch")
        qs = [self.seqs[u] for u in self.open]
        return ([q["in_flight"] for q in qs], [q["seen"] for q in qs],
                [list(q["blocks"]) for q in qs])

    def post_forward(self):
        if self.open is None:
            raise ValueError("no open batch")
        for u in self.open:
            q = self.seqs[u]
            q["seen"] += q["in_flight"]
            q["in_flight"] = 0
        self.open = None

    def flush(self, uid):
        uid = int(uid)
        q = self.seqs.get(uid)
        if q is None:
            raise ValueError(f"uid {uid} not tracked")
        if self.open is not None and uid in self.open:
            raise ValueError(f"uid {uid} is in the open batch")
        self.alloc.release(q["blocks"])
        del self.seqs[uid]

    def offload(self, uid):
        """Give up the blocks of a sequence (returned in key order) and keep its place and
        cached count; it must be restored before it runs again."""
        uid = int(uid)
        q = self.seqs.get(uid)
        if q is None or q.get("offloaded") or (self.open is not None and uid in self.open):
            raise ValueError(f"uid {uid} cannot be offloaded")
        ids = list(q["blocks"])
        self.alloc.release(ids)
        q["blocks"] = []
        q["offloaded"] = True
        return ids

    def restore(self, uid):
        """New blocks, ceil(cached / bs) of them, for an offloaded sequence (key order)."""
        uid = int(uid)
        q = self.seqs.get(uid)
        if q is None or not q.get("offloaded"):
            raise ValueError(f"uid {uid} is not offloaded")
        ids = self.alloc.allocate(ceil_div(q["seen"], self.block_size))
        q["blocks"] = list(ids)
        q["offloaded"] = False
        return ids


class ServingLoop:
    """Attention of a multi-step serving loop, computed from each sequence's own
    contiguous history of rotated keys and raw values (no blocks at all).

    ``step`` takes the batch (uids with their new-token counts, in batch order) and the
    fused new rows ``[T][Hq + 2 Hkv][d]`` in the storage dtype, rotates each token's Q
    and K at its absolute position (its sequence's cached count plus its index in the
    chunk), rounds rotated K, raw V and rotated Q to the storage dtype where the pass
    stores them, appends K and V to the history and returns the causal attention of
    the new tokens [T][Hq][d] in float64.  ``flush`` forgets a sequence.
    """

    def __init__(self, *, n_q_heads, n_kv_heads, head_dim, rope_base, dtype):
        self.Hq, self.Hkv, self.d = int(n_q_heads), int(n_kv_heads), int(head_dim)
        self.rope_base = float(rope_base)
        self.dtype = dtype
        self.K, self.V = {}, {}  # uid -> float64 [L][Hkv][d]

    def seen(self, uid) -> int:
        return 0 if uid not in self.K else int(self.K[uid].shape[0])

    def step(self, uids, n_new, qkv):
        x = storage_to_f64(np.asarray(qkv), self.dtype)
        T = x.shape[0]
        if int(sum(int(n) for n in n_new)) != T:
            raise ValueError("token count mismatch")
        Hq, Hkv, d = self.Hq, self.Hkv, self.d
        out = np.empty((T, Hq, d), dtype=np.float64)
        t0 = 0
        for u, n in zip(uids, n_new):
            u, n = int(u), int(n)
            s = self.seen(u)
            pos = np.arange(s, s + n)
            q, k, v = x[t0:t0 + n, :Hq], x[t0:t0 + n, Hq:Hq + Hkv], x[t0:t0 + n, Hq + Hkv:]
            if self.rope_base > 0:
                ang = rope_angles(pos, d, self.rope_base)[:, None, :]
                q, k = rotate(q, ang), rotate(k, ang)
            q = storage_to_f64(f64_to_storage(q, self.dtype), self.dtype)
            k = storage_to_f64(f64_to_storage(k, self.dtype), self.dtype)
            K = k if s == 0 else np.concatenate([self.K[u], k], axis=0)
            V = v if s == 0 else np.concatenate([self.V[u], v], axis=0)
            self.K[u], self.V[u] = K, V
            out[t0:t0 + n] = sequence_attention(q, K, V, pos)
            t0 += n
        return out

    def flush(self, uid):
        self.K.pop(uid, None)
        self.V.pop(uid, None)
