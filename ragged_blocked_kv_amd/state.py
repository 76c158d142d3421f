"""Python binding of librbkv's block allocator and sequence ledger (``include/rbkv_state.h``).

Argument marshalling only: the bookkeeping runs in the library's native code.  Both
classes own their native object and raise ``RbkvError`` on any non-OK status; verdicts
of the scheduling checks are returned as integers (``SCHED_*``), never raised.  No call
here needs a GPU except ``StateManager.finalize``.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np

from . import Batch, RbkvError, Shape, _ptr, _stream, check, lib

__all__ = [
    "BlockAllocator", "StateManager", "StateConfig", "SCHED_OK", "SCHED_ENGINE_SEQ_LIMIT",
    "SCHED_KV_LIMIT", "SCHED_BATCH_SEQ_LIMIT", "SCHED_BATCH_TOKEN_LIMIT",
    "SCHED_SEQ_TOKEN_LIMIT", "SCHED_NAMES",
]

SCHED_OK, SCHED_ENGINE_SEQ_LIMIT, SCHED_KV_LIMIT = 0, 1, 2
SCHED_BATCH_SEQ_LIMIT, SCHED_BATCH_TOKEN_LIMIT, SCHED_SEQ_TOKEN_LIMIT = 3, 4, 5
SCHED_NAMES = {
    SCHED_OK: "ok", SCHED_ENGINE_SEQ_LIMIT: "engine sequence limit",
    SCHED_KV_LIMIT: "kv cache limit", SCHED_BATCH_SEQ_LIMIT: "batch sequence limit",
    SCHED_BATCH_TOKEN_LIMIT: "batch token limit",
    SCHED_SEQ_TOKEN_LIMIT: "sequence token limit",
}


_I32 = ctypes.c_int32
_PI32 = ctypes.POINTER(ctypes.c_int32)
_PI64 = ctypes.POINTER(ctypes.c_int64)


class StateConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_blocks", "block_size", "max_tracked_seqs", "max_seqs", "max_tokens",
        "max_context")]


_bound = False


def _lib():
    global _bound
    L = lib()
    if not _bound:
        vp, pvp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)
        sigs = {
            "rbkv_allocator_create": [_I32, pvp],
            "rbkv_allocator_destroy": [vp],
            "rbkv_allocator_allocate": [vp, _I32, _PI32],
            "rbkv_allocator_free": [vp, _I32, _PI32],
            "rbkv_allocator_free_count": [vp, _PI32],
            "rbkv_state_create": [ctypes.POINTER(StateConfig), pvp],
            "rbkv_state_destroy": [vp],
            "rbkv_state_counts": [vp, _PI32, _PI32],
            "rbkv_state_sequence": [vp, ctypes.c_int64, _PI32, _PI32, _PI32],
            "rbkv_state_block_ids": [vp, ctypes.c_int64, _PI32, _I32, _PI32],
            "rbkv_state_query": [vp, ctypes.c_int64, _I32, _I32, _PI32, _PI32],
            "rbkv_state_can_schedule": [vp, _I32, _PI64, _PI32, _PI32],
            "rbkv_state_compose": [vp, _I32, _PI64, _PI32, _I32, _PI32, _PI64, _PI32],
            "rbkv_state_put": [vp, _I32, _PI64, _PI32, _PI32],
            "rbkv_state_batch": [vp, _PI32, ctypes.POINTER(_PI32), ctypes.POINTER(_PI32),
                                 ctypes.POINTER(ctypes.POINTER(_PI32)), ctypes.POINTER(_PI32)],
            "rbkv_state_finalize": [vp, ctypes.POINTER(Shape), vp, ctypes.c_size_t, vp,
                                    ctypes.c_size_t, vp, ctypes.POINTER(Batch)],
            "rbkv_state_post_forward": [vp],
            "rbkv_state_flush": [vp, ctypes.c_int64],
            "rbkv_state_offload": [vp, ctypes.c_int64, _PI32, _I32, _PI32],
            "rbkv_state_restore": [vp, ctypes.c_int64, _PI32, _I32, _PI32],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.restype = ctypes.c_int32
            fn.argtypes = args
        _bound = True
    return L


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


class BlockAllocator:
    """Free list over block ids 0 .. num_blocks - 1 (``rbkv_allocator_*``)."""

    def __init__(self, num_blocks: int):
        h = ctypes.c_void_p()
        check(_lib().rbkv_allocator_create(int(num_blocks), ctypes.byref(h)),
              "rbkv_allocator_create")
        self._h = h
        self.num_blocks = int(num_blocks)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            _lib().rbkv_allocator_destroy(h)
            self._h = None

    def allocate_status(self, n: int):
        """(status, ids) -- ids is an int32 array of length n (undefined on error)."""
        out = np.zeros(max(int(n), 0), dtype=np.int32)
        st = _lib().rbkv_allocator_allocate(self._h, int(n), out.ctypes.data_as(_PI32))
        return st, out

    def allocate(self, n: int) -> np.ndarray:
        st, out = self.allocate_status(n)
        check(st, "rbkv_allocator_allocate")
        return out

    def free_status(self, ids) -> int:
        a = _i32(ids)
        return _lib().rbkv_allocator_free(self._h, int(a.size), a.ctypes.data_as(_PI32))

    def free(self, ids) -> None:
        check(self.free_status(ids), "rbkv_allocator_free")

    @property
    def free_blocks(self) -> int:
        n = ctypes.c_int32()
        check(_lib().rbkv_allocator_free_count(self._h, ctypes.byref(n)),
              "rbkv_allocator_free_count")
        return n.value


class StateManager:
    """Sequence ledger with its own block allocator (``rbkv_state_*``)."""

    def __init__(self, *, num_blocks: int, block_size: int, max_tracked_seqs: int,
                 max_seqs: int, max_tokens: int, max_context: int):
        self.config = StateConfig(int(num_blocks), int(block_size), int(max_tracked_seqs),
                                  int(max_seqs), int(max_tokens), int(max_context))
        h = ctypes.c_void_p()
        check(_lib().rbkv_state_create(ctypes.byref(self.config), ctypes.byref(h)),
              "rbkv_state_create")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            _lib().rbkv_state_destroy(h)
            self._h = None

    # -- queries -------------------------------------------------------------------
    def counts(self):
        """(free_blocks, n_tracked)."""
        f, t = ctypes.c_int32(), ctypes.c_int32()
        check(_lib().rbkv_state_counts(self._h, ctypes.byref(f), ctypes.byref(t)),
              "rbkv_state_counts")
        return f.value, t.value

    @property
    def free_blocks(self) -> int:
        return self.counts()[0]

    @property
    def n_tracked(self) -> int:
        return self.counts()[1]

    def sequence(self, uid: int):
        """(seen, in_flight, n_blocks) of a tracked sequence, or None if untracked."""
        s, f, b = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        st = _lib().rbkv_state_sequence(self._h, int(uid), ctypes.byref(s), ctypes.byref(f),
                                        ctypes.byref(b))
        if st != 0:
            return None
        return s.value, f.value, b.value

    def block_ids(self, uid: int) -> np.ndarray:
        info = self.sequence(uid)
        if info is None:
            raise RbkvError(1, f"rbkv_state_block_ids: uid {uid} not tracked")
        out = np.zeros(max(info[2], 1), dtype=np.int32)
        n = ctypes.c_int32()
        check(_lib().rbkv_state_block_ids(self._h, int(uid), out.ctypes.data_as(_PI32),
                                          int(out.size), ctypes.byref(n)),
              "rbkv_state_block_ids")
        return out[:n.value].copy()

    def query_status(self, uid: int, max_new_tokens: int, max_new_blocks: int):
        """(status, tokens, blocks) -- the KV requirements of ``max_new_tokens`` more
        tokens."""
        t, b = ctypes.c_int32(), ctypes.c_int32()
        st = _lib().rbkv_state_query(self._h, int(uid), int(max_new_tokens),
                                     int(max_new_blocks), ctypes.byref(t), ctypes.byref(b))
        return st, t.value, b.value

    def query(self, uid: int, max_new_tokens: int, max_new_blocks: int):
        st, t, b = self.query_status(uid, max_new_tokens, max_new_blocks)
        check(st, "rbkv_state_query")
        return t, b

    def can_schedule_status(self, uids: Sequence[int], n_new: Sequence[int]):
        """(status, verdict)."""
        u, n = _i64(uids), _i32(n_new)
        v = ctypes.c_int32(-1)
        st = _lib().rbkv_state_can_schedule(self._h, int(u.size), u.ctypes.data_as(_PI64),
                                            n.ctypes.data_as(_PI32), ctypes.byref(v))
        return st, v.value

    def can_schedule(self, uids, n_new) -> int:
        st, v = self.can_schedule_status(uids, n_new)
        check(st, "rbkv_state_can_schedule")
        return v

    def compose_status(self, uids: Sequence[int], pending: Sequence[int], token_budget: int):
        """(status, uids, n): the Dynamic SplitFuse batch for a queue of candidates."""
        u, p = _i64(uids), _i32(pending)
        cap = max(1, min(int(u.size), int(self.config.max_seqs)))
        out_u = np.zeros(cap, dtype=np.int64)
        out_n = np.zeros(cap, dtype=np.int32)
        S = ctypes.c_int32(0)
        st = _lib().rbkv_state_compose(self._h, int(u.size), u.ctypes.data_as(_PI64),
                                       p.ctypes.data_as(_PI32), int(token_budget),
                                       ctypes.byref(S), out_u.ctypes.data_as(_PI64),
                                       out_n.ctypes.data_as(_PI32))
        return st, out_u[:S.value].copy(), out_n[:S.value].copy()

    def compose(self, uids, pending, token_budget):
        st, u, n = self.compose_status(uids, pending, token_budget)
        check(st, "rbkv_state_compose")
        return u, n

    # -- mutations -----------------------------------------------------------------
    def put_status(self, uids: Sequence[int], n_new: Sequence[int]):
        """(status, verdict)."""
        u, n = _i64(uids), _i32(n_new)
        v = ctypes.c_int32(-1)
        st = _lib().rbkv_state_put(self._h, int(u.size), u.ctypes.data_as(_PI64),
                                   n.ctypes.data_as(_PI32), ctypes.byref(v))
        return st, v.value

    def put(self, uids, n_new) -> int:
        st, v = self.put_status(uids, n_new)
        check(st, "rbkv_state_put")
        return v

    def batch(self):
        """The open batch as host arrays: (n_new, seen, [block list per sequence])."""
        S = ctypes.c_int32()
        pn, ps, pl = _PI32(), _PI32(), _PI32()
        pb = ctypes.POINTER(_PI32)()
        check(_lib().rbkv_state_batch(self._h, ctypes.byref(S), ctypes.byref(pn),
                                      ctypes.byref(ps), ctypes.byref(pb), ctypes.byref(pl)),
              "rbkv_state_batch")
        S = S.value
        n_new = np.array([pn[i] for i in range(S)], dtype=np.int32)
        seen = np.array([ps[i] for i in range(S)], dtype=np.int32)
        lens = [pl[i] for i in range(S)]
        lists = [np.array([pb[i][k] for k in range(lens[i])], dtype=np.int32) for i in range(S)]
        return n_new, seen, lists

    def finalize_status(self, shape: Shape, host_pinned, host_pinned_bytes, dev_meta,
                        dev_meta_bytes, stream=None):
        """(status, Batch): ragged_batch_finalize of the open batch."""
        out = Batch()
        st = _lib().rbkv_state_finalize(self._h, ctypes.byref(shape), _ptr(host_pinned),
                                        int(host_pinned_bytes), _ptr(dev_meta),
                                        int(dev_meta_bytes), _stream(stream),
                                        ctypes.byref(out))
        return st, out

    def finalize(self, shape, host_pinned, host_pinned_bytes, dev_meta, dev_meta_bytes,
                 stream=None) -> Batch:
        st, b = self.finalize_status(shape, host_pinned, host_pinned_bytes, dev_meta,
                                     dev_meta_bytes, stream)
        check(st, "rbkv_state_finalize")
        return b

    def post_forward(self) -> None:
        check(_lib().rbkv_state_post_forward(self._h), "rbkv_state_post_forward")

    def flush_status(self, uid: int) -> int:
        return _lib().rbkv_state_flush(self._h, int(uid))

    def flush(self, uid: int) -> None:
        check(self.flush_status(uid), "rbkv_state_flush")

    def _ids_call(self, fn, uid: int, cap: int):
        out = np.zeros(max(int(cap), 1), dtype=np.int32)
        n = ctypes.c_int32(0)
        st = fn(self._h, int(uid), out.ctypes.data_as(_PI32), int(cap), ctypes.byref(n))
        return st, out[:n.value].copy()

    def offload_status(self, uid: int):
        """(status, ids): give up the blocks of ``uid`` (returned in key order)."""
        info = self.sequence(uid)
        cap = info[2] if info is not None else 0
        return self._ids_call(_lib().rbkv_state_offload, uid, cap)

    def offload(self, uid: int) -> np.ndarray:
        st, ids = self.offload_status(uid)
        check(st, "rbkv_state_offload")
        return ids

    def restore_status(self, uid: int):
        """(status, ids): new blocks for an offloaded ``uid`` (in key order)."""
        info = self.sequence(uid)
        bs = self.config.block_size
        cap = -(-info[0] // bs) if info is not None else 0
        return self._ids_call(_lib().rbkv_state_restore, uid, cap)

    def restore(self, uid: int) -> np.ndarray:
        st, ids = self.restore_status(uid)
        check(st, "rbkv_state_restore")
        return ids

    @property
    def handle(self) -> Optional[int]:
        return self._h.value
