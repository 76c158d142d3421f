"""Runner for ``tests/golden/ledger_walk.txt`` against either side: the float-free CPU
model in ``oracle.state_manager`` or the library's native ledger.  Each side is wrapped
in an adapter that speaks the fixture's vocabulary (verdict names, "invalid" for an
argument error, "blocks" for a refused allocation or free)."""
from __future__ import annotations

import os
import re

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "ledger_walk.txt")

VERDICT_NAMES = ("ok", "engine_seq_limit", "kv_limit", "batch_seq_limit",
                 "batch_token_limit", "seq_token_limit")


class OracleSide:
    def __init__(self):
        import oracle.state_manager as M
        self.M = M

    def ledger(self, **cfg):
        return self.M.StateManager(**cfg)

    def allocator(self, n):
        return self.M.BlockAllocator(n)

    def _call(self, fn):
        try:
            r = fn()
        except self.M.OracleBlocksError:
            return "blocks", None
        except ValueError:
            return "invalid", None
        return "ok", r

    def query(self, L, uid, m, b):
        st, r = self._call(lambda: L.query(uid, m, b))
        return list(r) if st == "ok" else st

    def can_schedule(self, L, uids, n):
        st, r = self._call(lambda: L.can_schedule(uids, n))
        return r if st == "ok" else st

    def put(self, L, uids, n):
        st, r = self._call(lambda: L.put(uids, n))
        return r if st == "ok" else st

    def compose(self, L, budget, uids, pending):
        st, r = self._call(lambda: L.compose(uids, pending, budget))
        return [(int(u), int(n)) for u, n in r] if st == "ok" else st

    def offload(self, L, uid):
        st, r = self._call(lambda: L.offload(uid))
        return len(r) if st == "ok" else st

    def restore(self, L, uid):
        st, r = self._call(lambda: L.restore(uid))
        return len(r) if st == "ok" else st

    def batch(self, L):
        st, r = self._call(lambda: L.batch())
        if st != "ok":
            return st
        n_new, seen, lists = r
        return [(a, b, len(c)) for a, b, c in zip(n_new, seen, lists)]

    def post_forward(self, L):
        return self._call(L.post_forward)[0]

    def flush(self, L, uid):
        return self._call(lambda: L.flush(uid))[0]

    def seq(self, L, uid):
        return L.sequence(uid)

    def counts(self, L):
        return L.free_blocks, L.n_tracked

    def alloc(self, A, n):
        st, r = self._call(lambda: A.allocate(n))
        return st, r

    def release(self, A, ids):
        return self._call(lambda: A.release(ids))[0]

    def free_count(self, A):
        return A.free_blocks


class NativeSide:
    def __init__(self):
        import ragged_blocked_kv_amd as R
        import ragged_blocked_kv_amd.state as S
        self.R, self.S = R, S

    def _status(self, st):
        return {self.R.OK: "ok", self.R.ERR_INVALID_ARG: "invalid",
                self.R.ERR_BLOCKS: "blocks"}.get(st, f"status {st}")

    def ledger(self, **cfg):
        return self.S.StateManager(**cfg)

    def allocator(self, n):
        return self.S.BlockAllocator(n)

    def query(self, L, uid, m, b):
        st, t, n = L.query_status(uid, m, b)
        return [t, n] if st == self.R.OK else self._status(st)

    def can_schedule(self, L, uids, n):
        st, v = L.can_schedule_status(uids, n)
        return VERDICT_NAMES[v] if st == self.R.OK else self._status(st)

    def put(self, L, uids, n):
        st, v = L.put_status(uids, n)
        return VERDICT_NAMES[v] if st == self.R.OK else self._status(st)

    def compose(self, L, budget, uids, pending):
        st, u, n = L.compose_status(uids, pending, budget)
        if st != self.R.OK:
            return self._status(st)
        return [(int(a), int(b)) for a, b in zip(u, n)]

    def offload(self, L, uid):
        st, ids = L.offload_status(uid)
        return len(ids) if st == self.R.OK else self._status(st)

    def restore(self, L, uid):
        st, ids = L.restore_status(uid)
        return len(ids) if st == self.R.OK else self._status(st)

    def batch(self, L):
        try:
            n_new, seen, lists = L.batch()
        except self.R.RbkvError as e:
            return self._status(e.status)
        return [(int(a), int(b), len(c)) for a, b, c in zip(n_new, seen, lists)]

    def post_forward(self, L):
        try:
            L.post_forward()
        except self.R.RbkvError as e:
            return self._status(e.status)
        return "ok"

    def flush(self, L, uid):
        return self._status(L.flush_status(uid))

    def seq(self, L, uid):
        return L.sequence(uid)

    def counts(self, L):
        return L.counts()

    def alloc(self, A, n):
        st, ids = A.allocate_status(n)
        return self._status(st), ([int(i) for i in ids] if st == self.R.OK else None)

    def release(self, A, ids):
        return self._status(A.free_status(ids))

    def free_count(self, A):
        return A.free_blocks


def _pairs(tokens):
    uids, n = [], []
    for t in tokens:
        u, k = t.split(":")
        uids.append(int(u))
        n.append(int(k))
    return uids, n


def run(side, path=GOLDEN):
    """Run every line; return a list of (line number, text, got) for mismatches."""
    bad = []
    L = A = None
    named = {}
    held = set()  # ids the current allocator has handed out and not taken back
    n_alloc = 0
    for lineno, raw in enumerate(open(path), 1):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        lhs, _, rhs = line.partition("->")
        words, expect = lhs.split(), rhs.split()
        op, args = words[0], words[1:]
        got = None
        if op == "ledger":
            L = side.ledger(**{k: int(v) for k, v in (a.split("=") for a in args)})
            continue
        if op == "allocator":
            n_alloc = int(args[0])
            A, named, held = side.allocator(n_alloc), {}, set()
            continue
        if op == "query":
            got = side.query(L, int(args[0]), int(args[1]), int(args[2]))
            ok = (expect == ["invalid"] and got == "invalid") or \
                (got != "invalid" and got == [int(x) for x in expect])
        elif op in ("can_schedule", "put"):
            uids, n = _pairs(args)
            got = getattr(side, op)(L, uids, n)
            ok = [got] == expect
        elif op == "compose":
            uids, n = _pairs(args[1:])
            got = side.compose(L, int(args[0]), uids, n)
            ok = (expect == ["invalid"] and got == "invalid") or \
                (got != "invalid" and got == [tuple(int(x) for x in e.split(":")) for e in expect])
        elif op == "batch":
            got = side.batch(L)
            want = [tuple(int(x) for x in e.split("/")) for e in expect]
            ok = got == want
        elif op in ("post_forward",):
            got = side.post_forward(L)
            ok = [got] == expect
        elif op in ("offload", "restore"):
            got = getattr(side, op)(L, int(args[0]))
            ok = [str(got)] == expect
        elif op == "flush":
            got = side.flush(L, int(args[0]))
            ok = [got] == expect
        elif op == "seq":
            got = side.seq(L, int(args[0]))
            ok = (got is None and expect == ["untracked"]) or \
                (got is not None and list(got) == [int(x) for x in expect])
        elif op == "counts":
            got = list(side.counts(L))
            ok = got == [int(x) for x in expect]
        elif op == "free_count":
            got = side.free_count(A)
            ok = got == int(expect[0])
        elif op == "alloc":
            st, ids = side.alloc(A, int(args[0]))
            got = st
            ok = [st] == expect
            if st == "ok":
                # whatever ids come back must be distinct, in range and not held
                valid = (len(ids) == int(args[0]) and len(set(ids)) == len(ids) and
                         all(0 <= i < n_alloc for i in ids) and not (set(ids) & held))
                ok = ok and valid
                held |= set(ids)
                if len(args) > 1:
                    named[args[1].lstrip("@")] = ids
        elif op == "release":
            ids = []
            for a in args:
                m = re.fullmatch(r"@(\w+)(?:\[(\d+)\])?", a)
                if m:
                    v = named[m.group(1)]
                    ids.extend(v if m.group(2) is None else [v[int(m.group(2))]])
                else:
                    ids.append(int(a))
            got = side.release(A, ids)
            ok = [got] == expect
            if got == "ok":
                held -= set(ids)
        else:
            raise ValueError(f"{path}:{lineno}: unknown op {op}")
        if not ok:
            bad.append((lineno, raw.rstrip(), got))
    return bad
