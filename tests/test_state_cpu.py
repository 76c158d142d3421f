"""The native block allocator and sequence ledger (include/rbkv_state.h) on the host:
the hand-derived walk, bit-exact agreement with the oracle on random operation
sequences (verdicts, errors, counts, per-sequence state; the library's own choice of
block ids is checked for validity), its stated LIFO policy, the uid table under heavy
churn, and the argument errors.  No call here touches a GPU."""
import ctypes

import numpy as np
import pytest

import oracle.state_manager as M
import ragged_blocked_kv_amd as R
import ragged_blocked_kv_amd.state as S
from ledger_walk import NativeSide, VERDICT_NAMES, run


def test_golden_walk_on_library():
    assert run(NativeSide()) == []


def test_allocator_is_lifo_and_starts_at_zero():
    a = S.BlockAllocator(10)
    assert a.allocate(4).tolist() == [0, 1, 2, 3]
    a.free([2, 0])
    assert a.allocate(2).tolist() == [2, 0]  # given back in order, handed out first
    assert a.allocate(1).tolist() == [4]
    assert a.free_blocks == 5


def test_allocator_errors():
    L = S._lib()
    h = ctypes.c_void_p()
    assert L.rbkv_allocator_create(0, ctypes.byref(h)) == R.ERR_INVALID_ARG
    assert L.rbkv_allocator_create((1 << 26) + 1, ctypes.byref(h)) == R.ERR_UNSUPPORTED
    assert L.rbkv_allocator_create(4, None) == R.ERR_INVALID_ARG
    a = S.BlockAllocator(4)
    assert a.allocate_status(-1)[0] == R.ERR_INVALID_ARG
    assert L.rbkv_allocator_allocate(a._h, 2, None) == R.ERR_INVALID_ARG
    assert L.rbkv_allocator_allocate(None, 0, None) == R.ERR_INVALID_ARG
    assert L.rbkv_allocator_free(a._h, 1, None) == R.ERR_INVALID_ARG
    assert L.rbkv_allocator_free_count(a._h, None) == R.ERR_INVALID_ARG
    assert L.rbkv_allocator_destroy(None) == R.OK


def test_state_create_errors():
    L = S._lib()
    h = ctypes.c_void_p()
    good = dict(num_blocks=8, block_size=4, max_tracked_seqs=3, max_seqs=2, max_tokens=12,
                max_context=20)
    for k in good:
        c = S.StateConfig(*[0 if f == k else v for f, v in good.items()])
        assert L.rbkv_state_create(ctypes.byref(c), ctypes.byref(h)) == R.ERR_INVALID_ARG, k
    for k, v in [("num_blocks", (1 << 26) + 1), ("max_tracked_seqs", 65537),
                 ("max_seqs", 65537), ("max_tokens", (1 << 20) + 1), ("block_size", 4097)]:
        c = S.StateConfig(*[v if f == k else x for f, x in good.items()])
        assert L.rbkv_state_create(ctypes.byref(c), ctypes.byref(h)) == R.ERR_UNSUPPORTED, k
    c = S.StateConfig(*good.values())
    assert L.rbkv_state_create(None, ctypes.byref(h)) == R.ERR_INVALID_ARG
    assert L.rbkv_state_create(ctypes.byref(c), None) == R.ERR_INVALID_ARG
    assert L.rbkv_state_destroy(None) == R.OK


def test_state_null_and_shape_errors():
    L = S._lib()
    st = S.StateManager(num_blocks=8, block_size=4, max_tracked_seqs=3, max_seqs=2,
                        max_tokens=12, max_context=20)
    v = ctypes.c_int32()
    assert L.rbkv_state_counts(None, None, None) == R.ERR_INVALID_ARG
    assert L.rbkv_state_can_schedule(st._h, 1, None, None, ctypes.byref(v)) == R.ERR_INVALID_ARG
    assert L.rbkv_state_can_schedule(st._h, -1, None, None, ctypes.byref(v)) == R.ERR_INVALID_ARG
    assert st.can_schedule_status([1], [5])[0] == R.OK
    assert L.rbkv_state_query(st._h, 1, -1, 0, ctypes.byref(v), ctypes.byref(v)) == \
        R.ERR_INVALID_ARG
    assert L.rbkv_state_post_forward(st._h) == R.ERR_INVALID_ARG
    shape = R.Shape.make(max_tokens=12, max_seqs=2, num_blocks=8, block_size=4,
                         n_q_heads=2, n_kv_heads=1, head_dim=64, dtype="bf16")
    # no open batch: refused before anything reaches ragged_batch_finalize
    assert st.finalize_status(shape, 0x1000, 1 << 20, 0x1000, 1 << 20)[0] == R.ERR_INVALID_ARG
    assert st.put([1], [5]) == S.SCHED_OK
    bad = R.Shape.make(max_tokens=12, max_seqs=2, num_blocks=9, block_size=4,
                       n_q_heads=2, n_kv_heads=1, head_dim=64, dtype="bf16")
    assert st.finalize_status(bad, 0x1000, 1 << 20, 0x1000, 1 << 20)[0] == R.ERR_INVALID_ARG
    bad = R.Shape.make(max_tokens=12, max_seqs=2, num_blocks=8, block_size=16,
                       n_q_heads=2, n_kv_heads=1, head_dim=64, dtype="bf16")
    assert st.finalize_status(bad, 0x1000, 1 << 20, 0x1000, 1 << 20)[0] == R.ERR_INVALID_ARG
    ids = np.zeros(1, dtype=np.int32)
    n = ctypes.c_int32()
    assert L.rbkv_state_block_ids(st._h, 1, ids.ctypes.data_as(S._PI32), 1, ctypes.byref(n)) \
        == R.ERR_INVALID_ARG  # holds 2 blocks, room for 1
    assert st.block_ids(1).tolist() == [0, 1]


def _check_native_ids(nat, uids, num_blocks):
    """The library's block lists are disjoint, in range and add up with the free count."""
    seen_ids = []
    for u in uids:
        info = nat.sequence(u)
        if info is None:
            continue
        ids = nat.block_ids(u)
        assert len(ids) == info[2]
        seen_ids.extend(ids.tolist())
    assert len(seen_ids) == len(set(seen_ids))
    assert all(0 <= i < num_blocks for i in seen_ids)
    assert len(seen_ids) + nat.free_blocks == num_blocks


@pytest.mark.parametrize("seed", range(12))
def test_random_operations_match_oracle(seed):
    rng = np.random.default_rng(1000 + seed)
    bs = int(rng.choice([1, 4, 16, 64]))
    cfg = dict(num_blocks=int(rng.integers(2, 60)), block_size=bs,
               max_tracked_seqs=int(rng.integers(1, 8)), max_seqs=int(rng.integers(1, 6)),
               max_tokens=int(rng.integers(1, 80)), max_context=int(rng.integers(1, 300)))
    ora, nat = M.StateManager(**cfg), S.StateManager(**cfg)
    uids = [int(u) for u in rng.integers(-(1 << 62), 1 << 62, size=10)]
    names = {R.OK: "ok", R.ERR_INVALID_ARG: "invalid"}

    def oracle_call(fn):
        try:
            return "ok", fn()
        except ValueError:
            return "invalid", None

    for step in range(400):
        r = rng.random()
        if r < 0.2:
            o = oracle_call(ora.post_forward)[0]
            try:
                nat.post_forward()
                n = "ok"
            except R.RbkvError as e:
                n = names.get(e.status, e.status)
            assert o == n, step
        elif r < 0.7:
            k = int(rng.integers(0, 5))
            us = [int(u) for u in rng.choice(uids, size=k, replace=True)]  # duplicates too
            ns = [int(rng.integers(0 if rng.random() < 0.03 else 1, 30)) for _ in us]
            op = "put" if rng.random() < 0.6 else "can_schedule"
            st, v = getattr(nat, op + "_status")(us, ns)
            o_st, o_v = oracle_call(lambda: getattr(ora, op)(us, ns))
            assert names.get(st, st) == o_st, (step, op, us, ns)
            if st == R.OK:
                assert VERDICT_NAMES[v] == o_v, (step, op, us, ns)
        elif r < 0.8:
            u = int(rng.choice(uids))
            o = oracle_call(lambda: ora.flush(u))[0]
            assert names.get(nat.flush_status(u), "?") == o, step
        elif r < 0.85:
            u = int(rng.choice(uids))
            o_st, o_ids = oracle_call(lambda: ora.offload(u))
            st, ids = nat.offload_status(u)
            assert names.get(st, st) == o_st, step
            if st == R.OK:
                assert len(ids) == len(o_ids)
        elif r < 0.9:
            u = int(rng.choice(uids))
            try:
                o_st, o_n = "ok", len(ora.restore(u))
            except ValueError:
                o_st, o_n = "invalid", None
            except M.OracleBlocksError:
                o_st, o_n = "blocks", None
            st, ids = nat.restore_status(u)
            assert {R.OK: "ok", R.ERR_INVALID_ARG: "invalid", R.ERR_BLOCKS: "blocks"}[st] == o_st
            if st == R.OK:
                assert len(ids) == o_n
        else:
            u = int(rng.choice(uids))
            m, b = int(rng.integers(0, 70)), int(rng.integers(0, 6))
            st, t, n = nat.query_status(u, m, b)
            o_st, o_r = oracle_call(lambda: ora.query(u, m, b))
            assert names.get(st, st) == o_st, step
            if st == R.OK:
                assert (t, n) == tuple(o_r), step
        assert nat.counts() == (ora.free_blocks, ora.n_tracked), step
        for u in uids:
            assert nat.sequence(u) == ora.sequence(u), (step, u)
        if ora.open is not None:
            o_new, o_seen, o_lists = ora.batch()
            n_new, n_seen, n_lists = nat.batch()
            assert n_new.tolist() == o_new and n_seen.tolist() == o_seen
            assert [len(l) for l in n_lists] == [len(l) for l in o_lists]
        _check_native_ids(nat, uids, cfg["num_blocks"])


def test_uid_table_under_churn():
    """Thousands of distinct uids through a small ledger: the open-addressing uid table
    must keep finding every live sequence after many erasures."""
    rng = np.random.default_rng(7)
    cap = 64
    nat = S.StateManager(num_blocks=4096, block_size=16, max_tracked_seqs=cap, max_seqs=cap,
                         max_tokens=1 << 16, max_context=1 << 16)
    live = {}
    next_uid = 0
    for _ in range(3000):
        if len(live) < cap and rng.random() < 0.55:
            # many uids that collide in the low bits
            u = (next_uid << 20) | 5
            next_uid += 1
            n = int(rng.integers(1, 40))
            assert nat.put([u], [n]) == S.SCHED_OK
            nat.post_forward()
            live[u] = n
        elif live:
            u = list(live)[int(rng.integers(0, len(live)))]
            nat.flush(u)
            del live[u]
        assert nat.n_tracked == len(live)
    for u, n in live.items():
        assert nat.sequence(u) == (n, 0, -(-n // 16))
    assert nat.sequence(12345) is None


def test_batch_views_point_into_the_ledger():
    nat = S.StateManager(num_blocks=32, block_size=4, max_tracked_seqs=4, max_seqs=4,
                         max_tokens=64, max_context=64)
    assert nat.put([7, 9], [6, 1]) == S.SCHED_OK
    n_new, seen, lists = nat.batch()
    assert n_new.tolist() == [6, 1] and seen.tolist() == [0, 0]
    assert lists[0].tolist() == nat.block_ids(7).tolist()
    assert lists[1].tolist() == nat.block_ids(9).tolist()
    nat.post_forward()
    assert nat.put([9, 7], [4, 1]) == S.SCHED_OK  # 9 grows to 5 tokens: a 2nd block
    n_new, seen, lists = nat.batch()
    assert seen.tolist() == [1, 6] and [len(l) for l in lists] == [2, 2]


@pytest.mark.parametrize("seed", range(12))
def test_compose_matches_oracle(seed):
    """Dynamic SplitFuse composition is fixed by the ledger's counts alone, so the
    library's batch must equal the oracle's exactly, through a run of passes in which
    the composed batch is put, run and closed on both ledgers."""
    rng = np.random.default_rng(5000 + seed)
    bs = int(rng.choice([1, 4, 16, 64]))
    cfg = dict(num_blocks=int(rng.integers(2, 80)), block_size=bs,
               max_tracked_seqs=int(rng.integers(1, 10)), max_seqs=int(rng.integers(1, 8)),
               max_tokens=int(rng.integers(1, 200)), max_context=int(rng.integers(1, 400)))
    ora, nat = M.StateManager(**cfg), S.StateManager(**cfg)
    uids = [int(u) for u in rng.integers(-(1 << 62), 1 << 62, size=14)]
    prompt = {u: int(rng.integers(1, 150)) for u in uids}  # prompt tokens not yet fed
    decode = {u: int(rng.integers(1, 6)) for u in uids}  # decode passes still to run
    for step in range(120):
        live = [u for u in rng.permutation(uids).tolist() if prompt[u] or decode[u]]
        p = [prompt[u] if prompt[u] else 1 for u in live]
        budget = int(rng.integers(1, 250))
        want = ora.compose(live, p, budget)
        u, n = nat.compose(live, p, budget)
        assert list(zip(u.tolist(), n.tolist())) == want, step
        if want:
            assert nat.put(u, n) == S.SCHED_OK and ora.put(u, n) == "ok"
            nat.post_forward()
            ora.post_forward()
            for a, b in want:
                if prompt[a]:
                    prompt[a] -= b
                else:
                    decode[a] -= 1
        for a in uids:  # finished: flush, and a new request arrives on the same uid
            if not prompt[a] and not decode[a]:
                nat.flush(a)
                ora.flush(a)
                prompt[a], decode[a] = int(rng.integers(1, 150)), int(rng.integers(1, 6))
        assert nat.counts() == (ora.free_blocks, ora.n_tracked)
    # compose argument errors
    assert nat.compose_status([1, 1], [1, 1], 5)[0] == R.ERR_INVALID_ARG
    assert nat.compose_status([1], [0], 5)[0] == R.ERR_INVALID_ARG
    assert nat.compose_status([1], [1], 0)[0] == R.ERR_INVALID_ARG
    assert nat.compose_status([], [], 5)[0] == R.OK
