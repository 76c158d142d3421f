"""Pins of the ledger / allocator oracle (``oracle.state_manager``) to things other than
itself: a hand-derived walk (tests/golden/ledger_walk.txt), a token-by-token simulation
of block growth, conservation invariants under random operations, a planted mistake
that the walk must catch, and the serving loop's agreement with the pinned attention
oracle and with itself under re-chunking."""
import numpy as np
import pytest

import oracle
import oracle as O
import oracle.state_manager as M
import workloads as W
from ledger_walk import OracleSide, run


def test_golden_walk_on_oracle():
    assert run(OracleSide()) == []


def test_golden_walk_catches_a_planted_mistake(monkeypatch):
    # Round the block count down instead of up: the walk must notice.
    monkeypatch.setattr(M, "ceil_div", lambda a, b: int(a) // int(b))
    assert run(OracleSide()) != []


def _simulated_requirements(seen, held, m_max, budget, bs):
    """Feed tokens one at a time: a token that lands on a fresh block needs a new block
    unless one is still held in reserve; stop when the budget would be exceeded."""
    capacity = held * bs  # key slots already owned
    used = seen
    taken = 0
    fed = 0
    while fed < m_max:
        if used == capacity:
            if taken == budget:
                break
            taken += 1
            capacity += bs
        used += 1
        fed += 1
    return fed, taken


def test_kv_requirements_matches_token_by_token_simulation():
    for bs in (1, 3, 4, 16):
        for seen in range(0, 3 * bs + 2):
            min_held = -(-seen // bs)
            for held in (min_held, min_held + 1):
                for m in range(0, 3 * bs + 2):
                    for budget in range(0, 5):
                        got = M.kv_requirements(seen, held, m, budget, bs)
                        assert got == _simulated_requirements(seen, held, m, budget, bs), \
                            (bs, seen, held, m, budget)


def test_kv_requirements_rejects_negative_budgets():
    with pytest.raises(ValueError):
        M.kv_requirements(0, 0, -1, 0, 4)
    with pytest.raises(ValueError):
        M.kv_requirements(0, 0, 1, -1, 4)


def test_allocator_smallest_first_and_whole_refusal():
    a = M.BlockAllocator(6)
    assert a.allocate(2) == [0, 1]
    with pytest.raises(M.OracleBlocksError):
        a.allocate(5)
    assert a.free_blocks == 4
    with pytest.raises(M.OracleBlocksError):
        a.release([1, 2])  # 2 is free: nothing released
    assert a.free_blocks == 4
    a.release([1])
    assert a.allocate(1) == [1]


@pytest.mark.parametrize("seed", range(6))
def test_ledger_invariants_under_random_operations(seed):
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([1, 4, 16]))
    cfg = dict(num_blocks=int(rng.integers(4, 40)), block_size=bs,
               max_tracked_seqs=int(rng.integers(1, 6)), max_seqs=int(rng.integers(1, 5)),
               max_tokens=int(rng.integers(1, 60)), max_context=int(rng.integers(1, 200)))
    L = M.StateManager(**cfg)
    uids = list(range(100, 108))
    verdicts = set()
    for _ in range(300):
        r = rng.random()
        if L.open is not None and r < 0.5:
            L.post_forward()
        elif r < 0.75 and L.open is None:
            k = int(rng.integers(0, 4))
            live = [u for u in uids if not L.seqs.get(u, {}).get("offloaded")]
            us = [int(u) for u in rng.choice(live, size=min(k, len(live)), replace=False)]
            ns = [int(rng.integers(1, 20)) for _ in us]
            before = (L.free_blocks, L.n_tracked, {u: L.sequence(u) for u in uids})
            v = L.put(us, ns)
            verdicts.add(v)
            if v != "ok":  # a refused batch changes nothing
                assert before == (L.free_blocks, L.n_tracked, {u: L.sequence(u) for u in uids})
        elif r < 0.85:
            u = int(rng.choice(uids))
            if u in L.seqs and (L.open is None or u not in L.open):
                L.flush(u)
        elif r < 0.93:
            u = int(rng.choice(uids))
            if u in L.seqs and not L.seqs[u].get("offloaded") and \
                    (L.open is None or u not in L.open):
                L.offload(u)
        else:
            u = int(rng.choice(uids))
            if u in L.seqs and L.seqs[u].get("offloaded") and \
                    M.ceil_div(L.seqs[u]["seen"], bs) <= L.free_blocks:
                L.restore(u)
        # conservation and shape of the ledger
        lists = [q["blocks"] for q in L.seqs.values()]
        flat = [b for l in lists for b in l]
        assert len(flat) == len(set(flat))
        assert set(flat).isdisjoint(L.alloc.free)
        assert len(flat) + L.free_blocks == cfg["num_blocks"]
        assert L.n_tracked <= cfg["max_tracked_seqs"]
        for q in L.seqs.values():
            held = 0 if q.get("offloaded") else M.ceil_div(q["seen"] + q["in_flight"], bs)
            assert len(q["blocks"]) == held
            assert q["seen"] + q["in_flight"] <= cfg["max_context"]
    assert "ok" in verdicts


def test_serving_loop_matches_blocked_oracle_on_one_pass():
    """One mixed pass of the loop equals the pinned blocked-pool oracle on the same batch
    (empty history, fresh sequences, blocks laid out in batch order)."""
    import torch

    Hq, Hkv, d, bs = 4, 2, 16, 4
    n_new = [5, 1, 9]
    qkv = W.serving_step_qkv(3, 0, sum(n_new), Hq + 2 * Hkv, d, "bf16")
    bits = qkv.view(torch.int16).numpy().view(np.uint16)
    loop = M.ServingLoop(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, rope_base=1e4,
                         dtype="bf16")
    got = loop.step([10, 11, 12], n_new, bits)
    lists, at = [], 0
    for n in n_new:
        nb = -(-n // bs)
        lists.append(np.arange(at, at + nb, dtype=np.int32))
        at += nb
    meta = oracle.batch_metadata(n_new, [0, 0, 0], lists, bs)
    pool = np.zeros((at, 2, Hkv, bs, d), dtype=np.uint16)
    q_rot, pool = oracle.append_rotary(bits, pool, meta, Hq, Hkv, bs, 1e4, "bf16")
    want = oracle.ragged_attention(q_rot, pool, meta, Hq, Hkv, bs, "bf16")
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_serving_loop_is_chunking_invariant():
    """A prompt fed as one chunk or as several chunks over several passes gives the same
    attention rows: each token's output depends only on the keys up to its position."""
    Hq, Hkv, d = 4, 1, 16
    qkv = W.serving_step_qkv(5, 0, 23, Hq + 2 * Hkv, d, "f32").numpy()
    whole = M.ServingLoop(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, rope_base=1e4,
                          dtype="f32")
    a = whole.step([1], [23], qkv)
    parts = M.ServingLoop(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, rope_base=1e4,
                          dtype="f32")
    outs, t = [], 0
    for n in (7, 1, 10, 5):
        outs.append(parts.step([1], [n], qkv[t:t + n]))
        t += n
    np.testing.assert_allclose(np.concatenate(outs), a, rtol=0, atol=1e-12)
    assert parts.seen(1) == 23
    parts.flush(1)
    assert parts.seen(1) == 0


def _random_ledger(rng):
    bs = int(rng.choice([1, 4, 16]))
    cfg = dict(num_blocks=int(rng.integers(4, 60)), block_size=bs,
               max_tracked_seqs=int(rng.integers(1, 8)), max_seqs=int(rng.integers(1, 6)),
               max_tokens=int(rng.integers(1, 80)), max_context=int(rng.integers(1, 120)))
    L = M.StateManager(**cfg)
    uids = list(range(1, 11))
    for _ in range(int(rng.integers(0, 30))):  # random history
        if rng.random() < 0.7:
            us = [int(u) for u in rng.choice(uids, size=int(rng.integers(1, 4)), replace=False)]
            L.put(us, [int(rng.integers(1, 30)) for _ in us])
            if L.open is not None:
                L.post_forward()
        else:
            u = int(rng.choice(uids))
            if u in L.seqs:
                L.flush(u)
    return L, uids


def _fits(L, batch, budget):
    if not batch:
        return True
    if len(batch) > L.max_seqs or sum(n for _, n in batch) > min(budget, L.max_tokens):
        return False
    return L.can_schedule([u for u, _ in batch], [n for _, n in batch]) == "ok"


@pytest.mark.parametrize("seed", range(40))
def test_compose_is_schedulable_maximal_and_decodes_first(seed):
    """What Dynamic SplitFuse promises, checked through can_schedule rather than by
    re-running the greedy: the composed batch can be put; no candidate can take one
    more token without breaking a limit (the budget is filled as far as the limits
    allow); and a decode is left out only if it would not fit even beside the chosen
    decodes alone (prefill chunks never displace decodes)."""
    rng = np.random.default_rng(seed)
    L, uids = _random_ledger(rng)
    queue = [int(u) for u in rng.permutation(uids)[:int(rng.integers(0, 10))]]
    pending = [1 if rng.random() < 0.4 else int(rng.integers(2, 50)) for _ in queue]
    budget = int(rng.integers(1, 100))
    batch = L.compose(queue, pending, budget)
    assert _fits(L, batch, budget)
    got = dict(batch)
    # chosen in two walks: decodes first, each walk in queue order
    order = [u for u, p in zip(queue, pending) if p == 1] + \
        [u for u, p in zip(queue, pending) if p > 1]
    assert [u for u, _ in batch] == [u for u in order if u in got]
    for u, p in zip(queue, pending):
        assert got.get(u, 0) <= p
        if got.get(u, 0) < p:  # one more token for u must break a limit
            more = [(v, n + (v == u)) for v, n in batch] + ([] if u in got else [(u, 1)])
            assert not _fits(L, more, budget), (u, batch)
    decodes = [(u, got[u]) for u, p in zip(queue, pending) if p == 1 and u in got]
    for u, p in zip(queue, pending):
        if p == 1 and u not in got:
            assert not _fits(L, decodes + [(u, 1)], budget), (u, batch)
    if L.open is None and batch:
        assert L.put([u for u, _ in batch], [n for _, n in batch]) == "ok"


def test_compose_fills_the_budget_when_nothing_else_binds():
    L = M.StateManager(num_blocks=1000, block_size=16, max_tracked_seqs=64, max_seqs=64,
                       max_tokens=512, max_context=4096)
    queue = list(range(100, 140))
    pending = [1] * 20 + [300, 7, 250, 90] + [1000] * 16
    batch = L.compose(queue, pending, 512)
    assert sum(n for _, n in batch) == 512
    assert [n for _, n in batch[:20]] == [1] * 20
    assert batch[20:] == [(120, 300), (121, 7), (122, 185)]  # the third prompt is cut


def test_offload_restore_blocks_by_hand():
    """Three blocks of one element pair each: offload [2, 0], restore them into [1, 2]."""
    pool = np.arange(12, dtype=np.uint16).reshape(3, 2, 1, 1, 2)
    host = O.offload_blocks(pool, [2, 0])
    assert host.reshape(2, 4).tolist() == [[8, 9, 10, 11], [0, 1, 2, 3]]
    back = O.restore_blocks(np.zeros_like(pool), [1, 2], host)
    assert back.reshape(3, 4).tolist() == [[0, 0, 0, 0], [8, 9, 10, 11], [0, 1, 2, 3]]


def test_offload_restore_round_trip():
    rng = np.random.default_rng(3)
    pool = rng.integers(0, 1 << 16, size=(9, 2, 2, 4, 8)).astype(np.uint16)
    ids = [7, 1, 4, 0]
    host = O.offload_blocks(pool, ids)
    wiped = pool.copy()
    wiped[ids] = 0
    assert np.array_equal(O.restore_blocks(wiped, ids, host), pool)
