"""A multi-step serving loop on one evolving KV pool, driven by the native ledger,
against the oracle's loop over plain per-sequence histories.

Each pass follows the serving loop of the pages (flush finished requests, schedule,
feed new tokens): running sequences decode one token, waiting requests are admitted
whole while the ledger's can_schedule says yes, and when running decodes no longer fit
the pool the youngest sequence is flushed and queued again with everything it has seen
as its new prompt.  The library side runs the ledger, ragged_batch_finalize of its open
batch, the rotary append into the shared pool and the attention; the oracle side runs
its own ledger model (verdicts, counts and per-sequence state must agree exactly) and
computes attention from each sequence's contiguous history, with no blocks at all.
Blocks freed by one sequence are reused by later ones, so a wrong block table or a
stale slot shows up as an attention mismatch.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle.state_manager as M
import workloads as W

pytestmark = pytest.mark.gpu

VERDICTS = ("ok", "engine_seq_limit", "kv_limit", "batch_seq_limit", "batch_token_limit",
            "seq_token_limit")


@dataclasses.dataclass
class Case:
    name: str
    dtype: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_tracked: int
    max_seqs: int
    max_tokens: int
    n_requests: int
    max_prompt: int
    max_gen: int
    max_arrival: int
    seed: int


CASES = [
    # bf16 GQA 4: matrix-core prefill chunks, split-K decodes; a tight pool forces reuse
    Case("bf16_g4_bs16", "bf16", 8, 2, 128, 16, 22, 6, 6, 160, 14, 120, 24, 16, 0),
    # float32 MHA, head dim 64, 32-token blocks
    Case("f32_mha_bs32", "f32", 4, 4, 64, 32, 10, 5, 5, 128, 10, 90, 30, 10, 1),
    # bf16 GQA 8 (one wave per head decode kernel), 64-token blocks, few blocks
    Case("bf16_g8_bs64", "bf16", 16, 2, 128, 64, 9, 4, 4, 256, 9, 150, 70, 12, 2),
]


def _verdict(nat_v):
    return VERDICTS[nat_v]


def _storage_numpy(x: torch.Tensor, dtype: str):
    return x.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else x.numpy()


@pytest.mark.parametrize("preempt", ["recompute", "offload"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_serving_loop_matches_oracle(case, preempt):
    """``preempt``: a sequence pushed out of a full pool is either flushed and fed again
    from scratch ("recompute"), or has its blocks copied to host memory and released
    ("offload"), to be restored into whatever blocks are free when room returns; its
    history on the oracle side is never touched, so restored blocks must hold exactly
    what was offloaded."""
    import ragged_blocked_kv_amd as R
    from ragged_blocked_kv_amd.runtime import Engine
    from ragged_blocked_kv_amd.state import StateManager

    print(f"serving loop {case.name} preempt={preempt}", flush=True)
    dev = torch.device("cuda:0")
    c = case
    max_context = c.max_prompt + c.max_gen + 1
    # every request must fit an empty pool and one pass on its own
    assert c.max_prompt + c.max_gen <= c.max_tokens
    assert -(-max_context // c.block_size) <= c.num_blocks
    cfg = dict(num_blocks=c.num_blocks, block_size=c.block_size,
               max_tracked_seqs=c.max_tracked, max_seqs=c.max_seqs, max_tokens=c.max_tokens,
               max_context=max_context)
    nat, ora = StateManager(**cfg), M.StateManager(**cfg)
    loop = M.ServingLoop(n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                         rope_base=1e4, dtype=c.dtype)
    eng = Engine(max_tokens=c.max_tokens, max_seqs=c.max_seqs, num_blocks=c.num_blocks,
                 block_size=c.block_size, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads,
                 head_dim=c.head_dim, dtype=c.dtype, device=dev)
    pool = torch.zeros((c.num_blocks, 2, c.n_kv_heads, c.block_size, c.head_dim),
                       dtype=eng.torch_dtype, device=dev)
    tol = 2e-2 if c.dtype == "bf16" else 1e-4

    trace = W.serving_trace(c.seed, c.n_requests, max_prompt=c.max_prompt,
                            max_gen=c.max_gen, max_arrival=c.max_arrival)
    waiting = list(trace)  # arrival order
    running = []  # uids in admission order
    left = {}  # uid -> decode passes still to run
    tokens_of = {}  # uid -> tokens seen so far (for re-queueing a flushed sequence)
    finished = []
    owners = {}  # block id -> set of uids that held it
    stats = dict(kv_limit=0, preempted=0, restored=0, passes=0, prefill_tokens=0, decodes=0,
                 max_err=0.0)
    swapped = []  # (uid, pinned host buffer, its size), oldest first

    def both(fn_nat, fn_ora, what):
        st, v = fn_nat()
        assert st == 0, (what, st)
        o = fn_ora()
        assert _verdict(v) == o, (what, _verdict(v), o)
        return o

    step = 0
    while waiting or running or swapped:
        assert step < 400, "loop did not drain"
        # 1. flush finished sequences
        for u in [u for u in running if left[u] == 0]:
            nat.flush(u)
            ora.flush(u)
            loop.flush(u)
            running.remove(u)
            finished.append(u)
        # 1b. bring offloaded sequences back, oldest first, while their blocks fit
        while swapped:
            u, host, nbytes = swapped[0]
            st, ids = nat.restore_status(u)
            try:
                ora.restore(u)
                o_ok = True
            except M.OracleBlocksError:
                o_ok = False
            assert (st == R.OK) == o_ok, (st, o_ok)
            if st != R.OK:
                assert st == R.ERR_BLOCKS
                break
            assert R.blocked_kv_restore(eng.shape, pool, ids, host, nbytes) == R.OK
            swapped.pop(0)
            running.append(u)
            stats["restored"] += 1
        # 2. decodes of running sequences; preempt the youngest while they do not fit
        while True:
            decoding = set(running)
            batch = [(u, 1) for u in running]
            v = both(lambda: nat.can_schedule_status([u for u, _ in batch], [1] * len(batch)),
                     lambda: ora.can_schedule([u for u, _ in batch], [1] * len(batch)),
                     "decodes")
            if v == "ok":
                break
            assert v == "kv_limit", v
            stats["kv_limit"] += 1
            u = running.pop()
            stats["preempted"] += 1
            if preempt == "offload":
                ids = nat.offload(u)
                assert len(ora.offload(u)) == len(ids)
                st, nbytes = R.rbkv_kv_host_bytes(eng.shape, len(ids))
                host = torch.empty(nbytes, dtype=torch.uint8).pin_memory()
                assert R.blocked_kv_offload(eng.shape, pool, ids, host, nbytes) == R.OK
                swapped.append((u, host, nbytes))
            else:
                nat.flush(u)
                ora.flush(u)
                loop.flush(u)
                waiting.insert(0, W.Request(u, step, tokens_of[u], left[u]))
        # 3. admit arrived requests whole, in order, while the ledger says yes
        while waiting and waiting[0].arrival <= step:
            r = waiting[0]
            cand = batch + [(r.uid, r.prompt)]
            v = both(lambda: nat.can_schedule_status([u for u, _ in cand], [n for _, n in cand]),
                     lambda: ora.can_schedule([u for u, _ in cand], [n for _, n in cand]),
                     "admit")
            if v != "ok":
                stats[v] = stats.get(v, 0) + 1
                break
            batch = cand
            waiting.pop(0)
            running.append(r.uid)
            left[r.uid] = r.gen
        if not batch:
            step += 1
            continue
        uids, n_new = [u for u, _ in batch], [n for _, n in batch]
        # 4. open the batch on both ledgers
        v = both(lambda: nat.put_status(uids, n_new), lambda: ora.put(uids, n_new), "put")
        assert v == "ok"
        assert nat.counts() == (ora.free_blocks, ora.n_tracked)
        for u in uids:
            assert nat.sequence(u) == ora.sequence(u), u
            for b in nat.block_ids(u).tolist():
                owners.setdefault(b, set()).add(u)
        # 5. one pass: library on the pool, oracle on the histories
        T = int(sum(n_new))
        qkv_cpu = W.serving_step_qkv(c.seed, step, T, c.n_q_heads + 2 * c.n_kv_heads,
                                     c.head_dim, c.dtype)
        qkv = qkv_cpu.to(dev)
        out = torch.empty((T, c.n_q_heads, c.head_dim), dtype=eng.torch_dtype, device=dev)
        eng.finalize_state(nat)
        eng.append_rotary(qkv, pool, 1e4)
        eng.attention(qkv, pool, out)
        torch.cuda.synchronize()
        want = loop.step(uids, n_new, _storage_numpy(qkv_cpu, c.dtype))
        got = out.float().cpu().numpy().astype(np.float64)
        err = float(np.max(np.abs(got - want)))
        assert err <= tol, (step, uids, n_new, err)
        stats["max_err"] = max(stats["max_err"], err)
        # 6. close the pass
        nat.post_forward()
        ora.post_forward()
        for u, n in batch:
            if u in decoding:
                tokens_of[u] += 1
                left[u] -= 1
                stats["decodes"] += 1
            else:  # a prompt (possibly of one token) fed whole
                tokens_of[u] = n
                stats["prefill_tokens"] += n
        for u in uids:
            assert nat.sequence(u) == ora.sequence(u), u
            assert loop.seen(u) == nat.sequence(u)[0]
        stats["passes"] += 1
        step += 1

    print(f"  {case.name} {preempt}: {stats}", flush=True)
    assert sorted(finished) == sorted(r.uid for r in trace)
    assert nat.counts() == (c.num_blocks, 0) == (ora.free_blocks, ora.n_tracked)
    # the loop exercised what it is for
    assert stats["kv_limit"] > 0, "pool never ran short"
    assert any(len(s) > 1 for s in owners.values()), "no block was reused"
    if preempt == "offload":
        assert stats["restored"] == stats["preempted"] > 0


SPLITFUSE_CASES = [
    # prompts up to 3x the token budget: every long prompt is fed in chunks
    Case("sf_bf16_g4_bs16", "bf16", 8, 2, 128, 16, 30, 6, 6, 64, 12, 190, 20, 10, 3),
    Case("sf_f32_g2_bs32", "f32", 4, 2, 64, 32, 14, 5, 5, 48, 10, 140, 16, 8, 4),
    Case("sf_bf16_g8_bs64", "bf16", 16, 2, 64, 64, 10, 4, 4, 100, 8, 300, 40, 6, 5),
]


@pytest.mark.parametrize("two_stream", [False, True], ids=["serial", "two_stream"])
@pytest.mark.parametrize("case", SPLITFUSE_CASES, ids=lambda c: c.name)
def test_splitfuse_loop_matches_oracle(case, two_stream):
    """The same loop with batches composed by Dynamic SplitFuse on both ledgers (the
    composed batches must be identical): decodes first, then prompts in arrival order
    cut to fill the token budget, the rest of a prompt continuing in later passes.  With
    two_stream the attention is ragged_blocked_attention_concurrent (for the bf16 cases
    over 64-key blocks: persistent decodes beside the prefill, on batches whose mix of
    chunks and decodes changes every pass, some with no chunk at all)."""
    from ragged_blocked_kv_amd.runtime import Engine
    from ragged_blocked_kv_amd.state import StateManager

    print(f"splitfuse loop {case.name} two_stream={two_stream}", flush=True)
    dev = torch.device("cuda:0")
    c = case
    max_context = c.max_prompt + c.max_gen + 1
    assert -(-max_context // c.block_size) <= c.num_blocks
    cfg = dict(num_blocks=c.num_blocks, block_size=c.block_size,
               max_tracked_seqs=c.max_tracked, max_seqs=c.max_seqs, max_tokens=c.max_tokens,
               max_context=max_context)
    nat, ora = StateManager(**cfg), M.StateManager(**cfg)
    loop = M.ServingLoop(n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                         rope_base=1e4, dtype=c.dtype)
    eng = Engine(max_tokens=c.max_tokens, max_seqs=c.max_seqs, num_blocks=c.num_blocks,
                 block_size=c.block_size, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads,
                 head_dim=c.head_dim, dtype=c.dtype, device=dev)
    pool = torch.zeros((c.num_blocks, 2, c.n_kv_heads, c.block_size, c.head_dim),
                       dtype=eng.torch_dtype, device=dev)
    tol = 2e-2 if c.dtype == "bf16" else 1e-4

    trace = W.serving_trace(c.seed, c.n_requests, max_prompt=c.max_prompt,
                            max_gen=c.max_gen, max_arrival=c.max_arrival)
    arrival = {r.uid: r.arrival for r in trace}
    order = [r.uid for r in trace]  # queue order: arrival order, kept across preemption
    prompt_left = {r.uid: r.prompt for r in trace}
    dec_left = {r.uid: r.gen for r in trace}
    fed = {r.uid: 0 for r in trace}  # tokens cached for the sequence
    done = []
    stats = dict(passes=0, chunks=0, cut_prompts=0, decodes=0, preempted=0, max_err=0.0)

    def flush_both(u):
        nat.flush(u)
        ora.flush(u)
        loop.flush(u)

    step = 0
    while order:
        assert step < 600, "loop did not drain"
        for u in [u for u in order if prompt_left[u] == 0 and dec_left[u] == 0]:
            flush_both(u)
            order.remove(u)
            done.append(u)
        queue = [u for u in order if arrival[u] <= step]
        pending = [prompt_left[u] if prompt_left[u] else 1 for u in queue]
        while True:
            got_u, got_n = nat.compose(queue, pending, c.max_tokens)
            batch = list(zip(got_u.tolist(), got_n.tolist()))
            assert batch == ora.compose(queue, pending, c.max_tokens), step
            if batch or not queue:
                break
            # nothing fits: flush the youngest tracked sequence, its history becomes prompt
            tracked = [u for u in order if nat.sequence(u) is not None]
            assert tracked, "a lone request does not fit an empty pool"
            u = tracked[-1]
            flush_both(u)
            prompt_left[u] += fed[u]
            fed[u] = 0
            stats["preempted"] += 1
            pending = [prompt_left[v] if prompt_left[v] else 1 for v in queue]
        if not batch:
            step += 1
            continue
        uids, n_new = [u for u, _ in batch], [n for _, n in batch]
        assert nat.put(uids, n_new) == 0 and ora.put(uids, n_new) == "ok"
        T = int(sum(n_new))
        qkv_cpu = W.serving_step_qkv(c.seed, step, T, c.n_q_heads + 2 * c.n_kv_heads,
                                     c.head_dim, c.dtype)
        qkv = qkv_cpu.to(dev)
        out = torch.empty((T, c.n_q_heads, c.head_dim), dtype=eng.torch_dtype, device=dev)
        eng.finalize_state(nat)
        eng.append_rotary(qkv, pool, 1e4)
        if two_stream:
            eng.attention_concurrent(qkv, pool, out)
        else:
            eng.attention(qkv, pool, out)
        torch.cuda.synchronize()
        want = loop.step(uids, n_new, _storage_numpy(qkv_cpu, c.dtype))
        err = float(np.max(np.abs(out.float().cpu().numpy().astype(np.float64) - want)))
        assert err <= tol, (step, batch, err)
        stats["max_err"] = max(stats["max_err"], err)
        nat.post_forward()
        ora.post_forward()
        for u, n in batch:
            fed[u] += n
            if prompt_left[u]:
                stats["chunks"] += 1
                stats["cut_prompts"] += n < prompt_left[u]
                prompt_left[u] -= n
            else:
                dec_left[u] -= 1
                stats["decodes"] += 1
        assert nat.counts() == (ora.free_blocks, ora.n_tracked)
        for u in uids:
            assert nat.sequence(u) == ora.sequence(u) == (fed[u], 0, -(-fed[u] // c.block_size))
            assert loop.seen(u) == fed[u]
        stats["passes"] += 1
        step += 1

    print(f"  {case.name}: {stats}", flush=True)
    assert sorted(done) == sorted(r.uid for r in trace)
    assert nat.counts() == (c.num_blocks, 0)
    assert stats["cut_prompts"] > 0, "no prompt was split across passes"
