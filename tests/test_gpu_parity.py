"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded
inputs.  Metadata is compared bit for bit; V placement (and K placement with rotation
off) bit for bit; rotated Q/K within one storage ulp (bf16) or 1e-5 (float32); pool
bytes outside the written slots unchanged; attention within max-abs 2e-2 (bf16) or
1e-4 (float32).  Small batches are compared element by element in full; the five
full-size workloads (in the launch configuration the benchmark times) on sampled
sequences that the oracle computes one by one.  Work lists are checked for exact
coverage of every (token, query head, key)."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


def _engine(wl):
    from ragged_blocked_kv_amd.runtime import Engine

    return Engine.for_workload(wl)


def _np_storage(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _ordered(bits_u16):
    """bf16 patterns to integers whose difference counts representable steps."""
    b = bits_u16.astype(np.int32)
    return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)


def _assert_within_one_ulp(gpu, ref, dtype, what):
    if dtype == "bf16":
        d = np.abs(_ordered(gpu) - _ordered(ref))
        assert d.max() <= 1, f"{what}: {d.max()} ulp"
    else:
        d = np.abs(gpu.astype(np.float64) - ref.astype(np.float64)).max()
        assert d <= 1e-5, f"{what}: {d}"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_work_coverage(md, b, wl):
    """Every (token, kv head) is covered once, its keys 0..pos exactly once."""
    Hkv = wl.n_kv_heads
    T = wl.T
    cover = {}
    pos = md["pos"]
    slots = set()
    for tok, kvh, split, slot in md["decode_work"]:
        L = pos[tok] + 1
        tiles = -(-L // 64)
        if slot < 0:
            rng = (0, L)
        else:
            t0 = split * b.split_tiles
            rng = (t0 * 64, min(L, (t0 + b.split_tiles) * 64))
            assert 0 <= slot < b.n_partials and slot not in slots
            slots.add(slot)
            assert t0 < tiles
        cover.setdefault((tok, kvh), []).append(rng)
    # Whole splits come first: once an item shorter than a split of a single-token
    # sequence appears, only such items follow, each no longer than the one before.
    last_short = None
    tok_seq = np.searchsorted(np.asarray(md["cu_seqlens"]), np.arange(T), side="right") - 1
    for tok, kvh, split, slot in md["decode_work"]:
        tiles = -(-(pos[tok] + 1) // 64)
        length = tiles if slot < 0 else min(b.split_tiles, tiles - split * b.split_tiles)
        short = int(wl.n_new[tok_seq[tok]]) == 1 and length < b.split_tiles
        assert short or last_short is None, (tok, kvh, split, length)
        if short:
            assert last_short is None or length <= last_short, (tok, kvh, length, last_short)
            last_short = length
    cu = md["cu_seqlens"]
    # one record per chunk sequence, ranked by work (longest first); the prefill kernel
    # covers all its query tiles for every kv head
    ranked = [int(r[0]) for r in md["prefill_work"]]
    assert len(set(ranked)) == len(ranked) == b.n_prefill_seqs
    work = [(-(-int(wl.n_new[i]) // max(1, 256 // (wl.n_q_heads // Hkv)))) *
            (2 * int(wl.seen[i]) + int(wl.n_new[i])) for i in ranked]
    assert all(a >= c for a, c in zip(work, work[1:]))
    for seq, nqt, _, _ in md["prefill_work"]:
        assert nqt >= 1
        for kvh in range(Hkv):
            for tok in range(cu[seq], cu[seq + 1]):
                cover.setdefault((tok, kvh), []).append((0, pos[tok] + 1))
    assert len(cover) == T * Hkv
    for (tok, kvh), rs in cover.items():
        rs = sorted(rs)
        assert rs[0][0] == 0 and rs[-1][1] == pos[tok] + 1, (tok, kvh, rs)
        for a, c in zip(rs, rs[1:]):
            assert a[1] == c[0], (tok, kvh, rs)  # contiguous, no overlap
    for tok, kvh, slot0, ns in md["combine_work"]:
        got = sorted(r for r in cover[(tok, kvh)])
        assert len(got) == ns >= 2


def run_full(wl, rope_base=None, check_coverage=True):
    """Whole batch through GPU and oracle; compares everything element by element."""
    base = wl.rope_base if rope_base is None else rope_base
    eng = _engine(wl)
    qkv_in = W.make_qkv(wl)
    pool_in = W.make_pool_history(wl, device="cpu")
    qkv = qkv_in.cuda()
    pool = pool_in.cuda()
    b = eng.finalize(wl.n_new, wl.seen, wl.block_lists)
    eng.append_rotary(qkv, pool, base)
    out = eng.new_out()
    eng.attention(qkv, pool, out)
    torch.cuda.synchronize()

    md = eng.metadata()
    ref_md = O.batch_metadata(wl.n_new, wl.seen, wl.block_lists, wl.block_size)
    for k in ref_md:
        assert np.array_equal(md[k], ref_md[k]), k
    if check_coverage:
        check_work_coverage(md, b, wl)

    q_ref, pool_ref = O.append_rotary(_np_storage(qkv_in), _np_storage(pool_in), ref_md,
                                      wl.n_q_heads, wl.n_kv_heads, wl.block_size, base, wl.dtype)
    q_gpu, pool_gpu = _np_storage(qkv), _np_storage(pool)
    Hq, Hkv = wl.n_q_heads, wl.n_kv_heads
    assert np.array_equal(q_gpu[:, Hq:], q_ref[:, Hq:])  # K, V rows of qkv untouched
    if base <= 0:
        assert np.array_equal(q_gpu, q_ref)
        assert np.array_equal(pool_gpu, pool_ref)
    else:
        _assert_within_one_ulp(q_gpu[:, :Hq], q_ref[:, :Hq], wl.dtype, "rotated Q")
        assert np.array_equal(pool_gpu[:, 1], pool_ref[:, 1])  # values: raw, bit exact
        _assert_within_one_ulp(pool_gpu[:, 0], pool_ref[:, 0], wl.dtype, "rotated K / pool")
    ref = O.ragged_attention(q_ref, pool_ref, ref_md, Hq, Hkv, wl.block_size, wl.dtype)
    got = O.storage_to_f64(_np_storage(out), wl.dtype)
    err = np.max(np.abs(got - ref))
    assert err <= TOL[wl.dtype], f"{wl.name}: max abs err {err}"
    return err


# ---------------------------------------------------------------- small batches ----


def test_tiny_f32_workload():
    wl = W.make_workload("tiny_f32")
    _say(f"case tiny_f32 T={wl.T}")
    run_full(wl)
    run_full(wl, rope_base=0.0)


@pytest.mark.parametrize("seed", range(19))
def test_random_small_batches(seed):
    # Every decode kernel instantiation appears: per-wave (float32; bf16 G <= 4 over blocks
    # under 64 keys), lean one head per wave (bf16 G <= 4, blocks >= 64; d 64 and 128; its
    # two-stage form for G 2..4 at d 128: seeds 9, 17, 18),
    # lean two heads per wave (bf16 G 5..8, blocks >= 64; d 64 and 128) and grouped (bf16
    # G 9..16, or G 5..8 over blocks under 64 keys).
    combos = [  # dtype, Hq, Hkv, d, bs
        ("bf16", 4, 2, 64, 16), ("bf16", 8, 8, 128, 64), ("f32", 4, 1, 64, 32),
        ("bf16", 14, 2, 128, 32), ("f32", 8, 4, 128, 128), ("bf16", 16, 1, 64, 128),
        ("bf16", 8, 2, 128, 16), ("f32", 2, 2, 64, 64), ("bf16", 6, 2, 64, 64),
        ("bf16", 32, 8, 128, 64), ("f32", 4, 4, 128, 16), ("bf16", 3, 1, 128, 32),
        ("bf16", 16, 2, 128, 64), ("bf16", 24, 3, 64, 16), ("bf16", 12, 2, 64, 128),
        ("bf16", 40, 8, 128, 128), ("bf16", 7, 1, 64, 64), ("bf16", 4, 2, 128, 128),
        ("bf16", 6, 2, 128, 64),
    ]
    dt, Hq, Hkv, d, bs = combos[seed]
    wl = W.random_workload(seed, dtype=dt, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                           block_size=bs, max_new=150 if dt == "bf16" else 40,
                           max_seen=600, extra_ids=seed % 2)
    _say(f"case random seed={seed} {dt} Hq={Hq} Hkv={Hkv} d={d} bs={bs} T={wl.T} S={wl.S}")
    run_full(wl, rope_base=(0.0 if seed % 5 == 0 else 1e4))


def test_edge_single_key_and_tiny_chunks():
    # s = 0, n = 1 (one visible key: the output is V), n = 2 chunks, a chunk at s = 0
    for dt in ("bf16", "f32"):
        wl = W.random_workload(0, dtype=dt, n_q_heads=4, n_kv_heads=2, head_dim=64,
                               block_size=16, n_seqs=4)
        wl.n_new = np.array([1, 2, 1, 5], dtype=np.int32)
        wl.seen = np.array([0, 0, 63, 11], dtype=np.int32)
        need = [W.blocks_needed(a + b, 16) for a, b in zip(wl.n_new, wl.seen)]
        perm = np.random.default_rng(5).permutation(wl.num_blocks).astype(np.int32)
        at = np.cumsum([0] + need)
        wl.block_lists = [perm[at[i]:at[i + 1]] for i in range(4)]
        _say(f"case edge {dt}")
        run_full(wl)


def test_edge_capacity_limits_exact():
    """S = max_seqs and T = max_tokens exactly."""
    wl = W.random_workload(3, dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=128,
                           block_size=32, n_seqs=6, max_new=50, max_seen=200)
    wl.max_seqs = wl.S
    wl.max_tokens = wl.T
    _say(f"case capacity S={wl.S} T={wl.T}")
    run_full(wl)


def test_long_prefill_chunk_many_tiles():
    """One long chunk with a long history next to decodes: several query tiles and
    many key tiles, masked diagonal tiles, ragged tails."""
    wl = W.random_workload(7, dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=128,
                           block_size=64, n_seqs=3)
    wl.n_new = np.array([300, 1, 77], dtype=np.int32)
    wl.seen = np.array([700, 2000, 0], dtype=np.int32)
    need = [W.blocks_needed(a + b, 64) for a, b in zip(wl.n_new, wl.seen)]
    wl.num_blocks = sum(need) + 5
    perm = np.random.default_rng(9).permutation(wl.num_blocks).astype(np.int32)
    at = np.cumsum([0] + need)
    wl.block_lists = [perm[at[i]:at[i + 1]] for i in range(3)]
    _say("case long chunk")
    run_full(wl)


def test_empty_batch_on_gpu():
    wl = W.random_workload(1, dtype="bf16")
    eng = _engine(wl)
    b = eng.finalize([], [], [])
    assert b.S == 0 and b.T == 0
    qkv = torch.zeros(1, wl.qkv_heads, wl.head_dim, dtype=torch.bfloat16, device="cuda")
    pool = W.make_pool_history(wl, device="cuda")
    before = pool.clone()
    eng.append_rotary(qkv, pool, 1e4)
    eng.attention(qkv, pool, torch.empty(1, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(before, pool)


def test_rejects_host_memory_as_device_buffer():
    import ragged_blocked_kv_amd as R

    wl = W.random_workload(2, dtype="bf16")
    eng = _engine(wl)
    eng.finalize(wl.n_new, wl.seen, wl.block_lists)
    qkv_host = W.make_qkv(wl)  # CPU tensor
    pool = W.make_pool_history(wl, device="cuda")
    st = R.blocked_kv_append_rotary(eng.shape, eng.batch, qkv_host, pool, 1e4)
    assert st == R.ERR_DEVICE_PTR
    out_host = torch.empty(wl.T, wl.n_q_heads, wl.head_dim, dtype=torch.bfloat16)
    st = R.ragged_blocked_attention(eng.shape, eng.batch, qkv_host.cuda(), pool, out_host,
                                    eng.workspace, eng.workspace.numel())
    assert st == R.ERR_DEVICE_PTR


# ---------------------------------------------------------- full-size workloads ----


def _sample_seqs(wl, k_dec=4, k_chunk=2):
    """Longest and shortest sequences of each kind, plus seeded extras."""
    rng = np.random.default_rng(123)
    L = wl.seen + wl.n_new
    dec = np.nonzero(wl.n_new == 1)[0]
    chk = np.nonzero(wl.n_new > 1)[0]
    pick = []
    for idx, k in ((dec, k_dec), (chk, k_chunk)):
        if len(idx) == 0:
            continue
        order = idx[np.argsort(L[idx])]
        sel = {int(order[0]), int(order[-1])}
        extra = rng.permutation(idx)
        for e in extra:
            if len(sel) >= k:
                break
            sel.add(int(e))
        pick.extend(sorted(sel))
    return pick


def run_sampled(wl):
    """Full workload on the GPU (same launches the benchmark times); the oracle runs
    each sampled sequence alone on a sub-pool holding just that sequence's blocks."""
    eng = _engine(wl)
    qkv_in = W.make_qkv(wl)
    pool = W.make_pool_history(wl, device="cuda")
    seqs = _sample_seqs(wl)
    nb = [W.blocks_needed(int(a) + int(b), wl.block_size) for a, b in zip(wl.n_new, wl.seen)]
    hist = {i: _np_storage(pool[torch.as_tensor(wl.block_lists[i][:nb[i]].astype(np.int64),
                                                  device="cuda")]) for i in seqs}
    qkv = qkv_in.cuda()
    b = eng.finalize(wl.n_new, wl.seen, wl.block_lists)
    eng.append_rotary(qkv, pool, wl.rope_base)
    out = eng.new_out()
    eng.attention(qkv, pool, out)
    torch.cuda.synchronize()

    md = eng.metadata()
    ref_md = O.batch_metadata(wl.n_new, wl.seen, wl.block_lists, wl.block_size)
    for k in ref_md:
        assert np.array_equal(md[k], ref_md[k]), k
    check_work_coverage(md, b, wl)

    # canary: pool rows other than this pass's slots are unchanged
    fresh = W.make_pool_history(wl, device="cuda")
    changed = (fresh != pool).any(dim=4).any(dim=2).any(dim=1)  # [num_blocks, bs]
    written = torch.zeros_like(changed)
    blk = torch.as_tensor(ref_md["block_ids"][ref_md["block_offsets"][ref_md["token_to_seq"]] +
                                              ref_md["pos"] // wl.block_size].astype(np.int64),
                          device="cuda")
    slot = torch.as_tensor((ref_md["pos"] % wl.block_size).astype(np.int64), device="cuda")
    written[blk, slot] = True
    assert not bool((changed & ~written).any())
    # V placement bit exact for every token
    Hq, Hkv = wl.n_q_heads, wl.n_kv_heads
    assert torch.equal(pool[blk, 1, :, slot, :].cpu(), qkv_in[:, Hq + Hkv:])
    del fresh

    qkv_np = _np_storage(qkv_in)
    out_np = _np_storage(out)
    q_np = _np_storage(qkv)
    worst = 0.0
    for i in seqs:
        t0, t1 = int(ref_md["cu_seqlens"][i]), int(ref_md["cu_seqlens"][i + 1])
        sub_ids = np.arange(nb[i], dtype=np.int32)
        m1 = O.batch_metadata([wl.n_new[i]], [wl.seen[i]], [sub_ids], wl.block_size)
        q_ref, sub_pool = O.append_rotary(qkv_np[t0:t1], hist[i], m1, Hq, Hkv, wl.block_size,
                                          wl.rope_base, wl.dtype)
        _assert_within_one_ulp(q_np[t0:t1, :Hq], q_ref[:, :Hq], wl.dtype, f"Q seq {i}")
        pos = ref_md["pos"][t0:t1]
        gk = _np_storage(pool[blk[t0:t1], 0, :, slot[t0:t1], :])
        rk = sub_pool[pos // wl.block_size, 0, :, pos % wl.block_size, :]
        _assert_within_one_ulp(gk, rk, wl.dtype, f"K seq {i}")
        ref = O.ragged_attention(q_ref, sub_pool, m1, Hq, Hkv, wl.block_size, wl.dtype)
        got = O.storage_to_f64(out_np[t0:t1], wl.dtype)
        err = float(np.max(np.abs(got - ref)))
        worst = max(worst, err)
        assert err <= TOL[wl.dtype], f"{wl.name} seq {i}: max abs err {err}"
    # attention output is finite everywhere
    assert bool(torch.isfinite(out.float()).all())
    return worst


@pytest.mark.parametrize("name", ["decode_mha32", "splitfuse768_gqa4", "full8192_gqa4",
                                  "full8192_prefill_gqa4", "long_decode_gqa8"])
def test_full_size_workloads_sampled(name):
    wl = W.make_workload(name)
    _say(f"case {name} S={wl.S} T={wl.T} blocks={wl.num_blocks}")
    err = run_sampled(wl)
    _say(f"  {name}: worst sampled max-abs err {err:.3e}")
