"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded
inputs.  Metadata is compared bit for bit; V placement (and K placement with rotation
off) bit for bit; rotated Q/K within one storage ulp (bf16) or 1e-5 (float32); pool
bytes outside the written slots unchanged; attention within max-abs 2e-2 (bf16) or
1e-4 (float32).  Outputs start as NaN, so a row that no work item wrote fails.  Small
batches are compared element by element in full; the five full-size workloads (in the
launch configuration the benchmark times, serial and two-stream) on every row, the
oracle computing each sequence alone.  Work lists are checked for exact coverage of
every (token, query head, key)."""
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


def run_full(wl, rope_base=None, check_coverage=True, concurrent=False):
    """Whole batch through GPU and oracle; compares everything element by element.
    Outputs start as NaN, so a row that no work item wrote fails.  With ``concurrent``
    the two-stream call runs too (into its own output) and is compared the same way."""
    base = wl.rope_base if rope_base is None else rope_base
    eng = _engine(wl)
    qkv_in = W.make_qkv(wl)
    pool_in = W.make_pool_history(wl, device="cpu")
    qkv = qkv_in.cuda()
    pool = pool_in.cuda()
    b = eng.finalize(wl.n_new, wl.seen, wl.block_lists)
    eng.append_rotary(qkv, pool, base)
    outs = {"serial": eng.new_out().fill_(float("nan"))}
    eng.attention(qkv, pool, outs["serial"])
    if concurrent:
        outs["two-stream"] = eng.new_out().fill_(float("nan"))
        eng.attention_concurrent(qkv, pool, outs["two-stream"])
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
    worst = 0.0
    for which, out in outs.items():
        got = O.storage_to_f64(_np_storage(out), wl.dtype)
        assert np.isfinite(got).all(), f"{wl.name} ({which}): rows not written"
        err = float(np.max(np.abs(got - ref)))
        assert err <= TOL[wl.dtype], f"{wl.name} ({which}): max abs err {err}"
        worst = max(worst, err)
    return worst, b, eng.metadata()


# ---------------------------------------------------------------- small batches ----


def test_tiny_f32_workload():
    wl = W.make_workload("tiny_f32")
    _say(f"case tiny_f32 T={wl.T}")
    run_full(wl)
    run_full(wl, rope_base=0.0)


@pytest.mark.parametrize("seed", range(19))
def test_random_small_batches(seed):
    # Every decode kernel appears: per-wave (float32; bf16 G <= 4 over blocks under 64
    # keys), matrix-core (bf16 d 128, G 2..16, blocks >= 64: seeds 9, 12, 15, 17, 18),
    # register-only (bf16 d 128, G 1, blocks >= 64: seed 1), lean one head per wave (bf16
    # d 64, G <= 4, blocks >= 64), lean two heads per wave (bf16 d 64, G 5..8, blocks >=
    # 64) and grouped (bf16 G 9..16 at d 64, or G 5..16 over blocks under 64 keys).
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


MIXED_CASES = [  # name, Hq, Hkv, bs, (n_new, seen) per sequence: batches of the mixed launch
    # many chunks and one decode: the decode list runs dry at once, its workgroups move on
    ("one_decode_many_chunks", 16, 4, 64,
     [(300, 500), (257, 0), (64, 2000), (1, 3000), (129, 64), (400, 1000), (77, 7)]),
    # one short chunk and many decodes at groups of 16 over 128-key blocks
    ("one_chunk_many_decodes_g16", 32, 2, 128,
     [(45, 900)] + [(1, 300 + 97 * i) for i in range(40)]),
    # one chunk and one decode with two kv heads: fewer kv groups than XCDs, so most
    # XCDs' chunk lists are empty from the start and their workgroups take other lists
    ("tiny_two_groups", 8, 2, 64, [(70, 130), (1, 5000)]),
]


@pytest.mark.parametrize("case", [c[0] for c in MIXED_CASES])
def test_mixed_launch_edges(case):
    """Batches the library runs as one mixed launch of chunk tiles and decode items, at
    the edges of its work sharing; serial and concurrent calls against the oracle."""
    name, Hq, Hkv, bs, seqs = next(c for c in MIXED_CASES if c[0] == case)
    wl = W.random_workload(71, dtype="bf16", n_q_heads=Hq, n_kv_heads=Hkv, head_dim=128,
                           block_size=bs, n_seqs=len(seqs))
    wl.n_new = np.array([a for a, _ in seqs], dtype=np.int32)
    wl.seen = np.array([b for _, b in seqs], dtype=np.int32)
    need = [W.blocks_needed(a + b, bs) for a, b in seqs]
    wl.num_blocks = sum(need) + 3
    perm = np.random.default_rng(72).permutation(wl.num_blocks).astype(np.int32)
    at = np.cumsum([0] + need)
    wl.block_lists = [perm[at[i]:at[i + 1]] for i in range(len(seqs))]
    wl.max_tokens = max(wl.max_tokens, int(wl.n_new.sum()))
    wl.max_seqs = max(wl.max_seqs, len(seqs))
    _say(f"case mixed {name}")
    run_full(wl, concurrent=True)


def _mixed_random_workload(seed):
    """A random batch with both chunks and decodes for the mixed launch (redrawn under a
    derived seed until it has both)."""
    for attempt in range(50):
        rng = np.random.default_rng(900 + seed + 1000 * attempt)
        G = int(rng.choice([2, 3, 4, 6, 8, 12, 16]))
        Hkv = int(rng.choice([1, 2, 4])) if G <= 8 else int(rng.choice([1, 2]))
        bs = int(rng.choice([64, 128]))
        frac = float(rng.choice([0.1, 0.3, 0.5, 0.7, 0.9]))
        wl = W.random_workload(900 + seed + 1000 * attempt, dtype="bf16", n_q_heads=G * Hkv,
                               n_kv_heads=Hkv, head_dim=128, block_size=bs,
                               n_seqs=int(rng.integers(4, 40)),
                               max_new=int(rng.choice([40, 150, 400])),
                               max_seen=int(rng.choice([200, 1500, 6000])), decode_frac=frac,
                               max_tokens=20000)
        if (wl.n_new > 1).any() and (wl.n_new == 1).any():
            return wl, G, Hkv, bs
    raise AssertionError("no mixed draw")


@pytest.mark.parametrize("seed", range(12))
def test_mixed_launch_random(seed):
    """Random batches of the mixed launch (bf16, head dim 128, groups of 2-16 heads, 64- or
    128-key blocks) with every balance of chunks and decodes, from nearly all decodes to
    nearly all chunks; serial and concurrent calls against the oracle."""
    wl, G, Hkv, bs = _mixed_random_workload(seed)
    _say(f"case mixed random seed={seed} G={G} Hkv={Hkv} bs={bs} S={wl.S} T={wl.T}")
    run_full(wl, concurrent=True)


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


@pytest.mark.parametrize("d,bs", [(128, 64), (128, 16), (64, 32), (128, 128), (64, 128)])
def test_prefill_key_tile_counts(d, bs):
    """Chunks only (the prefill launch alone): work items that see 1, 2, 3 and 4 key
    tiles (64 keys each) and key counts one past and one short of a tile edge, so the
    tile-load schedule's prologue and last steps run with every short count; blocks of
    16 and 32 keys (a tile spans several blocks), 64 and 128 (a tile lies in one block)."""
    seqs = [(64, 0), (2, 63), (64, 64), (65, 63), (3, 126), (64, 128), (10, 183), (200, 0),
            (129, 255)]
    wl = W.random_workload(11, dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=d,
                           block_size=bs, n_seqs=len(seqs))
    wl.n_new = np.array([a for a, _ in seqs], dtype=np.int32)
    wl.seen = np.array([b for _, b in seqs], dtype=np.int32)
    need = [W.blocks_needed(a + b, bs) for a, b in seqs]
    wl.num_blocks = sum(need) + 3
    perm = np.random.default_rng(13).permutation(wl.num_blocks).astype(np.int32)
    at = np.cumsum([0] + need)
    wl.block_lists = [perm[at[i]:at[i + 1]] for i in range(len(seqs))]
    _say(f"case prefill tile counts d={d} bs={bs}")
    run_full(wl, concurrent=True)


SPLIT_CASES = [  # name, dtype, Hq, Hkv, d, bs, (n_new, seen) per sequence
    # matrix-core kernel (G 4, d 128), one long decode beside a chunk
    ("mfma_g4_d128", "bf16", 8, 2, 128, 64, [(1, 20000), (40, 300), (1, 150), (1, 5000)]),
    # matrix-core kernel (G 8)
    ("mfma_g8_d128", "bf16", 16, 2, 128, 64, [(1, 30000), (1, 900), (33, 2000)]),
    # matrix-core kernel (G 12) over 128-key blocks, with items that some waves see no
    # key of (40 keys) and a one-key decode
    ("mfma_g12_bs128", "bf16", 24, 2, 128, 128, [(1, 9000), (1, 40), (21, 500), (1, 0)]),
    # lean two heads per wave (G 8, d 64)
    ("lean2_g8_d64", "bf16", 16, 2, 64, 64, [(1, 24000), (1, 700), (19, 900)]),
    # lean one head per wave, one stage (G 1, d 64)
    ("lean_g1_d64", "bf16", 2, 2, 64, 128, [(1, 16000), (25, 100), (1, 63)]),
    # register-only kernel (G 1, d 128), with short items a wave sees no key of
    ("reg_g1_d128", "bf16", 4, 4, 128, 64, [(1, 14000), (30, 200), (1, 20), (1, 70)]),
    # matrix-core kernel (G 16)
    ("mfma_g16_d128", "bf16", 32, 2, 128, 64, [(1, 12000), (1, 1), (17, 4000)]),
    # grouped kernel (G 16, d 64)
    ("grouped_g16_d64", "bf16", 32, 2, 64, 64, [(1, 12000), (1, 1), (17, 4000)]),
    # per-wave kernel, bf16 over 16-key blocks
    ("perwave_g2_bf16", "bf16", 4, 2, 128, 16, [(1, 9000), (1, 777), (9, 50)]),
    # per-wave kernel, float32
    ("perwave_g2_f32", "f32", 4, 2, 64, 32, [(1, 12000), (1, 3000), (12, 80)]),
]


@pytest.mark.parametrize("case", [c[0] for c in SPLIT_CASES])
def test_long_decode_many_splits(case):
    """One long decode in a small batch is cut into dozens of splits (MIN_SPLIT_TILES
    keeps splits at four tiles), so the combine merges its partials over several of its
    load batches, each rescaling the sums of the ones before.  The serial and the
    two-stream call are both compared with the oracle."""
    name, dt, Hq, Hkv, d, bs, seqs = next(c for c in SPLIT_CASES if c[0] == case)
    wl = W.random_workload(61, dtype=dt, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                           block_size=bs, n_seqs=len(seqs))
    wl.n_new = np.array([a for a, _ in seqs], dtype=np.int32)
    wl.seen = np.array([b for _, b in seqs], dtype=np.int32)
    need = [W.blocks_needed(a + b, bs) for a, b in seqs]
    wl.num_blocks = sum(need) + 3
    perm = np.random.default_rng(62).permutation(wl.num_blocks).astype(np.int32)
    at = np.cumsum([0] + need)
    wl.block_lists = [perm[at[i]:at[i + 1]] for i in range(len(seqs))]
    _say(f"case many splits {name}")
    err, b, md = run_full(wl, concurrent=True)
    most = int(md["combine_work"][:, 3].max())
    assert most >= 32, f"only {most} splits"
    _say(f"  {name}: {most} splits, max-abs err {err:.3e}")


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
#
# Every sequence of every full-size workload is compared with the oracle, in the launch
# configuration the benchmark times (the serial call and the two-stream call, each into
# its own NaN-filled output, so a row no work item wrote fails).  The GPU pass runs once
# per workload (cached across its parts); each part then checks a share of the
# sequences, so no single test runs long.  The oracle takes each sequence alone on a
# sub-pool of just its blocks, read from a pool regenerated from the same seed (the
# pre-append history), so no host copy of a whole pool is ever made.

FULL_PARTS = {"decode_mha32": 1, "splitfuse768_gqa4": 1, "full8192_gqa4": 4,
              "full8192_prefill_gqa4": 2, "long_decode_gqa8": 4}
_FULL = {}


def _full_gpu_pass(name):
    """GPU side of one full-size workload, shared by its parts: finalize, append, the
    serial and the two-stream attention; whole-batch checks of metadata, work coverage,
    pool canaries and V placement."""
    if name in _FULL:
        return _FULL[name]
    _FULL.clear()
    torch.cuda.empty_cache()
    wl = W.make_workload(name)
    _say(f"gpu pass {name} S={wl.S} T={wl.T} blocks={wl.num_blocks}")
    eng = _engine(wl)
    qkv_in = W.make_qkv(wl)
    pool = W.make_pool_history(wl, device="cuda")
    qkv = qkv_in.cuda()
    b = eng.finalize(wl.n_new, wl.seen, wl.block_lists)
    eng.append_rotary(qkv, pool, wl.rope_base)
    out_s = eng.new_out().fill_(float("nan"))
    out_c = eng.new_out().fill_(float("nan"))
    eng.attention(qkv, pool, out_s)
    eng.attention_concurrent(qkv, pool, out_c)
    torch.cuda.synchronize()

    md = eng.metadata()
    ref_md = O.batch_metadata(wl.n_new, wl.seen, wl.block_lists, wl.block_size)
    for k in ref_md:
        assert np.array_equal(md[k], ref_md[k]), k
    check_work_coverage(md, b, wl)

    # the history before this pass's append, regenerated from the same seed
    fresh = W.make_pool_history(wl, device="cuda")
    # canary: pool rows other than this pass's slots are unchanged
    changed = (fresh != pool).any(dim=4).any(dim=2).any(dim=1)  # [num_blocks, bs]
    written = torch.zeros_like(changed)
    blk = torch.as_tensor(ref_md["block_ids"][ref_md["block_offsets"][ref_md["token_to_seq"]] +
                                              ref_md["pos"] // wl.block_size].astype(np.int64),
                          device="cuda")
    slot = torch.as_tensor((ref_md["pos"] % wl.block_size).astype(np.int64), device="cuda")
    written[blk, slot] = True
    assert not bool((changed & ~written).any())
    del changed, written
    # V placement bit exact for every token
    Hq, Hkv = wl.n_q_heads, wl.n_kv_heads
    assert torch.equal(pool[blk, 1, :, slot, :].cpu(), qkv_in[:, Hq + Hkv:])
    st = {
        "wl": wl, "ref_md": ref_md, "fresh": fresh,
        "qkv_in": _np_storage(qkv_in), "q": _np_storage(qkv),
        "k_new": _np_storage(pool[blk, 0, :, slot, :]),
        "out_s": _np_storage(out_s), "out_c": _np_storage(out_c),
        "checked": set(), "parts": set(),
    }
    del pool
    _FULL[name] = st
    return st


def check_full_part(name, part):
    """The oracle on this part's sequences (every nparts-th one), each alone on a
    sub-pool of its own blocks: rotated Q and K within one ulp, attention of the serial
    and the two-stream call within tolerance, every row of both."""
    st = _full_gpu_pass(name)
    wl, ref_md = st["wl"], st["ref_md"]
    Hq, Hkv, bs = wl.n_q_heads, wl.n_kv_heads, wl.block_size
    nparts = FULL_PARTS[name]
    worst = {"serial": 0.0, "two-stream": 0.0}
    seqs = list(range(part, wl.S, nparts))
    for i in seqs:
        t0, t1 = int(ref_md["cu_seqlens"][i]), int(ref_md["cu_seqlens"][i + 1])
        nb = int(ref_md["block_offsets"][i + 1] - ref_md["block_offsets"][i])
        ids = ref_md["block_ids"][int(ref_md["block_offsets"][i]):][:nb].astype(np.int64)
        hist = _np_storage(st["fresh"][torch.as_tensor(ids, device="cuda")])
        m1 = O.batch_metadata([wl.n_new[i]], [wl.seen[i]], [np.arange(nb, dtype=np.int32)], bs)
        q_ref, sub_pool = O.append_rotary(st["qkv_in"][t0:t1], hist, m1, Hq, Hkv, bs,
                                          wl.rope_base, wl.dtype)
        _assert_within_one_ulp(st["q"][t0:t1, :Hq], q_ref[:, :Hq], wl.dtype, f"Q seq {i}")
        pos = ref_md["pos"][t0:t1]
        rk = sub_pool[pos // bs, 0, :, pos % bs, :]
        _assert_within_one_ulp(st["k_new"][t0:t1], rk, wl.dtype, f"K seq {i}")
        ref = O.ragged_attention(q_ref, sub_pool, m1, Hq, Hkv, bs, wl.dtype)
        for which, key in (("serial", "out_s"), ("two-stream", "out_c")):
            got = O.storage_to_f64(st[key][t0:t1], wl.dtype)
            assert np.isfinite(got).all(), f"{name} seq {i} ({which}): rows not written"
            err = float(np.max(np.abs(got - ref)))
            worst[which] = max(worst[which], err)
            assert err <= TOL[wl.dtype], f"{name} seq {i} ({which}): max abs err {err}"
        st["checked"].add(i)
    st["parts"].add(part)
    if len(st["parts"]) == nparts:
        assert st["checked"] == set(range(wl.S))  # every sequence of the batch compared
    return len(seqs), worst


@pytest.mark.parametrize("name,part", [(n, p) for n, k in FULL_PARTS.items() for p in range(k)])
@pytest.mark.timeout(300)
def test_full_size_workloads_every_row(name, part):
    _say(f"case {name} part {part + 1}/{FULL_PARTS[name]}")
    n, worst = check_full_part(name, part)
    _say(f"  {name} part {part + 1}: {n} sequences, worst max-abs err serial "
         f"{worst['serial']:.3e}, two-stream {worst['two-stream']:.3e}")
    if len(_FULL[name]["parts"]) == FULL_PARTS[name]:
        _FULL.clear()
        torch.cuda.empty_cache()
