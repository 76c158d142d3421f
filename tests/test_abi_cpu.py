"""The C ABI without a GPU: the library loads, exports what include/rbkv.h declares, the
size queries answer, and every argument error comes back as a status code before any
HIP call (fake addresses are fine for that reason)."""
import ctypes
import os
import re

import numpy as np
import pytest

import ragged_blocked_kv_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000  # never dereferenced: validation fails before any use


def header_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if not fn.endswith(".h"):
            continue
        txt = open(os.path.join(inc, fn)).read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", txt, flags=re.M))
    return sorted(names)


def shape(**kw):
    base = dict(max_tokens=64, max_seqs=8, num_blocks=32, block_size=16, n_q_heads=4,
                n_kv_heads=2, head_dim=64, dtype="bf16")
    base.update(kw)
    return R.Shape.make(**base)


def sizes(s):
    st, d, h = R.rbkv_metadata_bytes(s)
    assert st == R.OK
    return d, h


def finalize(s, n_new, seen, lists, **kw):
    d, h = sizes(s)
    args = dict(host_pinned=FAKE, host_pinned_bytes=h, dev_meta=FAKE, dev_meta_bytes=d)
    args.update(kw)
    return R.ragged_batch_finalize(s, n_new, seen, lists, args["host_pinned"],
                                   args["host_pinned_bytes"], args["dev_meta"],
                                   args["dev_meta_bytes"], None)


def test_library_exports_every_declared_function():
    fns = header_functions()
    assert set(fns) == set(R.EXPORTED_SYMBOLS), fns
    L = ctypes.CDLL(R.LIB_PATH)
    for f in fns:
        assert hasattr(L, f), f


def test_status_strings():
    for st in range(9):
        assert R.status_string(st) and R.status_string(st) != "unknown status"
    assert R.status_string(99) == "unknown status"


def test_metadata_bytes_and_shape_support():
    d, h = sizes(shape())
    assert d > h > 0 and d % 256 == 0
    # capacities scale the buffers
    d2, h2 = sizes(shape(max_tokens=8192, max_seqs=256, num_blocks=20000))
    assert d2 > d and h2 > h
    assert h2 >= 4 * (16 + 2 * 256 + 20000)
    for bad in [dict(head_dim=96), dict(head_dim=256), dict(block_size=48), dict(block_size=8),
                dict(dtype=7), dict(n_q_heads=6, n_kv_heads=4), dict(n_q_heads=64, n_kv_heads=2),
                dict(max_seqs=4096)]:
        assert R.rbkv_metadata_bytes(shape(**bad))[0] == R.ERR_UNSUPPORTED, bad
    for bad in [dict(max_tokens=0), dict(num_blocks=0), dict(n_kv_heads=0)]:
        assert R.rbkv_metadata_bytes(shape(**bad))[0] == R.ERR_INVALID_ARG, bad
    for ok in [dict(head_dim=128), dict(block_size=128), dict(dtype="f32"),
               dict(n_q_heads=14, n_kv_heads=2), dict(n_q_heads=32, n_kv_heads=2)]:
        assert R.rbkv_metadata_bytes(shape(**ok))[0] == R.OK, ok


def test_finalize_validation_errors():
    s = shape()
    lists = [np.array([0, 1, 2]), np.array([3])]
    # capacity
    assert finalize(s, [1] * 9, [0] * 9, [np.array([i]) for i in range(9)])[0] == R.ERR_CAPACITY
    assert finalize(s, [40, 30], [0, 0], [np.arange(3), np.arange(3, 5)])[0] == R.ERR_CAPACITY
    # bad counts
    assert finalize(s, [0, 1], [0, 0], lists)[0] == R.ERR_INVALID_ARG
    assert finalize(s, [1, 1], [-1, 0], lists)[0] == R.ERR_INVALID_ARG
    # block lists: too short, out of range, duplicated (within and across sequences)
    assert finalize(s, [20, 1], [13, 0], [np.array([0, 1]), np.array([3])])[0] == R.ERR_BLOCKS
    assert finalize(s, [1, 1], [0, 0], [np.array([32]), np.array([3])])[0] == R.ERR_BLOCKS
    assert finalize(s, [1, 1], [0, 0], [np.array([-1]), np.array([3])])[0] == R.ERR_BLOCKS
    assert finalize(s, [1, 1], [0, 0], [np.array([4]), np.array([4])])[0] == R.ERR_BLOCKS
    assert finalize(s, [20, 1], [0, 0], [np.array([4, 4]), np.array([5])])[0] == R.ERR_BLOCKS
    # more blocks needed than the pool holds
    assert finalize(s, [1], [600], [np.arange(40)])[0] == R.ERR_BLOCKS
    # buffers: too small, null
    d, h = sizes(s)
    assert finalize(s, [1], [0], [np.array([0])], host_pinned_bytes=h - 1)[0] == R.ERR_WORKSPACE
    assert finalize(s, [1], [0], [np.array([0])], dev_meta_bytes=d - 4)[0] == R.ERR_WORKSPACE
    assert finalize(s, [1], [0], [np.array([0])], host_pinned=None)[0] == R.ERR_INVALID_ARG
    assert finalize(s, [1], [0], [np.array([0])], dev_meta=None)[0] == R.ERR_INVALID_ARG
    # unsupported shape comes first
    st, _ = R.ragged_batch_finalize(shape(head_dim=80), [1], [0], [np.array([0])], FAKE, h,
                                    FAKE, d, None)
    assert st == R.ERR_UNSUPPORTED


def _expected_finalize_status(s, n_new, seen, lists):
    """The validation rules of ragged_batch_finalize, in the order the header states them
    (capacity, per-sequence counts, block coverage, block ids), for batches small enough
    never to reach the work-list caps; None means valid."""
    bs, nb = s.block_size, s.num_blocks
    if len(n_new) > s.max_seqs:
        return R.ERR_CAPACITY
    T = nblk = 0
    for n, sn, ids in zip(n_new, seen, lists):
        if n < 1 or sn < 0:
            return R.ERR_INVALID_ARG
        T += n
        if T > s.max_tokens:
            return R.ERR_CAPACITY
        B = -(-(sn + n) // bs)
        if B > nb or len(ids) < B:
            return R.ERR_BLOCKS
        nblk += B
        if nblk > nb:
            return R.ERR_BLOCKS
    used = set()
    for n, sn, ids in zip(n_new, seen, lists):
        for b in ids[: -(-(sn + n) // bs)]:
            if b < 0 or b >= nb or b in used:
                return R.ERR_BLOCKS
            used.add(int(b))
    return None


def test_finalize_random_validation():
    """Seeded random batches, each valid or carrying one kind of defect (too many
    sequences or tokens, a zero or negative count, a short block list, an id out of range,
    an id shared by two sequences): the status equals the rules above, and valid batches
    get past validation to the first HIP call."""
    import torch

    rng = np.random.default_rng(2024)
    s = shape(max_tokens=96, max_seqs=8, num_blocks=48, block_size=16)
    kinds = ["valid", "seqs", "tokens", "count", "seen", "short", "range", "dup"]
    seen_kinds = set()
    for case in range(400):
        kind = kinds[case % len(kinds)]
        S = int(rng.integers(1, s.max_seqs + 1))
        n_new = rng.integers(1, 12, size=S)
        seen = rng.integers(0, 40, size=S)
        if kind == "seqs":
            S = s.max_seqs + 1
            n_new, seen = np.ones(S, np.int64), np.zeros(S, np.int64)
        elif kind == "tokens":
            n_new[0] = s.max_tokens + 1 - (n_new.sum() - n_new[0])
        elif kind == "count":
            n_new[int(rng.integers(S))] = int(rng.integers(-3, 1))
        elif kind == "seen":
            seen[int(rng.integers(S))] = -int(rng.integers(1, 5))
        need = [max(0, -(-(int(a) + int(b)) // s.block_size)) for a, b in zip(n_new, seen)]
        ids = rng.permutation(s.num_blocks)
        lists, at = [], 0
        for b in need:
            take = ids[at:at + b] if at + b <= s.num_blocks else np.arange(b)
            lists.append(np.array(take, dtype=np.int32))
            at += b
        if kind == "short":
            i = int(rng.integers(S))
            lists[i] = lists[i][: max(0, len(lists[i]) - int(rng.integers(1, 3)))]
        elif kind == "range":
            i = int(rng.integers(S))
            if len(lists[i]):
                lists[i][int(rng.integers(len(lists[i])))] = rng.choice([-1, s.num_blocks, 10**6])
        elif kind == "dup" and S > 1 and len(lists[0]) and len(lists[-1]):
            lists[-1][-1] = lists[0][0]
        want = _expected_finalize_status(s, n_new.tolist(), seen.tolist(), lists)
        st, _ = finalize(s, n_new.astype(np.int32), seen.astype(np.int32), lists)
        if want is None:
            assert st in (R.ERR_DEVICE_PTR, R.ERR_HIP), (case, kind, st)
        else:
            assert st == want, (case, kind, st, want)
        seen_kinds.add(kind if want is not None else "valid")
    assert seen_kinds == set(kinds)


def test_finalize_null_lists_and_negative_S():
    s = shape()
    d, h = sizes(s)
    st, _ = R.ragged_batch_finalize(s, [1], [0], [np.array([0])], FAKE, h, FAKE, d, None,
                                    null_lists=True)
    assert st == R.ERR_INVALID_ARG
    st, _ = R.ragged_batch_finalize(s, [1], [0], [np.array([0])], FAKE, h, FAKE, d, None, S=-1)
    assert st == R.ERR_INVALID_ARG


def test_finalize_empty_batch_is_a_noop():
    s = shape()
    st, b = finalize(s, [], [], [])
    assert st == R.OK and b.S == 0 and b.T == 0 and b.n_decode_items == 0
    st, need = R.rbkv_workspace_bytes(s, b)
    assert st == R.OK and need == 0
    # T = 0: append and attention return OK without touching memory
    assert R.blocked_kv_append_rotary(s, b, FAKE, FAKE, 1e4) == R.OK
    assert R.ragged_blocked_attention(s, b, FAKE, FAKE, FAKE, None, 0) == R.OK


def test_append_and_attention_validation():
    s = shape()
    b = R.Batch()
    b.shape = s
    b.T = 3
    b.n_partials = 5
    # null buffers
    assert R.blocked_kv_append_rotary(s, b, None, FAKE, 1e4) == R.ERR_INVALID_ARG
    assert R.ragged_blocked_attention(s, b, FAKE, None, FAKE, FAKE, 1 << 20) == R.ERR_INVALID_ARG
    # batch built for another shape
    other = shape(head_dim=128)
    assert R.blocked_kv_append_rotary(other, b, FAKE, FAKE, 1e4) == R.ERR_INVALID_ARG
    assert R.ragged_blocked_attention(other, b, FAKE, FAKE, FAKE, FAKE, 1 << 20) == \
        R.ERR_INVALID_ARG
    # workspace: 5 partial slots of G * (d + 2) floats
    st, need = R.rbkv_workspace_bytes(s, b)
    assert st == R.OK and need == 5 * 2 * (64 + 2) * 4
    assert R.ragged_blocked_attention(s, b, FAKE, FAKE, FAKE, FAKE, need - 1) == R.ERR_WORKSPACE
    assert R.ragged_blocked_attention(s, b, FAKE, FAKE, FAKE, None, need) == R.ERR_WORKSPACE
    # T beyond capacity is a corrupted batch
    b.T = 65
    assert R.blocked_kv_append_rotary(s, b, FAKE, FAKE, 1e4) == R.ERR_INVALID_ARG


def test_noalloc_attention_validation():
    """The allocation-free call checks its arguments like the others and refuses a batch
    whose split-K partials exceed the static scratch, before any HIP call."""
    s = shape()
    b = R.Batch()
    b.shape = s
    b.T = 3
    b.n_partials = 5
    assert R.ragged_blocked_attention_noalloc(s, b, FAKE, None, FAKE) == R.ERR_INVALID_ARG
    assert R.ragged_blocked_attention_noalloc(shape(head_dim=128), b, FAKE, FAKE, FAKE) == \
        R.ERR_INVALID_ARG
    assert R.ragged_blocked_attention_noalloc(shape(head_dim=96), b, FAKE, FAKE, FAKE) == \
        R.ERR_UNSUPPORTED
    # partials of G * (d + 2) floats: just fitting, then one slot too many
    per = 2 * (64 + 2) * 4
    fit = R.STATIC_SCRATCH_BYTES // per
    b.n_partials = fit + 1
    assert R.rbkv_workspace_bytes(s, b)[1] > R.STATIC_SCRATCH_BYTES
    assert R.ragged_blocked_attention_noalloc(s, b, FAKE, FAKE, FAKE) == R.ERR_WORKSPACE
    b.T = 0  # an empty batch launches nothing, whatever its counts
    b.n_partials = fit
    assert R.ragged_blocked_attention_noalloc(s, b, FAKE, FAKE, FAKE) == R.OK


def test_workspace_holds_claim_counter_for_overlapped_decodes():
    """bf16 batches with both phases, groups of <= 8 heads and 64-key blocks get a
    256-byte-aligned item counter after the partials (the two-stream call's persistent
    decodes claim items from it), and so does every decode batch at head dim 128 with
    groups of 2-16 heads (the matrix-core decode is persistent in the serial call too);
    other shapes and batches do not."""
    def need(s, n_partials, n_dec, n_pre):
        b = R.Batch()
        b.shape = s
        b.T = 3
        b.n_partials, b.n_decode_items, b.n_prefill_items = n_partials, n_dec, n_pre
        st, n = R.rbkv_workspace_bytes(s, b)
        assert st == R.OK
        return n
    lean = shape(block_size=64)
    part = 5 * 2 * (64 + 2) * 4                      # 2640 bytes of partials
    assert need(lean, 5, 7, 2) == 2816 + 256         # partials rounded up to 256, + counter
    assert need(lean, 0, 7, 2) == 256                # unsplit decodes: the counter alone
    assert need(lean, 5, 7, 0) == part               # no prefill: no overlap, no counter
    assert need(lean, 5, 0, 2) == part
    # head dim 128, groups of 2-16: the serial call's decodes are persistent too
    lean128 = shape(block_size=64, head_dim=128)
    part128 = 5 * 2 * (128 + 2) * 4                  # 5200 bytes of partials
    assert need(lean128, 5, 7, 0) == 5376 + 256      # decode-only batch: counter as well
    assert need(lean128, 5, 0, 2) == part128         # no decode: no counter
    assert need(shape(block_size=64, head_dim=128, n_q_heads=2, n_kv_heads=2), 5, 7, 0) == \
        5 * 1 * (128 + 2) * 4                        # single-head groups: one workgroup per item
    assert need(shape(block_size=32), 5, 7, 2) == part          # blocks under 64 keys
    assert need(shape(block_size=64, dtype="f32"), 5, 7, 2) == part
    g8 = shape(block_size=64, n_q_heads=16, n_kv_heads=2)        # groups of 8 heads: counter
    assert need(g8, 5, 7, 2) == 10752 + 256          # 10560 bytes of partials, rounded
    g16 = shape(block_size=64, n_q_heads=32, n_kv_heads=2)       # groups of 16: none
    assert need(g16, 5, 7, 2) == 5 * 16 * (64 + 2) * 4
    # at head dim 128 groups of 8 and 16 heads decode on the matrix cores: counter in
    # decode-only batches too; blocks under 64 keys keep the per-item kernels
    g8_128 = shape(block_size=64, head_dim=128, n_q_heads=16, n_kv_heads=2)
    assert need(g8_128, 5, 7, 0) == 20992 + 256      # 20800 bytes of partials, rounded
    g16_128 = shape(block_size=64, head_dim=128, n_q_heads=32, n_kv_heads=2)
    assert need(g16_128, 5, 7, 2) == 41728 + 256     # 41600 bytes of partials, rounded
    assert need(g16_128, 5, 7, 0) == 41728 + 256
    assert need(shape(block_size=32, head_dim=128, n_q_heads=32, n_kv_heads=2), 5, 7, 0) == 41600


def test_valid_call_without_gpu_reports_pointer_kind():
    """With every argument valid the first HIP call is the pointer-kind check; on a
    machine without a GPU (or with fake addresses) it fails as DEVICE_PTR or HIP, never
    as a crash."""
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present; the GPU tests cover real buffers")
    s = shape()
    st, _ = finalize(s, [20, 1], [5, 3], [np.array([0, 1]), np.array([3])])
    assert st in (R.ERR_DEVICE_PTR, R.ERR_HIP)


def _fake_batch(S=2, T=5):
    b = R.Batch()
    b.shape = shape()
    b.S, b.T = S, T
    b.cu_seqlens = FAKE
    return b


def test_gather_validation_errors():
    b = _fake_batch()
    emb = lambda **kw: R.ragged_embedding_gather(
        kw.get("batch", b), kw.get("ids", FAKE), kw.get("table", FAKE), kw.get("vocab", 10),
        kw.get("width", 64), kw.get("dtype", "bf16"), kw.get("out", FAKE))
    lg = lambda **kw: R.ragged_logits_gather(
        kw.get("batch", b), kw.get("rows", FAKE), kw.get("width", 64),
        kw.get("dtype", "bf16"), kw.get("out", FAKE))
    for f in (emb, lg):
        assert f(width=0) == R.ERR_INVALID_ARG
        assert f(dtype=7) == R.ERR_INVALID_ARG
        assert f(width=3) == R.ERR_UNSUPPORTED        # 6-byte rows
        assert f(width=4, dtype="bf16") == R.ERR_UNSUPPORTED
        # 5 rows of 2^31 - 4 floats: more than 2^31 16-byte words
        assert f(width=(1 << 31) - 4, dtype="f32", batch=_fake_batch(S=5, T=5)) == \
            R.ERR_UNSUPPORTED
        assert f(out=FAKE + 8) == R.ERR_INVALID_ARG   # misaligned
        assert f(batch=_fake_batch(S=3, T=2)) == R.ERR_INVALID_ARG
        assert f(batch=_fake_batch(S=2, T=1 << 20)) == R.ERR_INVALID_ARG  # over max_tokens
    assert emb(vocab=0) == R.ERR_INVALID_ARG
    assert emb(ids=None) == R.ERR_INVALID_ARG
    assert emb(table=FAKE + 4) == R.ERR_INVALID_ARG
    assert lg(rows=None) == R.ERR_INVALID_ARG
    # empty batches launch nothing and touch no pointer
    assert emb(batch=_fake_batch(S=0, T=0)) == R.OK
    assert lg(batch=_fake_batch(S=0, T=0)) == R.OK


def test_kv_offload_validation_errors():
    s = shape()  # 32 blocks of [2][2][16][64] bf16 = 8 KiB
    st, b = R.rbkv_kv_host_bytes(s, 3)
    assert st == R.OK and b == 3 * 2 * 2 * 16 * 64 * 2 + 3 * 4
    assert R.rbkv_kv_host_bytes(s, -1)[0] == R.ERR_INVALID_ARG
    assert R.rbkv_kv_host_bytes(shape(head_dim=96), 1)[0] == R.ERR_UNSUPPORTED
    for fn in (R.blocked_kv_offload, R.blocked_kv_restore):
        assert fn(s, FAKE, [0, 1, 2], FAKE, b - 1) == R.ERR_INVALID_ARG  # buffer too small
        assert fn(s, None, [0], FAKE, b) == R.ERR_INVALID_ARG
        assert fn(s, FAKE, [0], None, b) == R.ERR_INVALID_ARG
        assert fn(s, FAKE, [0, 32, 1], FAKE, b) == R.ERR_BLOCKS       # out of range
        assert fn(s, FAKE, [-1], FAKE, b) == R.ERR_BLOCKS
        assert fn(s, FAKE, [], FAKE, 0) == R.OK                       # nothing to move
    # a restore may not write one block twice; an offload may read one twice
    assert R.blocked_kv_restore(s, FAKE, [4, 5, 4], FAKE, b) == R.ERR_BLOCKS


def test_concurrent_attention_argument_errors():
    s = shape()
    b = _fake_batch(S=2, T=5)
    b.n_prefill_items, b.n_decode_items = 1, 1
    f = lambda **kw: R.ragged_blocked_attention_concurrent(
        kw.get("shape", s), b, FAKE, FAKE, FAKE, None, 0, kw.get("stream", 0x10),
        kw.get("side", 0x20), kw.get("fork", 0x30), kw.get("join", 0x40))
    assert f(side=None) == R.ERR_INVALID_ARG
    assert f(fork=None) == R.ERR_INVALID_ARG
    assert f(join=None) == R.ERR_INVALID_ARG
    assert f(side=0x10) == R.ERR_INVALID_ARG  # the same stream twice
    assert f(shape=shape(head_dim=96)) == R.ERR_UNSUPPORTED  # checked before any fork


def test_attention_phase_values():
    """Phases 0..4 (ALL, PREFILL, DECODE, COMBINE, ATTEND) are accepted; anything else is
    INVALID_ARG before any other check.  An empty batch launches nothing in any phase."""
    s = shape()
    b = R.Batch()
    b.shape = s
    for bad in (-1, 5, 99):
        assert R.ragged_blocked_attention_phase(s, b, bad, FAKE, FAKE, FAKE, None, 0) == \
            R.ERR_INVALID_ARG
    assert (R.PHASE_ALL, R.PHASE_PREFILL, R.PHASE_DECODE, R.PHASE_COMBINE, R.PHASE_ATTEND) == \
        (0, 1, 2, 3, 4)
    for ph in range(5):
        assert R.ragged_blocked_attention_phase(s, b, ph, FAKE, FAKE, FAKE, None, 0) == R.OK
