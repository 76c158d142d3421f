"""Pins for the CPU oracle: each test checks the oracle against something other than
itself -- hand-derived fixtures, closed forms, brute force in separate code,
invariants and special cases that reduce to a textbook or library routine.  A
plausible slip in the oracle (a dropped scale, a wrong sign or pair index, a shifted
position, a transposed operand, top-left instead of bottom-right causal alignment)
fails at least one of them."""
import cmath
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ bf16 storage ----


def _bf16_nearest_bruteforce(x: float) -> int:
    """Nearest bfloat16 pattern by search over ordered patterns and exact rational
    comparison; ties go to the even pattern."""
    if x == 0.0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0
    sign = 0x8000 if x < 0 else 0
    ax = Fraction(abs(x))

    def val(p):
        return Fraction(float(np.array([p << 16], dtype=np.uint32).view(np.float32)[0]))

    lo, hi = 0, 0x7F7F  # largest finite pattern
    while lo < hi:  # largest pattern with value <= ax
        mid = (lo + hi + 1) // 2
        if val(mid) <= ax:
            lo = mid
        else:
            hi = mid - 1
    a, b = lo, lo + 1
    da, db = ax - val(a), val(b) - ax
    if da < db:
        p = a
    elif db < da:
        p = b
    else:
        p = a if a % 2 == 0 else b
    return sign | p


def test_bf16_rne_matches_bruteforce():
    rng = np.random.default_rng(1)
    xs = np.concatenate([
        rng.standard_normal(300),
        rng.standard_normal(100) * 1e-20,
        rng.standard_normal(100) * 1e20,
        # exact ties and near-ties at several binades
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -30, 1 + 2 ** -8 - 2 ** -40,
                  -(2 + 2 ** -7), 3.0, -0.0, 0.0, 2.0 ** -126, 1.5 * 2.0 ** 100]),
    ])
    got = O.bf16_from_f64(xs)
    want = np.array([_bf16_nearest_bruteforce(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_bf16_rne_rounds_once_from_binary64():
    # 1 + 2^-8 + 2^-30 lies just above the midpoint between 1 and 1 + 2^-7.  Rounding
    # through binary32 first would land exactly on the midpoint and tie down to 1.0.
    assert int(O.bf16_from_f64(np.array([1 + 2 ** -8 + 2 ** -30]))[0]) == 0x3F81
    assert int(O.bf16_from_f64(np.array([1 + 2 ** -8]))[0]) == 0x3F80  # tie -> even
    assert int(O.bf16_from_f64(np.array([1 + 3 * 2 ** -8]))[0]) == 0x3F82  # tie -> even


def test_bf16_matches_torch_cast_on_binary32_values():
    import torch

    rng = np.random.default_rng(2)
    x32 = (rng.standard_normal(4096) * np.exp(rng.uniform(-20, 20, 4096))).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.bf16_from_f64(x32.astype(np.float64))
    assert np.array_equal(got, want)
    back = O.bf16_to_f64(want)
    assert np.array_equal(back, torch.from_numpy(want.view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy())


# ------------------------------------------------------------------ metadata ----


def test_metadata_matches_hand_derived_fixture():
    g = json.load(open(os.path.join(GOLDEN, "tiny_f32_metadata.json")))
    wl = W.make_workload("tiny_f32")
    assert list(wl.n_new) == g["n_new"] and list(wl.seen) == g["seen"]
    m = O.batch_metadata(wl.n_new, wl.seen, wl.block_lists, g["block_size"])
    assert m["cu_seqlens"].tolist() == g["cu_seqlens"]
    assert m["kv_len"].tolist() == g["kv_len"]
    assert m["block_offsets"].tolist() == g["block_offsets"]
    t2s = sum(([s] * c for s, c in g["token_to_seq_runs"]), [])
    assert m["token_to_seq"].tolist() == t2s
    pos = sum((list(range(a, a + c)) for a, c in g["pos_runs"]), [])
    assert m["pos"].tolist() == pos
    flat = sum((list(wl.block_lists[i][:b]) for i, b in enumerate(np.diff(g["block_offsets"]))),
               [])
    assert m["block_ids"].tolist() == flat


@pytest.mark.parametrize("seed", range(8))
def test_metadata_invariants(seed):
    wl = W.random_workload(seed, extra_ids=seed % 3, block_size=[16, 32, 64, 128][seed % 4])
    m = O.batch_metadata(wl.n_new, wl.seen, wl.block_lists, wl.block_size)
    cu, t2s, pos = m["cu_seqlens"], m["token_to_seq"], m["pos"]
    assert cu[0] == 0 and cu[-1] == wl.T and len(t2s) == wl.T and len(pos) == wl.T
    for t in range(wl.T):  # every token lies inside its owner's range, at seen + offset
        i = t2s[t]
        assert cu[i] <= t < cu[i + 1]
        assert pos[t] - wl.seen[i] == t - cu[i]
    bo = m["block_offsets"]
    for i in range(wl.S):
        nb = bo[i + 1] - bo[i]
        L = m["kv_len"][i]
        assert (nb - 1) * wl.block_size < L <= nb * wl.block_size  # just enough blocks
        assert list(m["block_ids"][bo[i]:bo[i + 1]]) == list(wl.block_lists[i][:nb])
    assert len(set(m["block_ids"].tolist())) == len(m["block_ids"])


def test_metadata_rejects_short_block_list():
    with pytest.raises(ValueError):
        O.batch_metadata([3], [14], [np.array([5], dtype=np.int32)], 16)


# ------------------------------------------------------------------ rotary ----


def test_rope_hand_examples():
    g = json.load(open(os.path.join(GOLDEN, "rope_d4_examples.json")))
    d, base = g["head_dim"], g["base"]
    assert np.allclose(O.rope_inv_freq(d, base), g["theta"], rtol=0, atol=1e-17)
    env = {"cos": math.cos, "sin": math.sin}
    for c in g["cases"]:
        got = O.rotate(np.array(c["x"], dtype=np.float64), O.rope_angles([c["p"]], d, base)[0])
        want = [eval(e, env) for e in c["expect"]]
        assert np.allclose(got, want, rtol=0, atol=1e-15), (c, got)


def test_rope_d2_is_complex_multiply():
    rng = np.random.default_rng(3)
    for p in [0, 1, 7, 1234, 40000]:
        x = rng.standard_normal(2)
        got = O.rotate(x, O.rope_angles([p], 2, 10000.0)[0])
        z = complex(x[0], x[1]) * cmath.exp(1j * p)  # theta_0 = 1 for any base
        assert abs(got[0] - z.real) < 1e-11 and abs(got[1] - z.imag) < 1e-11


def test_rope_invariants():
    rng = np.random.default_rng(4)
    d, base = 128, 1e6
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    rot = lambda x, p: O.rotate(x, O.rope_angles([p], d, base)[0])
    assert np.array_equal(rot(q, 0), q)  # position 0 is the identity
    r = rot(q, 977)
    h = d // 2
    assert np.allclose(q[:h] ** 2 + q[h:] ** 2, r[:h] ** 2 + r[h:] ** 2, atol=1e-12)
    # relative position: <R_m q, R_n k> depends only on n - m
    for m, n, c in [(3, 10, 100), (0, 500, 4000), (8000, 8001, 31000)]:
        assert abs(rot(q, m) @ rot(k, n) - rot(q, m + c) @ rot(k, n + c)) < 1e-9
    # rotations compose: R_a R_b = R_{a+b}
    a, b = O.rope_angles([11], d, base)[0], O.rope_angles([29], d, base)[0]
    assert np.allclose(O.rotate(O.rotate(q, a), b), O.rotate(q, a + b), atol=1e-12)


# ------------------------------------------------------------------ append ----


def _setup(wl, pool_device="cpu"):
    qkv = W.make_qkv(wl)
    pool = W.make_pool_history(wl, device=pool_device)
    if wl.dtype == "bf16":
        import torch

        to_np = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    else:
        to_np = lambda t: t.numpy()
    return to_np(qkv), to_np(pool)


@pytest.mark.parametrize("seed", range(4))
def test_append_placement_bruteforce(seed):
    """With rotation off, every new K/V row must appear in exactly the slot its
    sequence's block list assigns to its position, found by scanning the whole pool
    for the (unique, random) row; every other pool row is unchanged."""
    wl = W.random_workload(seed, dtype="bf16" if seed % 2 else "f32", n_q_heads=4,
                           n_kv_heads=2, head_dim=64, block_size=[16, 32][seed % 2],
                           extra_ids=seed % 2)
    qkv, pool = _setup(wl)
    m = O.batch_metadata(wl.n_new, wl.seen, wl.block_lists, wl.block_size)
    q2, p2 = O.append_rotary(qkv, pool, m, 4, 2, wl.block_size, 0.0, wl.dtype)
    assert np.array_equal(q2, qkv)
    written = np.zeros(pool.shape[:2] + (pool.shape[3],), dtype=bool)  # [blk][kv][slot]
    t = 0
    for i in range(wl.S):
        for k in range(int(wl.n_new[i])):
            p = int(wl.seen[i]) + k
            for kv in (0, 1):
                row = qkv[t, 4 + 2 * kv:4 + 2 * kv + 2]  # [Hkv][d] of K (kv=0) or V
                hits = [(b, s) for b in range(pool.shape[0]) for s in range(pool.shape[3])
                        if np.array_equal(p2[b, kv, :, s, :], row)]
                assert hits == [(int(wl.block_lists[i][p // wl.block_size]),
                                 p % wl.block_size)]
                written[hits[0][0], kv, hits[0][1]] = True
            t += 1
    untouched = ~written
    a = np.moveaxis(p2, 3, 2)[untouched]
    b = np.moveaxis(pool, 3, 2)[untouched]
    assert np.array_equal(a, b)


def test_append_rotates_q_and_k_at_absolute_positions():
    wl = W.random_workload(5, dtype="f32", n_q_heads=4, n_kv_heads=2, head_dim=64,
                           block_size=16)
    qkv, pool = _setup(wl)
    m = O.batch_metadata(wl.n_new, wl.seen, wl.block_lists, wl.block_size)
    q2, p2 = O.append_rotary(qkv, pool, m, 4, 2, 16, 1e4, "f32")
    t = 0
    for i in range(wl.S):
        for k in range(int(wl.n_new[i])):
            p = int(wl.seen[i]) + k
            for h in range(8):  # 4 Q heads then 2 K heads then 2 V heads
                x = qkv[t, h].astype(np.float64)
                if h < 6:  # rotate Q and K; each pair j, j + 32 turns by p * 1e4^(-j/32)
                    ang = p * 10000.0 ** (-np.arange(32) / 32.0)
                    want = np.concatenate([x[:32] * np.cos(ang) - x[32:] * np.sin(ang),
                                           x[32:] * np.cos(ang) + x[:32] * np.sin(ang)])
                else:
                    want = x
                if h < 4:
                    got = q2[t, h]
                else:
                    kv, g = (0, h - 4) if h < 6 else (1, h - 6)
                    got = p2[int(wl.block_lists[i][p // 16]), kv, g, p % 16]
                assert np.allclose(got.astype(np.float64), want, rtol=0, atol=2e-6)
            t += 1
    assert np.array_equal(q2[:, 4:], qkv[:, 4:])  # K and V rows of qkv are untouched


# ------------------------------------------------------------------ attention ----


def _bruteforce_attention(q, K, V, seen, G):
    """Dense causal attention of one sequence with Python loops over plain floats.
    q: [n][Hq][d]; K, V: [L][Hkv][d] contiguous; the query at offset k of the chunk
    sits at position seen + k and sees keys 0 .. seen + k."""
    n, Hq, d = q.shape
    out = np.zeros((n, Hq, d))
    for t in range(n):
        last = seen + t
        for h in range(Hq):
            g = h // G
            z = [sum(float(q[t, h, c]) * float(K[j, g, c]) for c in range(d)) / math.sqrt(d)
                 for j in range(last + 1)]
            mx = max(z)
            e = [math.exp(v - mx) for v in z]
            s = sum(e)
            for c in range(d):
                out[t, h, c] = sum(e[j] * float(V[j, g, c]) for j in range(last + 1)) / s
    return out


def _pool_from_contiguous(Ks, Vs, block_size, rng, spare=3):
    """Scatter per-sequence contiguous K/V into a pool at a random block permutation."""
    Hkv, d = Ks[0].shape[1], Ks[0].shape[2]
    need = [-(-len(K) // block_size) for K in Ks]
    nb = sum(need) + spare
    pool = rng.standard_normal((nb, 2, Hkv, block_size, d))  # garbage in unused slots
    perm = rng.permutation(nb)
    lists, at = [], 0
    for K, V, b in zip(Ks, Vs, need):
        ids = perm[at:at + b]
        at += b
        lists.append(ids.astype(np.int32))
        for p in range(len(K)):
            pool[ids[p // block_size], 0, :, p % block_size] = K[p]
            pool[ids[p // block_size], 1, :, p % block_size] = V[p]
    return pool.astype(np.float32), lists


def _oracle_on_contiguous(qs, Ks, Vs, seens, block_size, rng):
    """Run the oracle's gather + attention on a pool built from contiguous K/V."""
    pool, lists = _pool_from_contiguous(Ks, Vs, block_size, rng)
    n_new = [q.shape[0] for q in qs]
    m = O.batch_metadata(n_new, seens, lists, block_size)
    Hq, d = qs[0].shape[1], qs[0].shape[2]
    Hkv = Ks[0].shape[1]
    qkv = np.zeros((sum(n_new), Hq + 2 * Hkv, d), dtype=np.float32)
    qkv[:, :Hq] = np.concatenate(qs)
    return O.ragged_attention(qkv, pool, m, Hq, Hkv, block_size, "f32")


@pytest.mark.parametrize("G", [1, 2])
def test_attention_matches_bruteforce_dense(G):
    rng = np.random.default_rng(10 + G)
    Hkv, d, bs = 2, 8, 4
    Hq = Hkv * G
    shapes = [(5, 0), (1, 9), (3, 6), (1, 0)]  # (new, seen): prefill, decode, chunk, 1 key
    qs, Ks, Vs = [], [], []
    for n, s in shapes:
        qs.append(rng.standard_normal((n, Hq, d)).astype(np.float32))
        Ks.append(rng.standard_normal((n + s, Hkv, d)).astype(np.float32))
        Vs.append(rng.standard_normal((n + s, Hkv, d)).astype(np.float32))
    got = _oracle_on_contiguous(qs, Ks, Vs, [s for _, s in shapes], bs, rng)
    want = np.concatenate([_bruteforce_attention(q, K, V, s, G)
                           for q, K, V, (_, s) in zip(qs, Ks, Vs, shapes)])
    assert np.max(np.abs(got - want)) < 1e-12


def test_attention_two_key_closed_form():
    # d = 4, two keys: q.k0 = 2, q.k1 = 0, scale 1/sqrt(4) = 1/2, so the weights are
    # e^1 / (e^1 + 1) and 1 / (e^1 + 1).
    q = np.array([[[1.0, 1.0, 0.0, 0.0]]], dtype=np.float32)
    K = np.array([[[1.0, 1.0, 0.0, 0.0]], [[0.0, 0.0, 1.0, -1.0]]], dtype=np.float32)
    V = np.array([[[1.0, 0.0, 2.0, 0.0]], [[0.0, 3.0, 0.0, -1.0]]], dtype=np.float32)
    got = _oracle_on_contiguous([q], [K], [V], [1], 2, np.random.default_rng(0))[0, 0]
    w0 = math.e / (math.e + 1.0)
    w1 = 1.0 / (math.e + 1.0)
    want = [w0, 3 * w1, 2 * w0, -w1]
    assert np.allclose(got, want, rtol=0, atol=1e-15)


def test_attention_single_key_returns_v_and_zero_query_returns_mean():
    rng = np.random.default_rng(20)
    Hkv, d = 2, 16
    q1 = rng.standard_normal((1, 4, d)).astype(np.float32)
    K1 = rng.standard_normal((1, Hkv, d)).astype(np.float32)
    V1 = rng.standard_normal((1, Hkv, d)).astype(np.float32)
    out = _oracle_on_contiguous([q1], [K1], [V1], [0], 16, rng)
    for h in range(4):
        assert np.array_equal(out[0, h], V1[0, h // 2].astype(np.float64))
    q0 = np.zeros((3, 4, d), dtype=np.float32)
    K = rng.standard_normal((10, Hkv, d)).astype(np.float32)
    V = rng.standard_normal((10, Hkv, d)).astype(np.float32)
    out = _oracle_on_contiguous([q0], [K], [V], [7], 4, rng)
    for t in range(3):
        for h in range(4):
            want = V[:8 + t, h // 2].astype(np.float64).mean(axis=0)
            assert np.allclose(out[t, h], want, rtol=0, atol=1e-14)


def test_attention_convex_hull_and_causality():
    rng = np.random.default_rng(21)
    Hkv, d = 1, 8
    q = (3 * rng.standard_normal((6, 2, d))).astype(np.float32)
    K = (3 * rng.standard_normal((20, Hkv, d))).astype(np.float32)
    V = rng.standard_normal((20, Hkv, d)).astype(np.float32)
    out = _oracle_on_contiguous([q], [K], [V], [14], 4, rng)
    for t in range(6):
        vis = V[:15 + t, 0].astype(np.float64)
        assert np.all(out[t] >= vis.min(axis=0) - 1e-12)
        assert np.all(out[t] <= vis.max(axis=0) + 1e-12)
    # keys after a query's position must not matter (bottom-right causal alignment)
    K2, V2 = K.copy(), V.copy()
    K2[17:] = 100.0
    V2[17:] = -100.0
    out2 = _oracle_on_contiguous([q], [K2], [V2], [14], 4, rng)
    assert np.array_equal(out[:3], out2[:3])  # positions 14, 15, 16
    assert not np.allclose(out[3:], out2[3:])


def test_attention_ragged_equals_alone_and_block_invariance():
    rng = np.random.default_rng(22)
    Hq, Hkv, d = 4, 2, 16
    shapes = [(7, 3), (1, 40), (12, 0), (1, 1)]
    qs = [rng.standard_normal((n, Hq, d)).astype(np.float32) for n, _ in shapes]
    Ks = [rng.standard_normal((n + s, Hkv, d)).astype(np.float32) for n, s in shapes]
    Vs = [rng.standard_normal((n + s, Hkv, d)).astype(np.float32) for n, s in shapes]
    seens = [s for _, s in shapes]
    together = _oracle_on_contiguous(qs, Ks, Vs, seens, 8, np.random.default_rng(1))
    alone = np.concatenate([_oracle_on_contiguous([q], [K], [V], [s], 8,
                                                  np.random.default_rng(2 + j))
                            for j, (q, K, V, s) in enumerate(zip(qs, Ks, Vs, seens))])
    assert np.array_equal(together, alone)
    other_perm = _oracle_on_contiguous(qs, Ks, Vs, seens, 8, np.random.default_rng(99))
    assert np.array_equal(together, other_perm)
    for bs in (1, 2, 16, 128):
        assert np.array_equal(together, _oracle_on_contiguous(qs, Ks, Vs, seens, bs,
                                                              np.random.default_rng(bs)))


def test_attention_gqa_group_mapping():
    """Query heads h = 0..G-1 read kv head 0 and h = G..2G-1 kv head 1 (reading of the
    grouped layout): the same batch with each kv head copied G times and G = 1 must
    give the same result."""
    rng = np.random.default_rng(23)
    G, Hkv, d = 3, 2, 8
    q = rng.standard_normal((4, G * Hkv, d)).astype(np.float32)
    K = rng.standard_normal((9, Hkv, d)).astype(np.float32)
    V = rng.standard_normal((9, Hkv, d)).astype(np.float32)
    grouped = _oracle_on_contiguous([q], [K], [V], [5], 4, rng)
    Kx, Vx = np.repeat(K, G, axis=1), np.repeat(V, G, axis=1)
    mha = _oracle_on_contiguous([q], [Kx], [Vx], [5], 4, rng)
    assert np.array_equal(grouped, mha)


def test_full_workload_oracle_end_to_end_tiny():
    """The tiny float32 batch through all three oracle steps: the outputs of each
    sequence equal brute-force dense attention over its contiguous rotated history."""
    wl = W.make_workload("tiny_f32")
    qkv, pool = _setup(wl)
    m = O.batch_metadata(wl.n_new, wl.seen, wl.block_lists, wl.block_size)
    q2, p2 = O.append_rotary(qkv, pool, m, 4, 4, 16, wl.rope_base, "f32")
    out = O.ragged_attention(q2, p2, m, 4, 4, 16, "f32")
    # seq 1 (decode, 50 seen): rebuild its 51 keys from the pool by walking its list
    i, L = 1, 51
    ids = wl.block_lists[i]
    K = np.stack([p2[ids[p // 16], 0, :, p % 16] for p in range(L)])
    V = np.stack([p2[ids[p // 16], 1, :, p % 16] for p in range(L)])
    q = q2[37:38, :4]
    want = _bruteforce_attention(q, K, V, 50, 1)
    assert np.max(np.abs(out[37:38] - want)) < 1e-12


def test_gathers_hand_fixture():
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "gather_examples.json")))
    e = fx["embedding"]
    got = O.embedding_gather(np.array(e["table"], dtype=np.float32), e["token_ids"])
    assert got.tolist() == e["expect"]
    lg = fx["logits"]
    cu = O.batch_metadata(lg["n_new"], [0] * len(lg["n_new"]),
                          [np.arange(8, dtype=np.int32)] * len(lg["n_new"]), 16)["cu_seqlens"]
    got = O.logits_gather(np.array(lg["rows"], dtype=np.float32), cu)
    assert got.tolist() == lg["expect"]


@pytest.mark.parametrize("seed", range(4))
def test_logits_gather_is_the_last_token_of_each_sequence(seed):
    """The last-token row found another way: scan token_to_seq for the final token that
    belongs to each sequence."""
    wl = W.random_workload(seed, max_new=30)
    m = O.batch_metadata(wl.n_new, wl.seen, wl.block_lists, wl.block_size)
    rows = np.arange(wl.T * 3, dtype=np.float32).reshape(wl.T, 3)
    got = O.logits_gather(rows, m["cu_seqlens"])
    last = {}
    for t, i in enumerate(m["token_to_seq"]):
        last[int(i)] = t
    assert np.array_equal(got, rows[[last[i] for i in range(wl.S)]])


def test_embedding_gather_bit_patterns_and_range():
    """Rows move bit for bit (bf16 patterns, NaN payloads included) and only ids in
    [0, vocab) read the table."""
    table = np.array([[0x7FC1, 0x0001], [0x8000, 0xFFFF]], dtype=np.uint16)
    got = O.embedding_gather(table, [1, 0, 2, -5, 1])
    assert got.tolist() == [[0x8000, 0xFFFF], [0x7FC1, 0x0001], [0, 0], [0, 0],
                            [0x8000, 0xFFFF]]
    assert got.dtype == np.uint16
