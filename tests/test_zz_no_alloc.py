"""ragged_blocked_attention_noalloc (split-K partials in the library's static scratch, no
allocation) against ragged_blocked_attention with a caller workspace, through the C ABI:
two calls in a row on one GPU, the second with a smaller batch, each byte-equal to the
workspace call's output (same kernels), and within tolerance of the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


def _bytes(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _batch(seed, dtype, Hq, Hkv, d, bs, seqs):
    wl = W.random_workload(seed, dtype=dtype, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                           block_size=bs, n_seqs=len(seqs))
    wl.n_new = np.array([a for a, _ in seqs], dtype=np.int32)
    wl.seen = np.array([b for _, b in seqs], dtype=np.int32)
    need = [W.blocks_needed(a + b, bs) for a, b in seqs]
    wl.num_blocks = sum(need) + 2
    perm = np.random.default_rng(seed + 1).permutation(wl.num_blocks).astype(np.int32)
    at = np.cumsum([0] + need)
    wl.block_lists = [perm[at[i]:at[i + 1]] for i in range(len(seqs))]
    return wl


def _check(wl):
    import ragged_blocked_kv_amd as R
    from ragged_blocked_kv_amd.runtime import Engine

    dev = torch.device("cuda:0")
    eng = Engine.for_workload(wl, device=dev)
    qkv_in = W.make_qkv(wl)
    pool_in = W.make_pool_history(wl, device="cpu")
    qkv, pool = qkv_in.to(dev), pool_in.to(dev)
    b = eng.finalize(wl.n_new, wl.seen, wl.block_lists)
    eng.append_rotary(qkv, pool, wl.rope_base)
    ref = eng.new_out().fill_(float("nan"))
    eng.attention(qkv, pool, ref)
    got = eng.new_out().fill_(float("nan"))
    st = R.ragged_blocked_attention_noalloc(eng.shape, b, qkv, pool, got,
                                            torch.cuda.current_stream(dev))
    assert st == R.OK, R.status_string(st)
    torch.cuda.synchronize()
    assert b.n_partials > 0  # the static scratch is in use
    assert np.array_equal(_bytes(got), _bytes(ref))
    md = O.batch_metadata(wl.n_new, wl.seen, wl.block_lists, wl.block_size)
    u = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16) \
        if t.dtype == torch.bfloat16 else t.cpu().numpy()
    q_ref, pool_ref = O.append_rotary(u(qkv_in), u(pool_in), md, wl.n_q_heads, wl.n_kv_heads,
                                      wl.block_size, wl.rope_base, wl.dtype)
    want = O.ragged_attention(q_ref, pool_ref, md, wl.n_q_heads, wl.n_kv_heads,
                              wl.block_size, wl.dtype)
    err = float(np.max(np.abs(O.storage_to_f64(u(got), wl.dtype) - want)))
    assert err <= TOL[wl.dtype], err
    return b.n_partials


def test_noalloc_matches_workspace_call_twice():
    print("noalloc: large batch, then a smaller one", flush=True)
    big = _batch(71, "bf16", 16, 4, 128, 64, [(1, 20000), (37, 500), (1, 3000), (1, 9000)])
    small = _batch(72, "bf16", 16, 4, 128, 64, [(1, 5000), (5, 100)])
    n1 = _check(big)
    n2 = _check(small)
    assert n2 < n1


def test_noalloc_float32():
    print("noalloc: float32", flush=True)
    _check(_batch(73, "f32", 4, 2, 64, 32, [(1, 7000), (9, 40), (1, 200)]))
