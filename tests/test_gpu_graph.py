"""The attention calls under HIP graph capture: one step (device metadata rebuild, then the
serial or the concurrent attention) captured once and replayed several times, with the
program's own eager work and synchronisations between the replays; every replay must give
the bytes of the eager call.  The concurrent call's fork and join events, its side stream
and its counter reset kernels are all captured (the library records no memset); the
full-budget and the eight-head-group batches take the mixed launch, the head-dim-64 batch
the two streams."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def _bytes(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("name,concurrent", [
    ("full8192_gqa4", True), ("full8192_gqa4", False), ("random_bf16_g8", True),
    ("random_bf16_d64", True), ("random_f32", True)])
def test_graph_replays_match_eager(name, concurrent):
    from ragged_blocked_kv_amd.runtime import Engine
    print(f"graph {name} concurrent={concurrent}", flush=True)
    if name == "random_bf16_g8":
        wl = W.random_workload(41, dtype="bf16", n_q_heads=16, n_kv_heads=2, head_dim=128,
                               block_size=64, n_seqs=30, max_new=200, max_seen=3000)
    elif name == "random_bf16_d64":
        wl = W.random_workload(45, dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=64,
                               block_size=64, n_seqs=24, max_new=200, max_seen=3000)
    elif name == "random_f32":
        wl = W.random_workload(42, dtype="f32", n_q_heads=4, n_kv_heads=2, head_dim=64,
                               block_size=16, n_seqs=8, max_new=40, max_seen=300)
    else:
        wl = W.make_workload(name)
    dev = torch.device("cuda:0")
    eng = Engine.for_workload(wl, device=dev)
    qkv = W.make_qkv(wl).to(dev)
    pool = W.make_pool_history(wl, device=dev)
    eng.finalize(wl.n_new, wl.seen, wl.block_lists)
    eng.append_rotary(qkv, pool, wl.rope_base)

    def attend(out):
        if concurrent:
            eng.attention_concurrent(qkv, pool, out)
        else:
            eng.attention(qkv, pool, out)

    shape = (wl.T, wl.n_q_heads, wl.head_dim)
    ref = torch.full(shape, float("nan"), dtype=qkv.dtype, device=dev)
    attend(ref)  # eager (also creates the engine's side stream and events)
    torch.cuda.synchronize()
    ref_b = _bytes(ref)

    out = torch.full(shape, float("nan"), dtype=qkv.dtype, device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        eng.rebuild()
        attend(out)
    torch.cuda.synchronize()

    scratch = torch.empty(shape, dtype=qkv.dtype, device=dev)
    for rep in range(4):
        out.fill_(float("nan"))          # eager work between replays
        eng.attention(qkv, pool, scratch)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bytes(out), ref_b), f"replay {rep}"
    assert np.array_equal(_bytes(scratch), ref_b)
