"""ragged_blocked_attention_concurrent (decodes on a side stream beside the prefill
chunks, joined before the combine) gives exactly the bytes of the serial call, on mixed
batches of both dtypes and on the full-budget and SplitFuse batches, repeatedly."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def _run(wl, concurrent, reps=3):
    from ragged_blocked_kv_amd.runtime import Engine
    dev = torch.device("cuda:0")
    eng = Engine.for_workload(wl, device=dev)
    qkv = W.make_qkv(wl).to(dev)
    pool = W.make_pool_history(wl, device=dev)
    eng.finalize(wl.n_new, wl.seen, wl.block_lists)
    eng.append_rotary(qkv, pool, wl.rope_base)
    outs = []
    for _ in range(reps):
        out = torch.full((wl.T, wl.n_q_heads, wl.head_dim), float("nan"), dtype=qkv.dtype,
                         device=dev)
        if concurrent:
            eng.attention_concurrent(qkv, pool, out)
        else:
            eng.attention(qkv, pool, out)
        torch.cuda.synchronize()
        outs.append(out.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32)
                    .cpu().numpy())
    return outs


@pytest.mark.parametrize("name", ["random_bf16", "random_f32", "splitfuse768_gqa4",
                                  "full8192_gqa4"])
def test_concurrent_equals_serial(name):
    print(f"concurrent {name}", flush=True)
    if name == "random_bf16":
        wl = W.random_workload(31, dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=128,
                               block_size=32, n_seqs=8, max_new=90, max_seen=400)
    elif name == "random_f32":
        wl = W.random_workload(32, dtype="f32", n_q_heads=4, n_kv_heads=2, head_dim=64,
                               block_size=16, n_seqs=6, max_new=40, max_seen=200)
    else:
        wl = W.make_workload(name)
    assert (wl.n_new > 1).any() and (wl.n_new == 1).any()
    serial = _run(wl, False, reps=1)[0]
    for k, got in enumerate(_run(wl, True)):
        assert np.array_equal(got, serial), k
