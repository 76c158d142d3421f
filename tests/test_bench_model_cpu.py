"""The benchmark's algorithmic work model (the numerator of every roofline figure)
against a brute-force count over tokens, heads and visible keys on small batches."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def brute_force(wl):
    e = wl.elem_bytes
    Hq, Hkv, d = wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    dec_b = pre_b = pre_f = app_b = 0
    for n, s in zip(wl.n_new.tolist(), wl.seen.tolist()):
        # K and V rows of every visible key of the sequence, read once per kv head
        kv = sum(e * d * 2 for _ in range(Hkv) for _ in range(s + n))
        qo = 0
        flops = 0
        for t in range(n):
            qo += 2 * Hq * d * e  # the token's Q rows in, its output rows out
            flops += sum(4 * d for _ in range(Hq) for _ in range(s + t + 1))  # QK and PV per key
            app_b += 2 * e * d * (Hq + 2 * Hkv)  # its qkv row read, rotated Q / K / V written
        if n == 1:
            dec_b += kv + qo
        else:
            pre_b += kv + qo
            pre_f += flops
    return {"decode_bytes": dec_b, "prefill_bytes": pre_b, "prefill_flops": pre_f,
            "attention_bytes": dec_b + pre_b, "append_bytes": app_b}


def test_algorithmic_work_matches_brute_force():
    for seed in range(6):
        wl = W.random_workload(seed, dtype="bf16" if seed % 2 else "f32", n_q_heads=4 * (1 + seed % 3),
                               n_kv_heads=2, head_dim=64 if seed % 2 else 128, max_new=30,
                               max_seen=70)
        got = bench.algorithmic_work(wl)
        want = brute_force(wl)
        for k, v in want.items():
            assert got[k] == v, (seed, k, got[k], v)


def test_algorithmic_work_full_budget_batch_figures():
    """The full-budget batch's totals that the roofline lines quote: 4.522 GB of attention
    bytes (4.114 GB of them the decodes') and 520.5 GFLOP of causal prefill pairs."""
    got = bench.algorithmic_work(W.make_workload("full8192_gqa4"))
    assert round(got["attention_bytes"] / 1e9, 3) == 4.522
    assert round(got["decode_bytes"] / 1e9, 3) == 4.114
    assert round(got["prefill_flops"] / 1e9, 1) == 520.5
