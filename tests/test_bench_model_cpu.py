"""The benchmark's arithmetic: its algorithmic work model (the numerator of every roofline
figure) against a brute-force count over tokens, heads and visible keys on small batches,
and the reduction of HBM counter runs to bytes per launch on synthetic counter files."""
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


def _write_counter_csv(path, rows):
    import csv

    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, name, counter, value in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_traffic_reduction_scales_by_the_copy_calibration(tmp_path):
    """FETCH_SIZE / WRITE_SIZE (KiB, summed over a dispatch's rows) become bytes per launch
    through the factor that makes a copy of known size read and write exactly its size;
    the copy is the largest non-library dispatch, the kernel's launches are averaged."""
    cal = 1 << 30
    copy = "void at::native::copy_kernel(...)"
    _write_counter_csv(tmp_path / "cf.csv", [(1, copy, "FETCH_SIZE", 12.0),
                                            (2, copy, "FETCH_SIZE", 262144.0),  # two rows of one
                                            (2, copy, "FETCH_SIZE", 262144.0)])  # dispatch: 512 MiB
    _write_counter_csv(tmp_path / "cw.csv", [(2, copy, "WRITE_SIZE", 1048576.0)])
    kern = "void rbkv::(anonymous namespace)::decode_mfma_kernel<3>(...)"
    _write_counter_csv(tmp_path / "f.csv", [(7, kern, "FETCH_SIZE", 600.0), (7, kern, "FETCH_SIZE", 400.0),
                                           (9, kern, "FETCH_SIZE", 1200.0),
                                           (8, "void rbkv::combine_kernel<>(...)", "FETCH_SIZE", 5.0)])
    _write_counter_csv(tmp_path / "w.csv", [(7, kern, "WRITE_SIZE", 10.0), (9, kern, "WRITE_SIZE", 30.0),
                                           (8, "void rbkv::combine_kernel<>(...)", "WRITE_SIZE", 1.0)])
    out = tmp_path / "traffic.json"
    bench.traffic_from_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), cal,
                                "toy", str(out))
    import json

    rec = json.load(open(out))
    d = rec["attn_decode.hip:toy"]
    assert d["fetch_scale"] == 2.0 and d["write_scale"] == 1.0
    assert d["dispatches"] == 2
    assert d["fetch_bytes_per_launch"] == 1100.0 * 1024 * 2.0   # mean of 1000 and 1200 KiB
    assert d["write_bytes_per_launch"] == 20.0 * 1024           # mean of 10 and 30 KiB
    assert d["bytes_per_launch"] == d["fetch_bytes_per_launch"] + d["write_bytes_per_launch"]
    assert rec["attn_combine.hip:toy"]["bytes_per_launch"] == 5.0 * 1024 * 2.0 + 1.0 * 1024
    assert "attn_prefill.hip:toy" not in rec  # no dispatch of that group in the run


def test_mfma_reduction_per_launch_figures(tmp_path):
    """Matrix-core counters of the prefill kernel become per-launch flops (512 per MOPS
    unit), busy cycles, the busy fraction over the mean XCD's active cycles x 1024 SIMDs,
    and rocprofv3's MfmaUtil averaged over the dispatches of its own run."""
    kern = "void rbkv::(anonymous namespace)::prefill_attn_kernel<128>(...)"
    other = "void rbkv::combine_kernel<>(...)"
    rows = []
    for d, busy, mops, gui in ((3, 600.0, 1000.0, 8000.0), (5, 500.0, 1000.0, 8000.0)):
        rows += [(d, kern, "SQ_VALU_MFMA_BUSY_CYCLES", busy / 2), (d, kern, "SQ_VALU_MFMA_BUSY_CYCLES", busy / 2),
                 (d, kern, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops), (d, kern, "GRBM_GUI_ACTIVE", gui),
                 (d, kern, "SQ_BUSY_CU_CYCLES", 77.0)]
    rows += [(4, other, "SQ_VALU_MFMA_BUSY_CYCLES", 9999.0), (4, other, "GRBM_GUI_ACTIVE", 1.0)]
    _write_counter_csv(tmp_path / "m.csv", rows)
    _write_counter_csv(tmp_path / "u.csv", [(3, kern, "MfmaUtil", 60.0), (5, kern, "MfmaUtil", 62.0)])
    out = tmp_path / "mfma.json"
    bench.mfma_from_counters(str(tmp_path / "m.csv"), str(tmp_path / "u.csv"), "toy", str(out))
    import json

    r = json.load(open(out))["attn_prefill.hip:toy"]
    assert r["dispatches"] == 2
    assert r["mfma_flops_per_launch"] == 1000.0 * 512
    assert r["mfma_busy_cycles_per_launch"] == 550.0
    assert r["gui_active_cycles_per_xcd"] == 1000.0
    assert r["mfma_busy_frac_per_dispatch"] == [round(600.0 / (1000.0 * 1024), 4), round(500.0 / (1000.0 * 1024), 4)]
    assert r["MfmaUtil_percent"] == 61.0


def test_more_than_one_gpu_is_refused_with_a_message():
    """The path runs on one GPU: bench.py --gpus N with N > 1 exits with status 2 and says
    so on stderr, before it imports torch or touches a device."""
    import subprocess
    for n in (2, 8):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                           capture_output=True, text=True, timeout=120, cwd=ROOT)
        assert r.returncode == 2, (n, r.returncode, r.stderr[-500:])
        assert f"--gpus {n} is not supported" in r.stderr
        assert r.stdout == ""
