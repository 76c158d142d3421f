"""Throughput of one pass of the ragged-attention hot path on one MI355X.

A step is one pass over one batch with every input already resident in HBM: the device
metadata build (``ragged_batch_rebuild``), the rotary append
(``blocked_kv_append_rotary``) and the attention.  The timed steps run the attention as
``ragged_blocked_attention_concurrent``: for bf16 batches at head dim 128 with groups of
2-16 heads, one launch of persistent workgroups that take prefill tiles and decode
items from the same chip (the mixed launch, then the split-K combine); for other shapes
the chunks and the decodes on two streams.  A second pass times the mixed launch alone
(``RBKV_PHASE_ATTEND``) with HIP events on its stream (the roofline of the step's
dominant kernel), and a serial pass issues the prefill, decode and combine phases as
separate launches one after another, so that each kernel is timed on its own (their
rooflines and the phase breakdown).  The batch is the full-budget mixed batch: 8192 new tokens over
256 sequences (16 prefill chunks of 256..512 tokens and 240 decodes, seen ~ U[0, 8192]),
GQA 32 query / 8 kv heads, head dim 128, 64-token blocks, bf16.  The host half of
``ragged_batch_finalize`` (validation, packing, the small host-to-device upload) runs once
before the timed region and is reported separately.

Prints one JSON line.  ``--gpus N`` with N > 1 is refused: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix, TFLOP/s
DEFAULT_WORKLOAD = "full8192_gqa4"
PHASES = ("rebuild", "append", "prefill", "decode", "combine")


def algorithmic_work(wl):
    """Bytes each kernel must move and flops the prefill must do (no padding, no
    partials, no metadata)."""
    e = wl.elem_bytes
    Hq, Hkv, d = wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    n = wl.n_new.astype(np.int64)
    s = wl.seen.astype(np.int64)
    L = n + s
    dec = n == 1
    chunk = ~dec
    return {
        "decode_bytes": float(e * (2 * Hkv * d * L[dec].sum() + 2 * Hq * d * dec.sum())),
        "prefill_bytes": float(e * (2 * Hkv * d * L[chunk].sum() + 2 * Hq * d * n[chunk].sum())),
        "prefill_flops": float(4 * d * Hq * (n[chunk] * s[chunk] +
                                             n[chunk] * (n[chunk] + 1) // 2).sum()),
        "attention_bytes": float(e * (2 * Hkv * d * L.sum() + 2 * Hq * d * n.sum())),
        "append_bytes": float(2 * e * d * n.sum() * (Hq + 2 * Hkv)),
    }


def source_tokens_digest(text):
    """Digest of C++/HIP source text with comments removed and whitespace collapsed, so
    that edits to comments or layout alone keep a kernel's measured records valid."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def kernel_source_digest(names):
    """Digest of the sources a kernel group is built from (one name or a tuple)."""
    if isinstance(names, str):
        names = (names,)
    return source_tokens_digest("".join(
        open(os.path.join(ROOT, "ragged_blocked_kv_amd", "csrc", n)).read() for n in names))


def measured_traffic(label, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on
    the current source of that kernel group (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(f"{label}:{workload}")
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_sha") != kernel_source_digest(KERNEL_GROUPS[label][0]):
        return None
    return rec.get("bytes_per_launch")  # bytes per launch (fetch + write), scaled


# Library kernels in groups for the HBM-traffic reduction: label -> (source file, kernel
# name fragments).  A label's record is valid while its source file hashes the same.
KERNEL_GROUPS = {
    "attn_prefill.hip": ("attn_prefill.hip", ("prefill_attn_kernel",)),
    "attn_prefill.hip/mixed": (("attn_prefill.hip", "decode_mfma.h"), ("mixed_attn_kernel",)),
    "attn_decode.hip": (("attn_decode.hip", "decode_mfma.h"),
                        ("decode_attn_kernel", "decode_group_kernel", "decode_lean_kernel",
                         "decode_lean2_kernel", "decode_reg_kernel", "decode_mfma_kernel")),
    "append_rotary.hip": ("append_rotary.hip", ("append_rotary_kernel",)),
    "attn_combine.hip": ("attn_combine.hip", ("combine_kernel",)),
    "meta_build.hip": ("meta_build.hip", ("meta_build_kernel",)),
    "gather.hip/embedding": ("gather.hip", ("embedding_gather_kernel",)),
    "gather.hip/logits": ("gather.hip", ("logits_gather_kernel",)),
    "kv_offload.hip": ("kv_offload.hip", ("kv_block_copy_kernel",)),
}


def decode_kernel_name(wl):
    """The decode kernel a workload runs: bf16 over 64-key blocks at head dim 128 runs the
    matrix-core kernel for groups of 2-16 heads and the register-only kernel for single
    heads; at head dim 64 a lean workgroup with one K/V tile (one wave per head for groups
    of up to 4 heads, two heads per wave for 5-8); other bf16 groups of 5+ heads the
    grouped kernel (two LDS tile stages); float32, and bf16 groups of up to 4 over smaller blocks, one
    wave per item."""
    g = wl.n_q_heads // wl.n_kv_heads
    if wl.dtype == "bf16" and wl.block_size >= 64 and wl.head_dim == 128:
        return "decode_reg_kernel" if g == 1 else "decode_mfma_kernel"
    if wl.dtype == "bf16" and g <= 8 and wl.block_size >= 64:
        return "decode_lean_kernel" if g <= 4 else "decode_lean2_kernel"
    if wl.dtype == "bf16" and g > 4:
        return "decode_group_kernel"
    return "decode_attn_kernel"


def mixed_launch(wl):
    """Whether the library runs this batch's attention as one mixed launch (prefill tiles
    and decode items from one set of persistent workgroups)."""
    g = wl.n_q_heads // wl.n_kv_heads
    return (wl.dtype == "bf16" and wl.head_dim == 128 and wl.block_size >= 64 and 2 <= g <= 16
            and bool((wl.n_new > 1).any()) and bool((wl.n_new == 1).any()))


def copy_calibration(nbytes, reps):
    """A plain device-to-device copy of a known size, for scaling the HBM counters."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}))


def _counter_per_dispatch(csv_path, counter, name_filter):
    import csv as _csv
    import collections

    per = collections.defaultdict(float)
    for row in _csv.DictReader(open(csv_path)):
        if row["Counter_Name"] == counter and name_filter(row["Kernel_Name"]):
            per[row["Dispatch_Id"]] += float(row["Counter_Value"])
    return per


def traffic_from_counters(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, cal_bytes,
                          workload, out_path):
    """Reduce rocprofv3 FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch) to HBM bytes per
    launch of each library kernel, scaled by what the same counters read for a copy of
    cal_bytes bytes (which reads and writes exactly cal_bytes)."""
    is_copy = lambda n: "rbkv" not in n
    cf = _counter_per_dispatch(cal_fetch_csv, "FETCH_SIZE", is_copy)
    cw = _counter_per_dispatch(cal_write_csv, "WRITE_SIZE", is_copy)
    big = lambda d: max(d.values())  # the calibration copy is the largest dispatch
    f_scale = cal_bytes / (big(cf) * 1024.0)
    w_scale = cal_bytes / (big(cw) * 1024.0)
    rec = json.load(open(out_path)) if os.path.exists(out_path) else {}
    for label, (kfile, knames) in KERNEL_GROUPS.items():
        sel = lambda n, ks=knames: any(k in n for k in ks)
        fv = list(_counter_per_dispatch(fetch_csv, "FETCH_SIZE", sel).values())
        wv = list(_counter_per_dispatch(write_csv, "WRITE_SIZE", sel).values())
        if not fv or not wv:
            continue
        fb = float(np.mean(fv)) * 1024.0 * f_scale
        wb = float(np.mean(wv)) * 1024.0 * w_scale
        rec[f"{label}:{workload}"] = {
            "source_sha": kernel_source_digest(kfile),
            "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
            "bytes_per_launch": fb + wb, "dispatches": len(fv),
            "fetch_scale": f_scale, "write_scale": w_scale,
        }
    json.dump(rec, open(out_path, "w"), indent=1, sort_keys=True)
    print(json.dumps(rec, indent=1))


def host_cpu():
    """The host's CPU model and core counts (what the CPU baseline ran on)."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": affinity}


def _mapped(ref):
    """An array, or (path, offset, shape, dtype) of one held in a shared-memory file."""
    if isinstance(ref, np.ndarray):
        return ref
    path, off, shape, dt = ref
    return np.memmap(path, dtype=np.dtype(dt), mode="r", offset=off, shape=tuple(shape))


def _oracle_sequence(task):
    """One sequence through the oracle's append and attention on a sub-pool of its own
    blocks; returns (new tokens, seconds).  The unit of work of both CPU timings."""
    import oracle as O

    n, seen, qrows, sub_pool, Hq, Hkv, bs, base, dtype = task
    qrows, sub_pool = _mapped(qrows), _mapped(sub_pool)
    t0 = time.perf_counter()
    m1 = O.batch_metadata([n], [seen], [np.arange(sub_pool.shape[0], dtype=np.int32)], bs)
    q, p = O.append_rotary(qrows, sub_pool, m1, Hq, Hkv, bs, base, dtype)
    O.ragged_attention(q, p, m1, Hq, Hkv, bs, dtype)
    return n, time.perf_counter() - t0


_BLAS_LIMIT = None


def _single_blas_thread():
    """Worker initializer: one BLAS thread per process."""
    global _BLAS_LIMIT
    from threadpoolctl import threadpool_limits
    _BLAS_LIMIT = threadpool_limits(1)


SIMDS = 1024  # MI355X: 256 CUs x 4 SIMDs
XCDS = 8


def mfma_from_counters(csv_path, util_csv, workload, out_path):
    """Reduce a rocprofv3 --pmc run of SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16,
    SQ_BUSY_CU_CYCLES and GRBM_GUI_ACTIVE (values summed over every instance: SIMDs, shader
    engines, XCDs) on the prefill kernel, plus a run of rocprofv3's derived MfmaUtil
    metric, into per-launch matrix-core figures:

    * mfma_flops_per_launch = 512 x MOPS_BF16 (the counter counts flops / 512);
    * MfmaUtil_percent: rocprofv3's derived metric, MFMA busy cycles summed over the SIMDs /
      (the largest XCD's GUI-active cycles x 1024 SIMDs), from its own run;
    * mfma_busy_frac: the same ratio over the mean XCD's GUI-active cycles (GRBM_GUI_ACTIVE
      is summed over the 8 XCDs in this run, so the mean is the sum / 8)."""
    sel = lambda n: "prefill_attn_kernel" in n
    busy = _counter_per_dispatch(csv_path, "SQ_VALU_MFMA_BUSY_CYCLES", sel)
    mops = _counter_per_dispatch(csv_path, "SQ_INSTS_VALU_MFMA_MOPS_BF16", sel)
    gui = _counter_per_dispatch(csv_path, "GRBM_GUI_ACTIVE", sel)
    cu = _counter_per_dispatch(csv_path, "SQ_BUSY_CU_CYCLES", sel)
    util = _counter_per_dispatch(util_csv, "MfmaUtil", sel) if util_csv else {}
    ids = sorted(busy)
    fr = [busy[i] / (gui[i] / XCDS * SIMDS) for i in ids]
    rec = json.load(open(out_path)) if os.path.exists(out_path) else {}
    rec[f"attn_prefill.hip:{workload}"] = {
        "source_sha": kernel_source_digest("attn_prefill.hip"),
        "dispatches": len(ids),
        "mfma_flops_per_launch": float(np.mean([mops[i] for i in ids])) * 512.0,
        "mfma_busy_cycles_per_launch": float(np.mean([busy[i] for i in ids])),
        "gui_active_cycles_per_xcd": float(np.mean([gui[i] for i in ids])) / XCDS,
        "busy_cu_quad_cycles_per_launch": float(np.mean([cu[i] for i in ids])) if cu else None,
        "mfma_busy_frac": float(np.mean(fr)),
        "mfma_busy_frac_per_dispatch": [round(v, 4) for v in fr],
        "MfmaUtil_percent": float(np.mean(list(util.values()))) if util else None,
    }
    json.dump(rec, open(out_path, "w"), indent=1, sort_keys=True)
    print(json.dumps(rec, indent=1))


def cpu_baseline(wl, qkv_cpu, hist_fn, budget_s, max_workers=16):
    """The oracle as it stands, on a bounded sample of the same batch (sequences in a
    seeded order, chunks and decodes interleaved; each through the oracle's append and
    attention on a sub-pool holding its own blocks; input staging not timed), two ways:

    * one core: this process with its BLAS held to one thread, sequences one after
      another until ``budget_s`` of oracle time is spent;
    * one process per core: ``min(cpu count, affinity, max_workers)`` worker processes
      (spawned, so none inherits this process's GPU state), each with one BLAS thread,
      fed sequences in the same order until ``budget_s`` of wall time has passed, then
      drained; rate = tokens done / wall time from the first submission to the last
      result (worker start-up and the staging of inputs into a shared-memory file that
      the workers map excluded).

    ``value`` is the process-per-core rate, ``cores`` its worker count."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    rng = np.random.default_rng(2024)
    chunks = [int(i) for i in rng.permutation(np.nonzero(wl.n_new > 1)[0])]
    decs = [int(i) for i in rng.permutation(np.nonzero(wl.n_new == 1)[0])]
    order = []
    while chunks or decs:
        if chunks:
            order.append(chunks.pop())
        order.extend(decs[:15])
        decs = decs[15:]
    cu = np.concatenate([[0], np.cumsum(wl.n_new)])

    def task(i):
        nb = -(-(int(wl.seen[i]) + int(wl.n_new[i])) // wl.block_size)
        return (int(wl.n_new[i]), int(wl.seen[i]), qkv_cpu[cu[i]:cu[i + 1]], hist_fn(i, nb),
                wl.n_q_heads, wl.n_kv_heads, wl.block_size, wl.rope_base, wl.dtype)

    def describe(seqs, tok, secs, what):
        nch = sum(int(wl.n_new[i] > 1) for i in seqs)
        return (f"{len(seqs)} of {wl.S} sequences of {wl.name} ({nch} prefill chunks, "
                f"{len(seqs) - nch} decodes, {tok} of {wl.T} tokens): float64 oracle append + "
                f"attention, {secs:.1f} s {what}")

    # one core
    done, tok1, spent = [], 0, 0.0
    with threadpool_limits(1):
        for i in order:
            n, dt = _oracle_sequence(task(i))
            done.append(i)
            tok1 += n
            spent += dt
            if spent >= budget_s:
                break
    single = {"value": tok1 / spent, "unit": "tokens/s", "cores": 1, "blas_threads": 1,
              "sample": describe(done, tok1, spent, "of oracle time on one core")}

    # one process per core; the inputs go to the workers through one shared-memory file
    # written before the clock starts (input staging, not timed)
    import tempfile

    host = host_cpu()
    workers = max(1, min(host["os_cpu_count"] or 1, host["affinity_cpus"] or 1, max_workers))
    shm = "/dev/shm" if os.path.isdir("/dev/shm") else None
    with tempfile.NamedTemporaryFile(dir=shm, prefix="rbkv_oracle_") as f:
        refs, off = {}, 0
        for i in order:
            t = task(i)
            pair = []
            for a in (t[2], t[3]):
                a = np.ascontiguousarray(a)
                f.write(a.tobytes())
                pair.append((f.name, off, a.shape, a.dtype.str))
                off += a.nbytes
            refs[i] = t[:2] + tuple(pair) + t[4:]
        f.flush()
        ctx = mp.get_context("spawn")
        with ctx.Pool(workers, initializer=_single_blas_thread) as pool:
            pool.map(int, range(workers))  # every worker started before the clock
            pending, done_m, tokm = [], [], 0
            t0 = time.perf_counter()
            for i in order:
                while len(pending) >= 2 * workers:
                    j, r = pending.pop(0)
                    tokm += r.get()[0]
                    done_m.append(j)
                pending.append((i, pool.apply_async(_oracle_sequence, (refs[i],))))
                if time.perf_counter() - t0 >= budget_s:
                    break
            for j, r in pending:
                tokm += r.get()[0]
                done_m.append(j)
            wall = time.perf_counter() - t0
    return {
        "value": tokm / wall,
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "blas_threads_per_process": 1,
        "sample": describe(done_m, tokm, wall, f"of wall time over {workers} worker processes "
                                              f"(one BLAS thread each)"),
        "single_core": single,
        "host": host,
    }


def ledger_cost(wl, eng, stream, reps=20):
    """Host time of the native ledger around one pass of the bench batch: the batch's
    sequences are first given their cached tokens (in groups, outside the timing), then
    each rep runs can_schedule, put (blocks for the new tokens), the ledger's finalize
    (host packing plus the upload, enqueued) and post_forward, as a serving loop would
    before and after every forward pass.  Median microseconds per call."""
    import torch

    from ragged_blocked_kv_amd.state import SCHED_OK, StateManager

    st = StateManager(num_blocks=wl.num_blocks, block_size=wl.block_size,
                      max_tracked_seqs=wl.max_seqs, max_seqs=wl.max_seqs,
                      max_tokens=1 << 20, max_context=1 << 30)
    uids = np.arange(wl.S, dtype=np.int64) * 1_000_003 + 17
    for g in range(0, wl.S, 16):
        has = [i for i in range(g, min(wl.S, g + 16)) if wl.seen[i] > 0]
        if has:
            assert st.put(uids[has], wl.seen[has]) == SCHED_OK
            st.post_forward()
    n_new = wl.n_new.astype(np.int32)
    t = {k: [] for k in ("can_schedule", "put", "finalize", "post_forward")}
    done = 0
    for _ in range(reps):  # the sequences grow each rep; stop when the pool is full
        t0 = time.perf_counter()
        ok = st.can_schedule(uids, n_new) == SCHED_OK
        t1 = time.perf_counter()
        if not ok:
            break
        done += 1
        assert st.put(uids, n_new) == SCHED_OK
        t2 = time.perf_counter()
        eng.finalize_state(st, stream=stream)
        t3 = time.perf_counter()
        st.post_forward()
        t4 = time.perf_counter()
        for k, a, b in (("can_schedule", t0, t1), ("put", t1, t2), ("finalize", t2, t3),
                        ("post_forward", t3, t4)):
            t[k].append((b - a) * 1e6)
        torch.cuda.synchronize()
    med = {k: round(float(np.median(v)), 1) for k, v in t.items()}
    return {"host_us_per_pass": med, "total_us": round(sum(med.values()), 1),
            "sequences": wl.S, "new_tokens": wl.T, "reps": done}


def serving_leg(wl, eng, qkv, pool, out, stream, passes=12, warm=3):
    """A Dynamic SplitFuse serving loop on the bench's shapes, end to end per pass:
    compose the batch on the native ledger (the decodes of the batch's single-token
    sequences first, then a seeded queue of prompts of 256..4096 tokens cut to fill the
    8192-token budget), put, finalize from the ledger, rotary append, attention (one
    ragged_blocked_attention_concurrent call),
    synchronize (a serving loop needs the pass's output before composing the next one)
    and post_forward.  Finished prompts are flushed; decodes run on.  Times are medians
    over the timed passes."""
    import torch

    from ragged_blocked_kv_amd.state import SCHED_OK, StateManager

    # The ledger's own token cap only has to admit the history fill below; each pass's
    # budget is the batch capacity, given to compose.
    st = StateManager(num_blocks=wl.num_blocks, block_size=wl.block_size,
                      max_tracked_seqs=4 * wl.max_seqs, max_seqs=wl.max_seqs,
                      max_tokens=1 << 20, max_context=1 << 30)
    dec = [i for i in range(wl.S) if wl.n_new[i] == 1]
    dec_uids = [1_000_000 + i for i in dec]
    for g in range(0, len(dec), 16):  # cached history of the decoding sequences
        grp = [(u, int(wl.seen[i])) for u, i in zip(dec_uids[g:g + 16], dec[g:g + 16])
               if wl.seen[i] > 0]
        if grp:
            assert st.put([u for u, _ in grp], [n for _, n in grp]) == SCHED_OK
            st.post_forward()
    rng = np.random.default_rng(99)
    prompts = {}  # uid -> tokens still to feed, in arrival order
    next_uid = 2_000_000
    host, gpu, wall, tok = [], [], [], []
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for k in range(warm + passes):
        while sum(prompts.values()) < 2 * wl.max_tokens:  # keep the queue full
            prompts[next_uid] = int(rng.integers(256, 4096, endpoint=True))
            next_uid += 1
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        queue = dec_uids + list(prompts)
        pending = [1] * len(dec_uids) + list(prompts.values())
        uids, n_new = st.compose(queue, pending, wl.max_tokens)
        assert st.put(uids, n_new) == SCHED_OK
        b = eng.finalize_state(st, stream=stream)
        t1 = time.perf_counter()
        ev0.record(stream)
        eng.append_rotary(qkv, pool, wl.rope_base, stream=stream, batch=b)
        eng.attention_concurrent(qkv, pool, out, stream=stream, batch=b)
        ev1.record(stream)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        st.post_forward()
        for u, n in zip(uids.tolist(), n_new.tolist()):
            if u in prompts:
                prompts[u] -= n
                if prompts[u] == 0:
                    del prompts[u]
                    st.flush(u)
        t3 = time.perf_counter()
        if k >= warm:
            host.append((t1 - t0 + t3 - t2) * 1e3)
            gpu.append(ev0.elapsed_time(ev1))
            wall.append((t3 - t0) * 1e3)
            tok.append(int(n_new.sum()))
    return {
        "tokens_per_s": float(sum(tok) / (sum(wall) * 1e-3)),
        "ms_per_pass": round(float(np.median(wall)), 3),
        "host_ms_per_pass": round(float(np.median(host)), 3),
        "gpu_ms_per_pass": round(float(np.median(gpu)), 3),
        "tokens_per_pass": int(np.median(tok)),
        "passes": passes,
        "batch": f"{len(dec_uids)} decodes + prompts of 256..4096 tokens cut to fill "
                 f"{wl.max_tokens} tokens",
    }


def gathers_leg(wl, eng, stream, reps=20, warm=3):
    """The two row gathers around the layer stack on the bench batch, at Llama-2-7B widths
    (the model the pages' install example loads): embedding rows (hidden 4096) of the
    8192 packed tokens from a 32000-row table, and the last-token rows of the 256
    sequences from vocabulary-wide (32000) logits of every token.  Average microseconds
    per launch from HIP events on the stream; algorithmic bytes are the rows read and
    written plus the index words."""
    import torch

    dev = torch.device("cuda:0")
    vocab, hidden = 32000, 4096
    g = torch.Generator(device=dev).manual_seed(7)
    table = torch.randn((vocab, hidden), generator=g, device=dev).to(torch.bfloat16)
    ids = torch.randint(0, vocab, (wl.T,), generator=g, device=dev, dtype=torch.int32)
    emb = torch.empty((wl.T, hidden), dtype=torch.bfloat16, device=dev)
    logits = torch.randn((wl.T, vocab), generator=g, device=dev).to(torch.bfloat16)
    last = torch.empty((wl.S, vocab), dtype=torch.bfloat16, device=dev)
    res = {}
    for name, fn, nbytes in (
            ("embedding", lambda: eng.embedding_gather(ids, table, emb, stream=stream),
             2 * wl.T * hidden * 2 + 4 * wl.T),
            ("logits", lambda: eng.logits_gather(logits, last, stream=stream),
             2 * wl.S * vocab * 2 + 4 * (wl.S + 1))):
        for _ in range(warm):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"kernel": f"{name}_gather_kernel", "us": round(us, 2), "bytes": nbytes,
                     "GBs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"gather.hip/{name}", wl.name)}
    # Context: what a plain 1 GiB device copy (read + write) reaches on this part.
    big = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    big2 = torch.empty_like(big)
    big2.copy_(big)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        big2.copy_(big)
    e1.record(stream)
    torch.cuda.synchronize()
    res["copy_1GiB_GBs"] = round(2 * (1 << 30) * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    res["widths"] = f"hidden {hidden}, vocab {vocab}, bf16"
    return res


PCIE_PEAK_GBS = 64.0  # PCIe 5.0 x16 per direction, the MI355X host link


def kv_offload_leg(wl, eng, pool, stream, n=1024, reps=5, warm=2):
    """KV block offload and restore of n scattered pool blocks (seeded choice) through a
    page-locked host buffer, against plain contiguous copies of the same byte count
    between device memory and page-locked host memory (the host link's copy rate).
    Restore writes into other blocks than those offloaded; the pool's contents are not
    needed afterwards."""
    import torch

    import ragged_blocked_kv_amd as R

    dev = torch.device("cuda:0")
    n = min(n, wl.num_blocks // 2)
    perm = np.random.default_rng(17).permutation(wl.num_blocks).astype(np.int32)
    src_ids, dst_ids = perm[:n], perm[n:2 * n]
    st, nbytes = R.rbkv_kv_host_bytes(eng.shape, n)
    R.check(st, "rbkv_kv_host_bytes")
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    payload = n * (wl.pool_bytes() // wl.num_blocks)
    dev_buf = torch.empty(payload, dtype=torch.uint8, device=dev)
    host_buf = torch.empty(payload, dtype=torch.uint8, pin_memory=True)

    def timed(fn):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def offload():
        R.check(R.blocked_kv_offload(eng.shape, pool, src_ids, host, nbytes, stream),
                "blocked_kv_offload")

    def restore():
        R.check(R.blocked_kv_restore(eng.shape, pool, dst_ids, host, nbytes, stream),
                "blocked_kv_restore")

    t_off, t_res = timed(offload), timed(restore)
    t_d2h = timed(lambda: host_buf.copy_(dev_buf, non_blocking=True))
    t_h2d = timed(lambda: dev_buf.copy_(host_buf, non_blocking=True))
    gb = lambda us: payload / (us * 1e-6) / 1e9
    return {
        "blocks": n, "bytes": payload,
        "offload": {"us": round(t_off, 1), "GBs": round(gb(t_off), 1),
                    "frac_link_copy": round(t_d2h / t_off, 3),
                    "frac_pcie_peak": round(gb(t_off) / PCIE_PEAK_GBS, 3)},
        "restore": {"us": round(t_res, 1), "GBs": round(gb(t_res), 1),
                    "frac_link_copy": round(t_h2d / t_res, 3),
                    "frac_pcie_peak": round(gb(t_res) / PCIE_PEAK_GBS, 3)},
        "link_copy_GBs": {"d2h": round(gb(t_d2h), 1), "h2d": round(gb(t_h2d), 1)},
    }


# Every measured configuration, in the order of the table in workloads: the tiny float32
# batch, MHA decode, SplitFuse 768, the full-budget batch, its prefill chunks alone and
# long-context decode.
CONFIG_WORKLOADS = ("tiny_f32", "decode_mha32", "splitfuse768_gqa4", "full8192_gqa4",
                    "full8192_prefill_gqa4", "long_decode_gqa8")


def measured_mfma(label, workload):
    """Matrix-core counters per launch from committed rocprofv3 runs (profiles/mfma.json),
    if they were taken on the current source of that kernel (else None)."""
    p = os.path.join(ROOT, "profiles", "mfma.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(f"{label}:{workload}")
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_sha") != kernel_source_digest(KERNEL_GROUPS[label][0]):
        return None
    return {k: rec[k] for k in ("MfmaUtil_percent", "mfma_busy_frac", "mfma_flops_per_launch",
                                "dispatches") if k in rec}


def time_steps(wl, eng, qkv, pool, out, stream, steps, warmup, one_call=True):
    """Serial steps (metadata rebuild, append, prefill, decode, combine as separate
    launches) with HIP events between the phases on the stream they run on, then
    (``one_call``) steps with the attention as one ragged_blocked_attention_concurrent
    call and events around it, and, for batches it runs as the mixed launch, that launch
    alone (RBKV_PHASE_ATTEND) between events.  Each loop bracketed by synchronisations;
    wall-clock seconds of the step loops and the per-step event times."""
    import torch

    from ragged_blocked_kv_amd import PHASE_ATTEND, PHASE_COMBINE, PHASE_DECODE, PHASE_PREFILL

    def step(ev=None):
        def mark(k):
            if ev is not None:
                ev[k].record(stream)
        mark(0)
        eng.rebuild(stream=stream)
        mark(1)
        eng.append_rotary(qkv, pool, wl.rope_base, stream=stream)
        mark(2)
        eng.attention_phase(PHASE_PREFILL, qkv, pool, out, stream=stream)
        mark(3)
        eng.attention_phase(PHASE_DECODE, qkv, pool, out, stream=stream)
        mark(4)
        eng.attention_phase(PHASE_COMBINE, qkv, pool, out, stream=stream)
        mark(5)

    for _ in range(warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(events[k])
    torch.cuda.synchronize()
    wall_serial = time.perf_counter() - t0

    # The same work with the prefill and the decodes sharing the chip
    # (ragged_blocked_attention_concurrent).
    def step_concurrent(ev=None):
        eng.rebuild(stream=stream)
        eng.append_rotary(qkv, pool, wl.rope_base, stream=stream)
        if ev is not None:
            ev[0].record(stream)
        eng.attention_concurrent(qkv, pool, out, stream=stream)
        if ev is not None:
            ev[1].record(stream)  # after the join: both streams' work is done

    wall, ts, mixed = None, None, None
    if one_call:
        for _ in range(warmup):
            step_concurrent()
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            step_concurrent(cev[k])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ts = np.array([cev[k][0].elapsed_time(cev[k][1]) for k in range(steps)])
    if one_call and mixed_launch(wl):
        mev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for k in range(steps):
            mev[k][0].record(stream)
            eng.attention_phase(PHASE_ATTEND, qkv, pool, out, stream=stream)
            mev[k][1].record(stream)
        torch.cuda.synchronize()
        mixed = np.array([mev[k][0].elapsed_time(mev[k][1]) for k in range(steps)])
    return {
        "phase_ms": {p: float(np.mean([events[k][j].elapsed_time(events[k][j + 1])
                                       for k in range(steps)]))
                     for j, p in enumerate(PHASES)},
        "step_ms": np.array([events[k][0].elapsed_time(events[k][5]) for k in range(steps)]),
        "attn_ms": np.array([events[k][2].elapsed_time(events[k][5]) for k in range(steps)]),
        "call_ms": ts, "mixed_ms": mixed, "wall_serial": wall_serial, "wall_call": wall,
    }


def figures(wl, tm):
    """The per-configuration figures: attention tokens/s and whole-attention HBM
    fraction (separate launches one after another, and the one-call attention), each
    kernel against its own peak (the mixed launch, the prefill and decode kernels of the
    separate launches), append and combine."""
    work = algorithmic_work(wl)
    ph = tm["phase_ms"]
    pct = lambda a: [round(float(np.percentile(a, q)) * 1e3, 1) for q in (10, 50, 90)]

    def attention(ms, samples):
        gbs = work["attention_bytes"] / (ms * 1e-3) / 1e9
        return {"us": round(ms * 1e3, 1), "us_p10_p50_p90": pct(samples),
                "tokens_per_s": wl.T / (ms * 1e-3), "attention_algorithmic_GBs": gbs,
                "hbm_frac_attention": gbs / HBM_PEAK_GBS}

    serial_ms = ph["prefill"] + ph["decode"] + ph["combine"]
    att = {"bytes": work["attention_bytes"], "serial": attention(serial_ms, tm["attn_ms"]),
           "call": None}
    if tm["call_ms"] is not None:
        att["call"] = attention(float(np.median(tm["call_ms"])), tm["call_ms"])
    both = bool((wl.n_new > 1).any()) and bool((wl.n_new == 1).any())
    att["timed_call"] = ("serial" if att["call"] is None else
                         "mixed launch" if mixed_launch(wl) else
                         "two streams" if both else "one stream")
    att["hbm_frac"] = (att["call"] or att["serial"])["hbm_frac_attention"]
    mixed = None
    if tm.get("mixed_ms") is not None:
        us = float(np.mean(tm["mixed_ms"])) * 1e3
        gbs = work["attention_bytes"] / (us * 1e-6) / 1e9
        mixed = {"kernel": "mixed_attn_kernel", "us": round(us, 2),
                 "us_p10_p50_p90": pct(tm["mixed_ms"]), "bytes": work["attention_bytes"],
                 "flops": work["prefill_flops"], "GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                 "mfma_frac": work["prefill_flops"] / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS}
    dec = pre = None
    # float32 batches run every item (chunks too) on the vector-ALU decode kernel
    dec_bytes = work["decode_bytes"] if wl.dtype == "bf16" else work["attention_bytes"]
    if dec_bytes > 0 and ph["decode"] > 0:
        gbs = dec_bytes / (ph["decode"] * 1e-3) / 1e9
        dec = {"kernel": decode_kernel_name(wl), "us": round(ph["decode"] * 1e3, 2),
               "bytes": dec_bytes, "GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
    if wl.dtype == "bf16" and work["prefill_flops"] > 0 and ph["prefill"] > 0:
        tfs = work["prefill_flops"] / (ph["prefill"] * 1e-3) / 1e12
        pre = {"kernel": "prefill_attn_kernel", "us": round(ph["prefill"] * 1e3, 2),
               "flops": work["prefill_flops"], "TFLOPs": tfs,
               "mfma_frac": tfs / MFMA_BF16_PEAK_TFS}
    app_gbs = work["append_bytes"] / (ph["append"] * 1e-3) / 1e9
    return {
        "S": wl.S, "T": wl.T, "dtype": wl.dtype,
        "attention": att,
        "mixed": mixed,
        "decode": dec,
        "prefill": pre,
        "append": {"us": round(ph["append"] * 1e3, 2), "bytes": work["append_bytes"],
                   "hbm_frac": app_gbs / HBM_PEAK_GBS},
        "combine_us": round(ph["combine"] * 1e3, 2),
        "rebuild_us": round(ph["rebuild"] * 1e3, 2),
        "step_us_p10_p50_p90": pct(tm["step_ms"]),
    }


def measure_config(name, dev, stream, steps, warmup):
    """One configuration end to end on its own buffers (its pool freed afterwards)."""
    import torch

    import workloads as W
    from ragged_blocked_kv_amd.runtime import Engine

    wl = W.make_workload(name)
    eng = Engine.for_workload(wl, device=dev)
    qkv = W.make_qkv(wl).to(dev)
    pool = W.make_pool_history(wl, device=dev)
    out = torch.empty((wl.T, wl.n_q_heads, wl.head_dim), dtype=qkv.dtype, device=dev)
    eng.finalize(wl.n_new, wl.seen, wl.block_lists, stream=stream)
    fig = figures(wl, time_steps(wl, eng, qkv, pool, out, stream, steps, warmup))
    del pool, qkv, out, eng
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return fig


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # Under sustained load the chip's clocks settle over the first ~20 steps of a mixed
    # batch (the mixed launch runs 5-7% slower there, then stays within a few percent):
    # the default warm-up covers that, so the timed steps measure the steady state.
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    # The extra legs launch library kernels on other batches; profiles of the main step
    # switch them off so that per-kernel averages cover the bench batch only.
    ap.add_argument("--no-ledger", action="store_true", help="skip the ledger host-cost leg")
    ap.add_argument("--no-serving", action="store_true", help="skip the SplitFuse serving leg")
    ap.add_argument("--no-gathers", action="store_true", help="skip the row-gather leg")
    ap.add_argument("--no-offload", action="store_true", help="skip the KV offload leg")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration measurements (every other workload)")
    ap.add_argument("--serial-only", action="store_true",
                    help="time only the serial step (value from it): every library kernel then "
                         "runs once per step with its whole work list, as the kernel-trace and "
                         "counter profiles need")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a device copy of BYTES (HBM counter calibration)")
    ap.add_argument("--traffic-from", nargs=5, default=None,
                    metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV",
                             "CAL_BYTES"),
                    help="reduce rocprofv3 counter CSVs into profiles/traffic.json and exit")
    ap.add_argument("--mfma-from", nargs=2, default=None, metavar=("PMC_CSV", "MFMAUTIL_CSV"),
                    help="reduce rocprofv3 matrix-core counter CSVs into profiles/mfma.json and "
                         "exit")
    args = ap.parse_args()
    if args.mfma_from:
        mfma_from_counters(args.mfma_from[0], args.mfma_from[1], args.workload,
                           os.path.join(ROOT, "profiles", "mfma.json"))
        return
    if args.traffic_from:
        f, w, cf, cw, cb = args.traffic_from
        traffic_from_counters(f, w, cf, cw, int(cb), args.workload,
                              os.path.join(ROOT, "profiles", "traffic.json"))
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 3)
        return
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              f"(shard by heads or by sequences and run one process per GPU instead)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as W
    from ragged_blocked_kv_amd.runtime import Engine

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = W.make_workload(args.workload)
    eng = Engine.for_workload(wl, device=dev)
    qkv_cpu = W.make_qkv(wl)
    qkv = qkv_cpu.to(dev)
    pool = W.make_pool_history(wl, device=dev)
    out = torch.empty((wl.T, wl.n_q_heads, wl.head_dim), dtype=qkv.dtype, device=dev)
    stream = torch.cuda.current_stream(dev)

    # Whole finalize call from Python (argument marshalling, host validation and packing,
    # upload, metadata kernel, synchronize), outside the timed region: the first (cold)
    # call and the median of ten more.
    fin_us = []
    for _ in range(11):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        eng.finalize(wl.n_new, wl.seen, wl.block_lists, stream=stream)
        torch.cuda.synchronize()
        fin_us.append((time.perf_counter() - t0) * 1e6)
    finalize_us = {"first": round(fin_us[0], 1), "median_warm": round(float(np.median(fin_us[1:])), 1)}

    # Native ledger around the same batch (host only; its finalize rewrites the device
    # metadata, so the bench batch is finalized again afterwards).
    ledger = None
    if not args.no_ledger:
        ledger = ledger_cost(wl, eng, stream)
        eng.finalize(wl.n_new, wl.seen, wl.block_lists, stream=stream)
        torch.cuda.synchronize()

    # CPU-baseline inputs: the pool history of the sampled sequences, copied before the
    # first append overwrites this pass's slots.
    hist = {}
    if not args.no_cpu_baseline:
        nb = [-(-(int(a) + int(b)) // wl.block_size) for a, b in zip(wl.n_new, wl.seen)]
        for i in range(wl.S):
            ids = torch.as_tensor(wl.block_lists[i][:nb[i]].astype(np.int64), device=dev)
            blk = pool.index_select(0, ids).cpu()
            hist[i] = blk.view(torch.int16).numpy().view(np.uint16) if wl.dtype == "bf16" \
                else blk.numpy()

    tm = time_steps(wl, eng, qkv, pool, out, stream, args.steps, args.warmup,
                    one_call=not args.serial_only)

    # Dynamic SplitFuse serving loop (rewrites the metadata and pool slots, so it runs
    # after the timed steps and after the CPU-baseline history has been copied).
    gathers = None if args.no_gathers else gathers_leg(wl, eng, stream)
    offload = None if args.no_offload else kv_offload_leg(wl, eng, pool, stream)
    serving = None if args.no_serving else serving_leg(wl, eng, qkv, pool, out, stream)

    fig = figures(wl, tm)
    phase_ms = tm["phase_ms"]
    wall = tm["wall_call"] if tm["wall_call"] is not None else tm["wall_serial"]
    ms_per_step = wall * 1e3 / args.steps
    if fig["mixed"]:
        # The timed step's dominant kernel does the whole attention: its HBM bound
        # (every K/V row, Q and output once at 8 TB/s) exceeds its matrix-core bound.
        mx = fig["mixed"]
        roof = {"kernel": mx["kernel"], "bound": "hbm", "achieved": mx["GBs"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": mx["hbm_frac"],
                "traffic": measured_traffic("attn_prefill.hip/mixed", wl.name),
                "per_launch": {"bytes": mx["bytes"], "flops": mx["flops"], "us": mx["us"]},
                "mfma_frac": mx["mfma_frac"]}
        if fig["decode"]:
            dc = fig["decode"]
            roof["decode_kernel"] = {"kernel": dc["kernel"], "us": dc["us"], "GBs": dc["GBs"],
                                     "frac": dc["hbm_frac"],
                                     "traffic": measured_traffic("attn_decode.hip", wl.name)}
        if fig["prefill"]:
            pf = fig["prefill"]
            roof["prefill_kernel"] = {"kernel": pf["kernel"], "us": pf["us"],
                                      "TFLOPs": pf["TFLOPs"], "frac": pf["mfma_frac"],
                                      "traffic": measured_traffic("attn_prefill.hip", wl.name)}
    elif fig["prefill"] and (not fig["decode"] or phase_ms["prefill"] >= phase_ms["decode"]):
        pf = fig["prefill"]
        roof = {"kernel": "prefill_attn_kernel", "bound": "mfma", "achieved": pf["TFLOPs"],
                "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s", "frac": pf["mfma_frac"],
                "traffic": measured_traffic("attn_prefill.hip", wl.name),
                "per_launch": {"flops": pf["flops"], "us": pf["us"]}}
    else:
        dc = fig["decode"]
        roof = {"kernel": dc["kernel"], "bound": "hbm", "achieved": dc["GBs"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dc["hbm_frac"],
                "traffic": measured_traffic("attn_decode.hip", wl.name),
                "per_launch": {"bytes": dc["bytes"], "us": dc["us"]}}
    # The step-level figure next to the dominant kernel's: the whole attention (every K/V
    # row and Q/output of the batch once) over the timed call's time.
    roof["attention_call"] = fig["attention"]["timed_call"]
    roof["attention_frac_hbm"] = fig["attention"]["hbm_frac"]
    roof["prefill_mfma_counters"] = measured_mfma("attn_prefill.hip", wl.name)

    configs = None
    if not args.no_configs:
        configs = {}
        for name in CONFIG_WORKLOADS:
            if name == wl.name:
                configs[name] = fig
                continue
            configs[name] = measure_config(name, dev, stream, min(args.steps, 20),
                                           min(args.warmup, 20))
            print(f"bench: measured {name}", file=sys.stderr, flush=True)

    base = None
    if not args.no_cpu_baseline:
        base = cpu_baseline(wl, qkv_cpu.view(torch.int16).numpy().view(np.uint16)
                            if wl.dtype == "bf16" else qkv_cpu.numpy(),
                            lambda i, nb: hist[i], args.cpu_seconds)

    rec = {
        "metric": "ragged attention tokens/s on 1 GPU + % peak HBM GB/s (decode) / % MFMA (prefill)",
        "value": wl.T * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "batch": f"{wl.S} sequences, {wl.T} new tokens "
                     f"({int((wl.n_new > 1).sum())} prefill chunks, {int((wl.n_new == 1).sum())} decodes)",
            "heads": f"{wl.n_q_heads} q / {wl.n_kv_heads} kv",
            "head_dim": wl.head_dim,
            "block_size": wl.block_size,
            "kv_pool_blocks": wl.num_blocks,
            "step": "metadata rebuild + rotary append + attention (prefill, decode, combine "
                    "one after another)" if args.serial_only else
                    "metadata rebuild + rotary append + attention (prefill tiles and decode "
                    "items from one launch of persistent workgroups, then the split-K combine)"
                    if mixed_launch(wl) else
                    "metadata rebuild + rotary append + attention (prefill chunks and decodes "
                    "sharing the chip on two streams, then the split-K combine)",
        },
        "roofline": roof,
        "cpu_baseline": base,
        "phases_us": {p: round(v * 1e3, 2) for p, v in phase_ms.items()},
        "attention_only": fig["attention"]["serial"],
        "step_us_p10_p50_p90": fig["step_us_p10_p50_p90"],
        "finalize_call_us": finalize_us,
        "attention_call": fig["attention"]["call"],
        "serial_step": {"ms_per_step": tm["wall_serial"] * 1e3 / args.steps,
                        "tokens_per_s": wl.T * args.steps / tm["wall_serial"],
                        "step": "the same phases one after another on one stream, with HIP "
                                "events between them (the per-kernel times above)"},
        "configs": configs,
        "ledger": ledger,
        "splitfuse_serving": serving,
        "gathers": gathers,
        "kv_offload": offload,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
