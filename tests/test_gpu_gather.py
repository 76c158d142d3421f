"""Ragged embedding gather and last-token (logits) gather on the GPU, bit exact against
the oracle: random small batches in both dtypes and several row widths (one, two and
four 16-byte words per lane, partial slices), ids outside the table, and the full-budget
batch at Llama-2-7B widths (hidden 4096, vocabulary 32000) in the launch configuration
the benchmark times."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu


def _bits(x: torch.Tensor) -> np.ndarray:
    x = x.cpu()
    return x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 \
        else x.numpy()


def _engine(wl, dev):
    from ragged_blocked_kv_amd.runtime import Engine
    eng = Engine.for_workload(wl, device=dev)
    eng.finalize(wl.n_new, wl.seen, wl.block_lists)
    return eng


@pytest.mark.parametrize("seed,dtype,width", [
    (0, "bf16", 64), (1, "bf16", 2048), (2, "f32", 96), (3, "bf16", 4104),
    (4, "f32", 1028), (5, "bf16", 8), (6, "bf16", 32000), (7, "f32", 4),
])
def test_gathers_small(seed, dtype, width):
    print(f"gather seed={seed} {dtype} width={width}", flush=True)
    dev = torch.device("cuda:0")
    wl = W.random_workload(seed, dtype=dtype, max_new=30)
    eng = _engine(wl, dev)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(seed)
    vocab = 97
    table = torch.randn((vocab, width), generator=g).to(tdt)
    ids = torch.randint(-3, vocab + 3, (wl.T,), generator=g, dtype=torch.int32)
    ids[0] = vocab  # first id outside the table
    out = torch.full((wl.T, width), 7.0, dtype=tdt, device=dev)
    eng.embedding_gather(ids.to(dev), table.to(dev), out)
    rows = torch.randn((wl.T, width), generator=g).to(tdt)
    last = torch.full((wl.S, width), 7.0, dtype=tdt, device=dev)
    eng.logits_gather(rows.to(dev), last)
    torch.cuda.synchronize()
    cu = eng.metadata()["cu_seqlens"]
    assert np.array_equal(_bits(out), O.embedding_gather(_bits(table), ids.numpy()))
    assert np.array_equal(_bits(last), O.logits_gather(_bits(rows), cu))


def test_gathers_full_budget_batch():
    """8192 tokens / 256 sequences of the full-budget batch, hidden 4096 (embedding) and
    vocabulary-wide logits rows (32000), bf16."""
    print("gather full8192_gqa4 hidden 4096 vocab 32000", flush=True)
    dev = torch.device("cuda:0")
    wl = W.make_workload("full8192_gqa4")
    eng = _engine(wl, dev)
    g = torch.Generator().manual_seed(11)
    gd = torch.Generator(device=dev).manual_seed(12)
    vocab, hidden = 32000, 4096
    table = torch.randn((vocab, hidden), generator=gd, device=dev).to(torch.bfloat16)
    ids = torch.randint(0, vocab, (wl.T,), generator=g, dtype=torch.int32)
    out = torch.empty((wl.T, hidden), dtype=torch.bfloat16, device=dev)
    eng.embedding_gather(ids.to(dev), table, out)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), O.embedding_gather(_bits(table), ids.numpy()))
    logits = torch.randn((wl.T, vocab), generator=gd, device=dev).to(torch.bfloat16)
    last = torch.empty((wl.S, vocab), dtype=torch.bfloat16, device=dev)
    eng.logits_gather(logits, last)
    torch.cuda.synchronize()
    cu = eng.metadata()["cu_seqlens"]
    want = O.logits_gather(_bits(logits), cu)
    assert np.array_equal(_bits(last), want)


def test_gather_errors_on_device_buffers():
    import ragged_blocked_kv_amd as R
    dev = torch.device("cuda:0")
    wl = W.random_workload(9, max_new=10)
    eng = _engine(wl, dev)
    table = torch.zeros((10, 64), dtype=torch.bfloat16, device=dev)
    ids = torch.zeros(wl.T, dtype=torch.int32, device=dev)
    out = torch.zeros((wl.T, 64), dtype=torch.bfloat16, device=dev)
    b = eng.batch
    # buffers in host memory are refused before anything is launched
    host = torch.zeros((wl.T, 64), dtype=torch.bfloat16)
    assert R.ragged_logits_gather(b, host, 64, "bf16", out) == R.ERR_DEVICE_PTR
    assert R.ragged_embedding_gather(b, ids.cpu(), table, 10, 64, "bf16", out) == \
        R.ERR_DEVICE_PTR
    assert R.ragged_embedding_gather(b, ids, table.cpu(), 10, 64, "bf16", out) == \
        R.ERR_DEVICE_PTR
    assert R.ragged_embedding_gather(b, ids, table, 10, 64, "bf16", out) == R.OK
    torch.cuda.synchronize()
