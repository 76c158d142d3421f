"""KV block offload (pool -> page-locked host buffer) and restore (host -> pool) on the
GPU, bit exact against the oracle: small pools in both dtypes and several block shapes,
and 1024 scattered blocks of the full-budget pool (256 MiB), restored into other
blocks with every block outside the destinations left untouched."""
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


def _tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


@pytest.mark.parametrize("dtype,hkv,bs,d,nb,n", [
    ("bf16", 2, 16, 128, 40, 13), ("f32", 4, 32, 64, 24, 24), ("bf16", 8, 64, 128, 30, 1),
    ("bf16", 1, 128, 64, 9, 5),
])
def test_offload_restore_bit_exact(dtype, hkv, bs, d, nb, n):
    import ragged_blocked_kv_amd as R
    print(f"kv offload {dtype} Hkv={hkv} bs={bs} d={d} blocks={nb} n={n}", flush=True)
    dev = torch.device("cuda:0")
    shape = R.Shape.make(max_tokens=64, max_seqs=8, num_blocks=nb, block_size=bs,
                         n_q_heads=hkv, n_kv_heads=hkv, head_dim=d, dtype=dtype)
    g = torch.Generator(device=dev).manual_seed(nb * 7 + n)
    pool = torch.randn((nb, 2, hkv, bs, d), generator=g, device=dev).to(_tdt(dtype))
    rng = np.random.default_rng(n)
    ids = rng.permutation(nb)[:n].astype(np.int32)
    st, nbytes = R.rbkv_kv_host_bytes(shape, n)
    assert st == R.OK
    host = torch.full((nbytes,), 0xAB, dtype=torch.uint8).pin_memory()
    before = _bits(pool)
    assert R.blocked_kv_offload(shape, pool, ids, host, nbytes) == R.OK
    torch.cuda.synchronize()
    slab_bytes = nbytes - 4 * n
    slabs = host[:slab_bytes].view(_tdt(dtype)).reshape(n, 2, hkv, bs, d)
    want = O.offload_blocks(before, ids)
    assert np.array_equal(_bits(slabs), want)
    assert host[slab_bytes:].view(torch.int32).numpy().tolist() == ids.tolist()
    assert np.array_equal(_bits(pool), before)  # offload leaves the pool alone
    dest = rng.permutation(nb)[:n].astype(np.int32)
    assert R.blocked_kv_restore(shape, pool, dest, host, nbytes) == R.OK
    torch.cuda.synchronize()
    assert np.array_equal(_bits(pool), O.restore_blocks(before, dest, want))
    assert host[slab_bytes:].view(torch.int32).numpy().tolist() == dest.tolist()


def test_offload_restore_full_budget_pool():
    import ragged_blocked_kv_amd as R
    print("kv offload full8192_gqa4: 1024 blocks", flush=True)
    dev = torch.device("cuda:0")
    wl = W.make_workload("full8192_gqa4")
    shape = R.Shape.make(max_tokens=wl.max_tokens, max_seqs=wl.max_seqs,
                         num_blocks=wl.num_blocks, block_size=wl.block_size,
                         n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                         head_dim=wl.head_dim, dtype=wl.dtype)
    pool = W.make_pool_history(wl, device=dev)
    rng = np.random.default_rng(5)
    perm = rng.permutation(wl.num_blocks).astype(np.int32)
    ids, dest = perm[:1024], perm[1024:2048]
    st, nbytes = R.rbkv_kv_host_bytes(shape, 1024)
    host = torch.empty(nbytes, dtype=torch.uint8).pin_memory()
    assert R.blocked_kv_offload(shape, pool, ids, host, nbytes) == R.OK
    torch.cuda.synchronize()
    blk = wl.pool_bytes() // wl.num_blocks
    slabs = host[:1024 * blk].view(torch.bfloat16).reshape((1024,) + tuple(pool.shape[1:]))
    for k in range(0, 1024, 1):  # every slab against its block, one by one
        assert torch.equal(slabs[k], pool[int(ids[k])].cpu()), k
    snapshot = pool.clone()
    assert R.blocked_kv_restore(shape, pool, dest, host, nbytes) == R.OK
    torch.cuda.synchronize()
    changed = (pool != snapshot).flatten(1).any(dim=1).cpu().numpy()
    assert set(np.nonzero(changed)[0].tolist()) <= set(dest.tolist())
    for k in range(0, 1024, 37):  # sampled destinations hold their source block
        assert torch.equal(pool[int(dest[k])], snapshot[int(ids[k])]), k
    sel = torch.as_tensor(dest.astype(np.int64), device=dev)
    src = torch.as_tensor(ids.astype(np.int64), device=dev)
    assert torch.equal(pool.index_select(0, sel), snapshot.index_select(0, src))
