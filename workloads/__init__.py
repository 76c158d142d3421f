"""Seeded synthetic inputs for ragged attention over a blocked KV cache.

This module only *draws inputs*: batch composition (new tokens and seen tokens per
sequence), per-sequence block-id lists, the new fused Q/K/V rows and the KV pool
history.  It holds none of the method's arithmetic (no prefix sums, no rotation, no
softmax) and imports neither the HIP library nor the oracle; both sides read the same
inputs from here.

Workload shapes follow the engine limits given in the tutorial chapter
"DeepSpeed-Inference and DeepSpeed-MII" (jwzheng96.github.io, section 10.3: at most 256
ragged sequences and 8192 ragged tokens per forward pass) and the Dynamic SplitFuse idea
described there and in section 10.10 (prefill chunks and single-token decodes share one
forward pass).  Sizes, head counts, block sizes and
distributions are the five measured configurations of this project:

========================  =====  ==========  ====  ====  ==================================
name                      dtype  Hq / Hkv    d     bs    batch
========================  =====  ==========  ====  ====  ==================================
tiny_f32                  f32    4 / 4       64    16    (37 new, 0 seen), (1, 50), (20, 30)
decode_mha32              bf16   32 / 32     128   64    64 decodes, seen ~ U[128, 2048]
splitfuse768_gqa4         bf16   32 / 8      128   64    1 chunk of 512 (seen 1024) + 256
                                                         decodes with seen ~ U[64, 4096]
full8192_gqa4             bf16   32 / 8      128   64    16 chunks 256..512 + 240 decodes,
                                                         8192 tokens, seen ~ U[0, 8192]
full8192_prefill_gqa4     bf16   32 / 8      128   64    the 16 chunks of full8192 alone
long_decode_gqa8          bf16   64 / 8      128   64    256 decodes, seen ~ LogU[4096, 32768]
========================  =====  ==========  ====  ====  ==================================

Readings where the configuration text leaves a choice open:

* integer Uniform[a, b] is inclusive; LogUniform seen = round(4096 * 8**u), u ~ U[0, 1);
* the 16 chunk sizes of full8192 are ``512 - r_k`` with ``r ~ Multinomial(240, 1/16)``
  (the only split that fills 8192 tokens with 16 chunks of 256..512 and 240 decodes);
* sequences are placed in the batch in a seeded random order;
* "randomly fragmented" pools hold ``ceil(1.25 * total blocks)`` blocks and hand out a
  seeded permutation of the block ids in batch order;
* the long-decode pool holds exactly the blocks needed and hands them out round-robin
  (in round r every sequence that still needs an r-th block takes the next id), so the
  blocks of one sequence are far apart in memory;
* splitfuse768 carries 257 sequences, so it runs with a sequence capacity of 512.

Random streams: workload ``k`` (k = 0..4 in the table order, the prefill-only slice
shares k = 3) uses ``numpy.random.SeedSequence(k).spawn(4)`` for lengths, block ids,
new Q/K/V and pool history.  All values are N(0, 1) drawn in float32 and stored in the
workload dtype by torch's own cast.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_workload",
    "random_workload",
    "make_qkv",
    "make_pool_history",
    "blocks_needed",
    "Request",
    "serving_trace",
    "serving_step_qkv",
]


def blocks_needed(n_tokens: int, block_size: int) -> int:
    """Number of fixed-size blocks a caller must hand out to hold ``n_tokens`` keys."""
    return -(-int(n_tokens) // int(block_size))


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str  # "f32" or "bf16"
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    rope_base: float
    n_new: np.ndarray  # int32 [S]
    seen: np.ndarray  # int32 [S]
    block_lists: List[np.ndarray]  # S int32 arrays (>= blocks needed each)
    max_tokens: int = 8192
    max_seqs: int = 256
    seed: int = 0

    @property
    def S(self) -> int:
        return int(len(self.n_new))

    @property
    def T(self) -> int:
        return int(np.sum(self.n_new, dtype=np.int64))

    @property
    def qkv_heads(self) -> int:
        return self.n_q_heads + 2 * self.n_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def streams(self):
        return np.random.SeedSequence(self.seed).spawn(4)

    def pool_shape(self):
        return (self.num_blocks, 2, self.n_kv_heads, self.block_size, self.head_dim)

    def pool_bytes(self) -> int:
        return int(np.prod(self.pool_shape())) * self.elem_bytes


def _torch_dtype(name: str):
    import torch

    return torch.float32 if name == "f32" else torch.bfloat16


def _torch_seed(ss: np.random.SeedSequence) -> int:
    return int(ss.generate_state(1, dtype=np.uint32)[0])


def _fragmented_lists(rng, need, pool_factor=1.25):
    total = int(sum(need))
    num_blocks = int(math.ceil(pool_factor * total))
    perm = rng.permutation(num_blocks).astype(np.int32)
    lists, at = [], 0
    for b in need:
        lists.append(perm[at:at + b].copy())
        at += b
    return num_blocks, lists


def _interleaved_lists(need):
    """Round-robin hand-out: in round r every sequence still needing an r-th block
    takes the next free id."""
    lists = [[] for _ in need]
    nxt, r = 0, 0
    while any(len(l) < b for l, b in zip(lists, need)):
        for i, b in enumerate(need):
            if r < b:
                lists[i].append(nxt)
                nxt += 1
        r += 1
    return nxt, [np.asarray(l, dtype=np.int32) for l in lists]


def _tiny_f32() -> Workload:
    s_len, s_ids, _, _ = np.random.SeedSequence(0).spawn(4)
    n_new = np.array([37, 1, 20], dtype=np.int32)
    seen = np.array([0, 50, 30], dtype=np.int32)
    bs, pool = 16, 32
    need = [blocks_needed(a + b, bs) for a, b in zip(n_new, seen)]
    perm = np.random.default_rng(s_ids).permutation(pool).astype(np.int32)
    lists, at = [], 0
    for b in need:
        lists.append(perm[at:at + b].copy())
        at += b
    return Workload("tiny_f32", "f32", 4, 4, 64, bs, pool, 1e4, n_new, seen, lists,
                    max_tokens=8192, max_seqs=256, seed=0)


def _decode_mha32() -> Workload:
    s_len, s_ids, _, _ = np.random.SeedSequence(1).spawn(4)
    rng = np.random.default_rng(s_len)
    S, bs = 64, 64
    seen = rng.integers(128, 2048, size=S, endpoint=True).astype(np.int32)
    n_new = np.ones(S, dtype=np.int32)
    need = [blocks_needed(a + b, bs) for a, b in zip(n_new, seen)]
    num_blocks, lists = _fragmented_lists(np.random.default_rng(s_ids), need)
    return Workload("decode_mha32", "bf16", 32, 32, 128, bs, num_blocks, 1e4, n_new, seen,
                    lists, seed=1)


def _splitfuse768() -> Workload:
    s_len, s_ids, _, _ = np.random.SeedSequence(2).spawn(4)
    rng = np.random.default_rng(s_len)
    bs = 64
    seen = np.concatenate([[1024], rng.integers(64, 4096, size=256, endpoint=True)])
    n_new = np.concatenate([[512], np.ones(256, dtype=np.int64)])
    order = rng.permutation(257)
    seen, n_new = seen[order].astype(np.int32), n_new[order].astype(np.int32)
    need = [blocks_needed(a + b, bs) for a, b in zip(n_new, seen)]
    num_blocks, lists = _fragmented_lists(np.random.default_rng(s_ids), need)
    return Workload("splitfuse768_gqa4", "bf16", 32, 8, 128, bs, num_blocks, 1e6, n_new,
                    seen, lists, max_tokens=8192, max_seqs=512, seed=2)


def _full8192() -> Workload:
    s_len, s_ids, _, _ = np.random.SeedSequence(3).spawn(4)
    rng = np.random.default_rng(s_len)
    bs = 64
    r = rng.multinomial(240, [1.0 / 16] * 16)
    chunks = 512 - r
    n_new = np.concatenate([chunks, np.ones(240, dtype=np.int64)])
    seen = rng.integers(0, 8192, size=256, endpoint=True)
    order = rng.permutation(256)
    n_new, seen = n_new[order].astype(np.int32), seen[order].astype(np.int32)
    need = [blocks_needed(a + b, bs) for a, b in zip(n_new, seen)]
    num_blocks, lists = _fragmented_lists(np.random.default_rng(s_ids), need)
    return Workload("full8192_gqa4", "bf16", 32, 8, 128, bs, num_blocks, 1e4, n_new, seen,
                    lists, seed=3)


def _full8192_prefill() -> Workload:
    full = _full8192()
    keep = np.nonzero(full.n_new > 1)[0]
    return Workload("full8192_prefill_gqa4", "bf16", 32, 8, 128, full.block_size,
                    full.num_blocks, full.rope_base, full.n_new[keep].copy(),
                    full.seen[keep].copy(), [full.block_lists[i] for i in keep], seed=3)


def _long_decode() -> Workload:
    s_len, _, _, _ = np.random.SeedSequence(4).spawn(4)
    rng = np.random.default_rng(s_len)
    S, bs = 256, 64
    u = rng.random(S)
    seen = np.rint(4096.0 * np.power(8.0, u)).astype(np.int32)
    n_new = np.ones(S, dtype=np.int32)
    need = [blocks_needed(a + b, bs) for a, b in zip(n_new, seen)]
    num_blocks, lists = _interleaved_lists(need)
    return Workload("long_decode_gqa8", "bf16", 64, 8, 128, bs, num_blocks, 1e4, n_new, seen,
                    lists, seed=4)


WORKLOADS = {
    "tiny_f32": _tiny_f32,
    "decode_mha32": _decode_mha32,
    "splitfuse768_gqa4": _splitfuse768,
    "full8192_gqa4": _full8192,
    "full8192_prefill_gqa4": _full8192_prefill,
    "long_decode_gqa8": _long_decode,
}


def make_workload(name: str) -> Workload:
    return WORKLOADS[name]()


def random_workload(seed: int, *, dtype="bf16", n_q_heads=4, n_kv_heads=2, head_dim=64,
                    block_size=16, max_new=40, max_seen=100, n_seqs: Optional[int] = None,
                    decode_frac=0.5, spare_blocks=7, extra_ids=0, max_tokens=8192,
                    max_seqs=256) -> Workload:
    """A small random ragged batch: a seeded mix of decodes and chunks with random
    seen lengths, fragmented block lists, and optionally ``extra_ids`` surplus ids at
    the end of each list (allowed: only the first blocks-needed ids are used)."""
    ss = np.random.SeedSequence([10_000, seed])
    s_len, s_ids, s_qkv, s_pool = ss.spawn(4)
    rng = np.random.default_rng(s_len)
    S = int(n_seqs if n_seqs is not None else rng.integers(1, 9))
    is_dec = rng.random(S) < decode_frac
    n_new = np.where(is_dec, 1, rng.integers(1, max_new, size=S, endpoint=True))
    seen = rng.integers(0, max_seen, size=S, endpoint=True)
    n_new, seen = n_new.astype(np.int32), seen.astype(np.int32)
    need = [blocks_needed(a + b, block_size) + extra_ids for a, b in zip(n_new, seen)]
    num_blocks = int(sum(need)) + spare_blocks
    perm = np.random.default_rng(s_ids).permutation(num_blocks).astype(np.int32)
    lists, at = [], 0
    for b in need:
        lists.append(perm[at:at + b].copy())
        at += b
    wl = Workload(f"random_{seed}", dtype, n_q_heads, n_kv_heads, head_dim, block_size,
                  num_blocks, 1e4, n_new, seen, lists, max_tokens=max_tokens,
                  max_seqs=max_seqs, seed=0)
    wl._streams = (s_len, s_ids, s_qkv, s_pool)
    return wl


def _stream(wl: Workload, k: int):
    st = getattr(wl, "_streams", None)
    return st[k] if st is not None else wl.streams()[k]


def make_qkv(wl: Workload):
    """New fused rows ``[T][Hq + 2*Hkv][d]`` (Q heads, then K heads, then V heads),
    N(0, 1) in float32 on the CPU, stored in the workload dtype."""
    import torch

    g = torch.Generator(device="cpu")
    g.manual_seed(_torch_seed(_stream(wl, 2)))
    x = torch.randn((wl.T, wl.qkv_heads, wl.head_dim), generator=g, dtype=torch.float32)
    return x.to(_torch_dtype(wl.dtype))


def make_pool_history(wl: Workload, device="cpu", chunk_blocks: int = 4096):
    """KV pool ``[num_blocks][2][Hkv][bs][d]`` filled with N(0, 1) history, drawn with
    torch's generator on ``device`` (block chunks keep the float32 temporaries small)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(_stream(wl, 3)))
    pool = torch.empty(wl.pool_shape(), dtype=_torch_dtype(wl.dtype), device=device)
    for b0 in range(0, wl.num_blocks, chunk_blocks):
        b1 = min(wl.num_blocks, b0 + chunk_blocks)
        shp = (b1 - b0,) + tuple(wl.pool_shape()[1:])
        pool[b0:b1] = torch.randn(shp, generator=g, dtype=torch.float32, device=device).to(
            pool.dtype)
    return pool


# --------------------------------------------------------------------------------------
# Multi-step serving traces
# --------------------------------------------------------------------------------------


@dataclasses.dataclass
class Request:
    uid: int
    arrival: int  # first step at which the request may be admitted
    prompt: int  # prompt tokens (the first pass's chunk)
    gen: int  # tokens generated after the prompt, one per later pass


def serving_trace(seed: int, n_requests: int, *, max_prompt: int, max_gen: int,
                  max_arrival: int, min_prompt: int = 1, min_gen: int = 1):
    """Seeded arrival list for a multi-step serving loop: uid, arrival step ~ U[0,
    max_arrival], prompt length ~ U[min_prompt, max_prompt], generated tokens ~ U[min_gen,
    max_gen] (integer uniforms, inclusive), sorted by arrival then uid.  Uids are large,
    scattered int64 values, so that a ledger cannot rely on small dense keys."""
    rng = np.random.default_rng(np.random.SeedSequence([20_000, seed]))
    arrival = rng.integers(0, max_arrival, size=n_requests, endpoint=True)
    prompt = rng.integers(min_prompt, max_prompt, size=n_requests, endpoint=True)
    gen = rng.integers(min_gen, max_gen, size=n_requests, endpoint=True)
    uids = rng.choice(np.arange(1, 1 << 20), size=n_requests, replace=False) * 7919 + \
        (1 << 40)
    reqs = [Request(int(u), int(a), int(p), int(g))
            for u, a, p, g in zip(uids, arrival, prompt, gen)]
    return sorted(reqs, key=lambda r: (r.arrival, r.uid))


def serving_step_qkv(seed: int, step: int, T: int, qkv_heads: int, head_dim: int,
                     dtype: str):
    """Fused new rows ``[T][qkv_heads][head_dim]`` of pass ``step`` of a serving loop:
    N(0, 1) in float32 on the CPU from a generator seeded by (seed, step), stored in
    ``dtype`` by torch's own cast."""
    import torch

    g = torch.Generator(device="cpu")
    g.manual_seed(_torch_seed(np.random.SeedSequence([30_000, seed, step])))
    x = torch.randn((T, qkv_heads, head_dim), generator=g, dtype=torch.float32)
    return x.to(_torch_dtype(dtype))
