"""Plain float64 CPU oracle for the three steps of ragged attention over a blocked KV
cache: batch metadata, rotary append into the block pool, and causal attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use it.

Sources, by page title and section:

* "DeepSpeed Inference v2 source tour" (pyshine.com/deepspeed-2), section "Ragged
  batches: packing a whole server into four tensors": the live tokens of all
  sequences are concatenated into one stream with no padding; a metadata buffer says
  where each sequence's tokens start and stop; a tokens-to-sequence map rides beside
  it; kernels read per-sequence integer block ids and address the KV pools directly.
* same page, section "The front desk: put, query, can_schedule": each sequence keeps
  integer block ids into flat, block-indexed pools, one pool per cache group, with key
  and value views split out of it.
* tutorial chapter "DeepSpeed-Inference and DeepSpeed-MII" (jwzheng96.github.io),
  section 10.10: the ragged batch carries offsets and ``cu_seqlens``; section 10.3 /
  10.10: Dynamic SplitFuse puts prefill chunks (many tokens) and decodes (one token)
  in the same forward pass, so a chunk continues a sequence that already has ``seen``
  tokens in the cache.
* The attention a transformer layer computes is softmax(Q K^T / sqrt(d)) V, causal,
  per sequence, with grouped-query heads; rotary position embedding is the usual
  rotation of (x_j, x_{j+d/2}) pairs by angle p * base**(-2j/d).  The pages name
  FlashAttention-style blocked attention but print neither formula, so these are the
  textbook definitions.

Readings of points the sources leave open (each is a choice, stated once here):

1. RoPE pairs element j with element j + d/2 ("rotate half", the Hugging Face Llama
   layout) and rotates the whole head; frequencies are base**(-2j/d).
2. Positions are absolute: token k of a chunk whose sequence has ``seen`` = s sits at
   position s + k.  Only the new Q and K are rotated; V never is; pool history is
   already-rotated K.
3. A value is rounded to the storage dtype (round to nearest, ties to even, straight
   from float64) exactly where it is stored: rotated Q back into its row, rotated K and
   raw V into the pool, the attention output.  Everything else is float64 here.
4. Scale 1/sqrt(d), natural-exp softmax, no soft cap, no window.
5. Causal alignment is bottom-right: the query at position p sees keys 0..p of its own
   sequence, which for a chunk with seen > 0 includes all of its history.
6. Grouped-query attention maps query head h to kv head h // G with G = Hq / Hkv.
7. Fused rows are ``qkv[T][Hq + 2*Hkv][d]``: Q heads, then K heads, then V heads.
8. The pool is ``pool[num_blocks][2][Hkv][bs][d]``: index 0 holds keys, 1 values.
   Key p of a sequence lives in block ``block_ids[p // bs]`` at slot ``p % bs``.
9. A block list longer than needed is allowed; only its first ceil(L / bs) ids count.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------------------
# Storage dtypes
# --------------------------------------------------------------------------------------


def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to float64, exactly: a bfloat16 is the upper half
    of a binary32 pattern."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_from_f64(x) -> np.ndarray:
    """float64 to bfloat16 bit patterns, round to nearest with ties to even, taken in
    one step from binary64 (no intermediate binary32 rounding).

    bfloat16 keeps 8 significant bits, binary64 has 53, so the low 45 fraction bits of
    a normal binary64 number are dropped with RNE.  Finite inputs inside the normal
    binary32 range are required (every value on this path is).
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_from_f64: non-finite input")
    a = np.abs(x)
    if np.any((a != 0) & ((a < 2.0 ** -126) | (a >= 2.0 ** 127))):
        raise ValueError("bf16_from_f64: input outside the normal binary32 range")
    u = x.view(np.uint64)
    drop = np.uint64(45)
    half = np.uint64(1) << np.uint64(44)
    lsb = (u >> drop) & np.uint64(1)
    r = (u + (half - np.uint64(1)) + lsb) >> drop << drop
    y = r.view(np.float64)  # exactly representable in binary32 (8 significant bits)
    return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def storage_to_f64(arr, dtype: str) -> np.ndarray:
    """Storage array (float32 values, or bfloat16 bit patterns as uint16) to float64."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(arr)
    raise ValueError(dtype)


def f64_to_storage(x, dtype: str) -> np.ndarray:
    """float64 to the storage dtype, round to nearest even (NumPy's binary64 to binary32
    conversion is RNE)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        return bf16_from_f64(x)
    raise ValueError(dtype)


# --------------------------------------------------------------------------------------
# Step 1: ragged batch metadata
# --------------------------------------------------------------------------------------


def batch_metadata(n_new, seen, block_lists, block_size):
    """Device metadata of one ragged batch, as the pages' finalize produces it: where
    each sequence's new tokens start and stop in the packed stream (``cu_seqlens``),
    its seen tokens and total cached length, its block table (the first
    ceil(kv_len / bs) ids of its list, concatenated, with ``block_offsets`` marking
    where each sequence's table starts) and, per packed token, the owning sequence and
    the absolute position.  All int32.
    """
    n_new = [int(v) for v in n_new]
    seen = [int(v) for v in seen]
    S = len(n_new)
    cu = [0]
    for i in range(S):
        cu.append(cu[-1] + n_new[i])
    kv_len = [seen[i] + n_new[i] for i in range(S)]
    n_blocks = [-(-kv_len[i] // block_size) for i in range(S)]
    block_offsets = [0]
    flat = []
    for i in range(S):
        ids = list(np.asarray(block_lists[i]).tolist())
        if len(ids) < n_blocks[i]:
            raise ValueError(f"sequence {i}: {len(ids)} block ids < {n_blocks[i]} needed")
        flat.extend(ids[:n_blocks[i]])
        block_offsets.append(block_offsets[-1] + n_blocks[i])
    token_to_seq, pos = [], []
    for i in range(S):
        for k in range(n_new[i]):
            token_to_seq.append(i)
            pos.append(seen[i] + k)
    i32 = lambda v: np.asarray(v, dtype=np.int32)
    return {
        "cu_seqlens": i32(cu),
        "seen": i32(seen),
        "kv_len": i32(kv_len),
        "block_offsets": i32(block_offsets),
        "block_ids": i32(flat),
        "token_to_seq": i32(token_to_seq),
        "pos": i32(pos),
    }


# --------------------------------------------------------------------------------------
# Step 2: rotary embedding and append into the block pool
# --------------------------------------------------------------------------------------


def rope_inv_freq(head_dim: int, base: float) -> np.ndarray:
    """theta_j = base ** (-2j / d) for j = 0 .. d/2 - 1 (float64)."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * j / np.float64(head_dim))


def rope_angles(positions, head_dim: int, base: float) -> np.ndarray:
    """Angles p * theta_j, shape [len(positions), d/2], float64."""
    p = np.asarray(positions, dtype=np.float64)
    return p[:, None] * rope_inv_freq(head_dim, base)[None, :]


def rotate(x, angles) -> np.ndarray:
    """Rotate each pair (x_j, x_{j+d/2}) of the last axis by ``angles[..., j]``:
    x'_j = x_j cos a - x_{j+d/2} sin a;  x'_{j+d/2} = x_{j+d/2} cos a + x_j sin a."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    c, s = np.cos(angles), np.sin(angles)
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def append_rotary(qkv, pool, meta, n_q_heads, n_kv_heads, block_size, rope_base, dtype):
    """Rotate the new Q and K rows at their absolute positions and store rotated K and
    raw V into the pool slots of their sequence.

    ``qkv``: storage array [T][Hq + 2 Hkv][d]; ``pool``: storage array
    [num_blocks][2][Hkv][bs][d].  Returns new copies (qkv with rotated Q heads, pool
    with the new slots written); the inputs are not modified.  ``rope_base <= 0``
    means no rotation (placement only).
    """
    qkv_out = np.array(qkv, copy=True)
    pool_out = np.array(pool, copy=True)
    T, _, d = qkv_out.shape
    Hq, Hkv = n_q_heads, n_kv_heads
    pos = meta["pos"]
    x = storage_to_f64(qkv_out, dtype)
    q, k, v = x[:, :Hq], x[:, Hq:Hq + Hkv], x[:, Hq + Hkv:]
    if rope_base > 0:
        ang = rope_angles(pos, d, rope_base)[:, None, :]  # [T, 1, d/2]
        q = rotate(q, ang)
        k = rotate(k, ang)
    qkv_out[:, :Hq] = f64_to_storage(q, dtype)
    k_st = f64_to_storage(k, dtype)
    v_st = np.asarray(qkv_out[:, Hq + Hkv:])
    for t in range(T):
        i = int(meta["token_to_seq"][t])
        p = int(pos[t])
        blk = int(meta["block_ids"][int(meta["block_offsets"][i]) + p // block_size])
        slot = p % block_size
        pool_out[blk, 0, :, slot, :] = k_st[t]
        pool_out[blk, 1, :, slot, :] = v_st[t]
    return qkv_out, pool_out


# --------------------------------------------------------------------------------------
# Step 3: causal attention per sequence over its blocks
# --------------------------------------------------------------------------------------


def gather_sequence_kv(pool, ids, length, block_size, dtype):
    """Contiguous K, V [length][Hkv][d] (float64) of one sequence, key by key from its
    block ids: key p comes from block ids[p // bs], slot p % bs."""
    Hkv, d = pool.shape[2], pool.shape[4]
    K = np.empty((length, Hkv, d), dtype=np.float64)
    V = np.empty((length, Hkv, d), dtype=np.float64)
    for p in range(0, length, block_size):
        blk = int(ids[p // block_size])
        m = min(block_size, length - p)
        # pool[blk][0] is [Hkv][bs][d]; move the slot axis first
        K[p:p + m] = storage_to_f64(pool[blk, 0, :, :m, :], dtype).transpose(1, 0, 2)
        V[p:p + m] = storage_to_f64(pool[blk, 1, :, :m, :], dtype).transpose(1, 0, 2)
    return K, V


def sequence_attention(q, K, V, positions):
    """Causal grouped-query attention of one sequence's new tokens.

    q: [n][Hq][d] rotated queries (float64); K, V: [L][Hkv][d]; positions: [n]
    absolute positions.  Query (t, h) attends to keys 0..positions[t] of kv head
    h // G with weights softmax(q . k / sqrt(d)), max subtracted in float64.
    Returns [n][Hq][d] float64.
    """
    n, Hq, d = q.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    out = np.empty((n, Hq, d), dtype=np.float64)
    visible = np.arange(L)[None, :] <= np.asarray(positions)[:, None]  # [n, L]
    scale = 1.0 / np.sqrt(np.float64(d))
    for h in range(Hq):
        g = h // G
        z = (q[:, h, :] @ K[:, g, :].T) * scale  # [n, L]
        z = np.where(visible, z, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        w = np.exp(z)
        w = w / w.sum(axis=1, keepdims=True)
        out[:, h, :] = w @ V[:, g, :]
    return out


def ragged_attention(qkv_rot, pool, meta, n_q_heads, n_kv_heads, block_size, dtype,
                     seqs=None):
    """Attention output [T][Hq][d] (float64) for every new token of the batch, computed
    sequence by sequence from the gathered contiguous K/V.  ``qkv_rot`` holds the
    rotated Q (storage dtype, as stored by the append step); ``pool`` already holds the
    new keys and values.  ``seqs`` restricts the work to some sequences (rows of other
    sequences are NaN)."""
    T, _, d = qkv_rot.shape
    Hq = n_q_heads
    out = np.full((T, Hq, d), np.nan, dtype=np.float64)
    cu, kv_len, bo = meta["cu_seqlens"], meta["kv_len"], meta["block_offsets"]
    S = len(kv_len)
    for i in (range(S) if seqs is None else seqs):
        t0, t1 = int(cu[i]), int(cu[i + 1])
        ids = meta["block_ids"][int(bo[i]):int(bo[i + 1])]
        K, V = gather_sequence_kv(pool, ids, int(kv_len[i]), block_size, dtype)
        q = storage_to_f64(qkv_rot[t0:t1, :Hq, :], dtype)
        out[t0:t1] = sequence_attention(q, K, V, meta["pos"][t0:t1])
    return out
