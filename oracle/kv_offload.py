"""Plain CPU model of KV block offload and restore.

TEST INFRASTRUCTURE ONLY (see the package docstring): only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use it.

Source: "DeepSpeed Inference v2 source tour" (pyshine.com/deepspeed-2), section "The
front desk: put, query, can_schedule": the blocked KV cache copies chosen blocks out to
host memory to free device room and copies them back when their sequence is scheduled
again.  Reading: a block moves whole (keys and values of every kv head), the host copy
keeps the blocks in list order, and a restore may place them in other block ids.

Parity status: pinned by a hand-written example and the round-trip identity
(``tests/test_oracle_pins.py``).
"""
from __future__ import annotations

import numpy as np


def offload_blocks(pool, block_ids):
    """Host copy [n][2][Hkv][bs][d] of the listed pool blocks, in list order."""
    pool = np.asarray(pool)
    out = np.empty((len(block_ids),) + pool.shape[1:], dtype=pool.dtype)
    for k, b in enumerate(block_ids):
        out[k] = pool[int(b)]
    return out


def restore_blocks(pool, block_ids, host):
    """A copy of the pool with block block_ids[k] replaced by host slab k."""
    out = np.array(pool, copy=True)
    for k, b in enumerate(block_ids):
        out[int(b)] = host[k]
    return out
