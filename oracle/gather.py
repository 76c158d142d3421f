"""Plain CPU model of the two row gathers that frame the layer stack over a ragged batch.

TEST INFRASTRUCTURE ONLY (see the package docstring): only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use it.

Source: "DeepSpeed Inference v2 source tour" (pyshine.com/deepspeed-2), section "Ragged
batches: packing a whole server into four tensors": the ragged embedding kernel gathers
embedding rows for the packed token stream, and the logits gather copies out only the
last-token row of each sequence for sampling.

Readings: a token id outside [0, vocab) yields a zero row (the library cannot refuse
device-resident ids without a synchronisation); rows are copied bit for bit, so both
functions work on the storage arrays (bf16 bit patterns or float32) unchanged.

Parity status: pinned by the hand-written fixture ``tests/golden/gather_examples.json``
and by the last-token rule derived independently from ``token_to_seq``
(``tests/test_oracle_pins.py``).
"""
from __future__ import annotations

import numpy as np


def embedding_gather(table, token_ids):
    """out[t] = table[token_ids[t]] row by row; a zero row where the id is not a row
    of the table."""
    table = np.asarray(table)
    vocab = table.shape[0]
    out = np.zeros((len(token_ids),) + table.shape[1:], dtype=table.dtype)
    for t, i in enumerate(token_ids):
        i = int(i)
        if 0 <= i < vocab:
            out[t] = table[i]
    return out


def logits_gather(rows, cu_seqlens):
    """out[i] = rows[cu_seqlens[i + 1] - 1]: the row of the last new token of every
    sequence, in batch order."""
    rows = np.asarray(rows)
    S = len(cu_seqlens) - 1
    out = np.empty((S,) + rows.shape[1:], dtype=rows.dtype)
    for i in range(S):
        out[i] = rows[int(cu_seqlens[i + 1]) - 1]
    return out
