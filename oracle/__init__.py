"""CPU oracle for ragged attention over a blocked KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or runs this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may use it.  It shares no code with the HIP library (no headers, tables,
kernels or helpers); the two meet only through the seeded inputs of ``workloads``.

Everything here is plain NumPy in float64 and is written to be checked by eye against
the definitions it cites.  See ``oracle.ragged_attention`` for the functions.

Parity status per function (what pins each one, in ``tests/test_oracle_pins.py``):

* ``bf16_from_f64`` / ``bf16_to_f64``   -- pinned: exhaustive neighbour search, torch casts
* ``batch_metadata``                    -- pinned: hand-derived fixture, invariants
* ``rope_inv_freq`` / ``rotate``        -- pinned: closed forms, d = 2 complex multiply,
                                           shift invariance; the half-split *pairing* is a
                                           reading (parity unpinned: the pages never
                                           describe rotary embeddings, and every invariant
                                           holds for the interleaved pairing too)
* ``append_rotary``                     -- pinned: slot placement brute force, canaries
* ``ragged_attention``                  -- pinned: brute-force dense attention, two-key
                                           closed form, single key, q = 0, convex hull,
                                           ragged = alone, block permutation / size
                                           invariance; the GQA head map h // G is a
                                           reading (parity unpinned beyond Hq = Hkv)
* ``embedding_gather`` / ``logits_gather`` -- pinned: hand fixture, last token derived
                                           from token_to_seq
* ``offload_blocks`` / ``restore_blocks``  -- pinned: hand example, round trip
* ``state_manager`` (allocator, ledger,  -- pinned: hand-derived walk
  compose, kv_requirements, ServingLoop)   (``tests/golden/ledger_walk.txt``), token-by-token
                                           block-growth simulation, conservation invariants,
                                           compose properties through can_schedule, loop =
                                           blocked oracle on one pass, chunking invariance
"""
from .ragged_attention import (  # noqa: F401
    bf16_to_f64,
    bf16_from_f64,
    storage_to_f64,
    f64_to_storage,
    batch_metadata,
    rope_inv_freq,
    rope_angles,
    rotate,
    append_rotary,
    gather_sequence_kv,
    sequence_attention,
    ragged_attention,
)
from .gather import embedding_gather, logits_gather  # noqa: F401
from .kv_offload import offload_blocks, restore_blocks  # noqa: F401
