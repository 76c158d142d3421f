"""Buffer plumbing around the C ABI for tests and benchmarks.

``Engine`` owns (through PyTorch) the buffers one layer shape needs -- pinned host
staging, device metadata, the split-K workspace -- and calls the three entry points on
a stream.  It does no arithmetic of the method: every step runs in librbkv's kernels.
It raises ``RbkvError`` on any non-OK status.
"""
from __future__ import annotations

import torch

from . import (DTYPE_BF16, DTYPE_F32, Batch, Shape, blocked_kv_append_rotary, check,
               ragged_batch_finalize, ragged_batch_rebuild, ragged_blocked_attention,
               ragged_blocked_attention_concurrent, ragged_blocked_attention_phase,
               ragged_embedding_gather, ragged_logits_gather,
               rbkv_metadata_bytes, rbkv_workspace_bytes)

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
_DTYPE_CODE = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}


class Engine:
    def __init__(self, *, max_tokens, max_seqs, num_blocks, block_size, n_q_heads,
                 n_kv_heads, head_dim, dtype, device="cuda"):
        if not torch.cuda.is_available():
            raise RuntimeError("Engine needs a HIP device")
        self.shape = Shape.make(max_tokens=max_tokens, max_seqs=max_seqs, num_blocks=num_blocks,
                                block_size=block_size, n_q_heads=n_q_heads,
                                n_kv_heads=n_kv_heads, head_dim=head_dim, dtype=dtype)
        self.dtype = dtype
        self.device = torch.device(device)
        st, dev_b, host_b = rbkv_metadata_bytes(self.shape)
        check(st, "rbkv_metadata_bytes")
        self.dev_meta = torch.empty(dev_b, dtype=torch.uint8, device=self.device)
        self.host_pinned = torch.empty(host_b, dtype=torch.uint8, pin_memory=True)
        self.workspace = torch.empty(0, dtype=torch.uint8, device=self.device)
        self.batch: Batch | None = None
        self._staged = None  # event after the last upload from host_pinned
        self._side = self._fork = self._join = None  # for attention_concurrent

    @classmethod
    def for_workload(cls, wl, device="cuda"):
        return cls(max_tokens=wl.max_tokens, max_seqs=wl.max_seqs, num_blocks=wl.num_blocks,
                   block_size=wl.block_size, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                   head_dim=wl.head_dim, dtype=wl.dtype, device=device)

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.dtype]

    def stream(self, stream=None):
        return torch.cuda.current_stream(self.device) if stream is None else stream

    def _staging_free(self):
        # The pinned staging buffer is rewritten by the next finalize: wait until the
        # stream has consumed the previous upload.
        if self._staged is not None:
            self._staged.synchronize()
            self._staged = None

    def _adopt(self, b: Batch, stream) -> Batch:
        self._staged = torch.cuda.Event()
        self._staged.record(stream)
        st, need = rbkv_workspace_bytes(self.shape, b)
        check(st, "rbkv_workspace_bytes")
        if need > self.workspace.numel():
            self.workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        self.batch = b
        return b

    def finalize(self, n_new, seen, block_lists, stream=None) -> Batch:
        self._staging_free()
        stream = self.stream(stream)
        st, b = ragged_batch_finalize(self.shape, n_new, seen, block_lists, self.host_pinned,
                                      self.host_pinned.numel(), self.dev_meta,
                                      self.dev_meta.numel(), stream)
        check(st, "ragged_batch_finalize")
        return self._adopt(b, stream)

    def finalize_state(self, state, stream=None) -> Batch:
        """Finalize the open batch of a ``state.StateManager`` ledger (its sequences, token
        counts and block lists go straight from the native ledger to the library)."""
        self._staging_free()
        stream = self.stream(stream)
        st, b = state.finalize_status(self.shape, self.host_pinned, self.host_pinned.numel(),
                                      self.dev_meta, self.dev_meta.numel(), stream)
        check(st, "rbkv_state_finalize")
        return self._adopt(b, stream)

    def rebuild(self, stream=None, batch=None):
        check(ragged_batch_rebuild(self.shape, batch or self.batch, self.stream(stream)),
              "ragged_batch_rebuild")

    def attention_phase(self, phase, qkv, kv_pool, out, stream=None, batch=None):
        check(ragged_blocked_attention_phase(self.shape, batch or self.batch, phase, qkv,
                                             kv_pool, out, self.workspace,
                                             self.workspace.numel(), self.stream(stream)),
              "ragged_blocked_attention_phase")

    def append_rotary(self, qkv, kv_pool, rope_base, stream=None, batch=None):
        check(blocked_kv_append_rotary(self.shape, batch or self.batch, qkv, kv_pool, rope_base,
                                       self.stream(stream)), "blocked_kv_append_rotary")

    def attention(self, qkv, kv_pool, out, stream=None, batch=None):
        b = batch or self.batch
        check(ragged_blocked_attention(self.shape, b, qkv, kv_pool, out, self.workspace,
                                       self.workspace.numel(), self.stream(stream)),
              "ragged_blocked_attention")

    def embedding_gather(self, token_ids, table, out, stream=None, batch=None):
        """out[t] = table[token_ids[t]] for the batch's tokens (ids outside the table give
        zero rows)."""
        check(ragged_embedding_gather(batch or self.batch, token_ids, table, table.shape[0],
                                      table.shape[1], _DTYPE_CODE[table.dtype], out,
                                      self.stream(stream)), "ragged_embedding_gather")

    def logits_gather(self, rows, out, stream=None, batch=None):
        """out[i] = rows[last new token of sequence i]."""
        check(ragged_logits_gather(batch or self.batch, rows, rows.shape[1],
                                   _DTYPE_CODE[rows.dtype], out, self.stream(stream)),
              "ragged_logits_gather")

    def attention_concurrent(self, qkv, kv_pool, out, stream=None, batch=None):
        """ragged_blocked_attention_concurrent: decodes on a side stream of this engine,
        prefill chunks on ``stream``, joined before the combine (same result)."""
        stream = self.stream(stream)
        if self._side is None:
            self._side = torch.cuda.Stream(device=self.device)  # default priority
            self._fork, self._join = torch.cuda.Event(), torch.cuda.Event()
            # torch creates an event's handle on its first record
            self._fork.record(stream)
            self._join.record(stream)
        check(ragged_blocked_attention_concurrent(
            self.shape, batch or self.batch, qkv, kv_pool, out, self.workspace,
            self.workspace.numel(), stream, self._side, self._fork, self._join),
            "ragged_blocked_attention_concurrent")

    def new_out(self, T=None):
        T = self.batch.T if T is None else T
        return torch.empty((T, self.shape.n_q_heads, self.shape.head_dim),
                           dtype=self.torch_dtype, device=self.device)

    def metadata(self, batch=None):
        """Device metadata of a finalized batch copied to host int32 arrays."""
        b = batch or self.batch
        base = self.dev_meta.data_ptr()
        u8 = self.dev_meta

        def arr(ptr, n):
            off = int(ptr) - base
            return u8[off:off + 4 * n].view(torch.int32).cpu().numpy()

        S, T = b.S, b.T
        return {
            "cu_seqlens": arr(b.cu_seqlens, S + 1),
            "seen": arr(b.seen, S),
            "kv_len": arr(b.kv_len, S),
            "block_offsets": arr(b.block_offsets, S + 1),
            "block_ids": arr(b.block_ids, b.n_blocks_used),
            "token_to_seq": arr(b.token_to_seq, T),
            "pos": arr(b.pos, T),
            "decode_work": arr(b.decode_work, 4 * b.n_decode_items).reshape(-1, 4),
            "prefill_work": arr(b.prefill_work, 4 * b.n_prefill_seqs).reshape(-1, 4),
            "combine_work": arr(b.combine_work, 4 * b.n_combine_items).reshape(-1, 4),
        }
