"""Python binding of librbkv: ragged-batch attention over a blocked KV cache on MI355X.

Argument marshalling only.  Every step of the path -- metadata build, rotary append,
attention -- runs in the library's gfx950 kernels behind its C ABI (``include/rbkv.h``);
this module converts shapes, host arrays and device pointers and returns the C status
codes.  PyTorch is used only to own device memory and streams.  Importing this module
does not need a GPU, but it needs the built library: it raises if ``librbkv.so`` is
missing (build it with ``python -m ragged_blocked_kv_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "RbkvError", "Shape", "Batch", "lib", "status_string", "check",
    "rbkv_metadata_bytes", "rbkv_workspace_bytes", "ragged_batch_finalize",
    "blocked_kv_append_rotary", "ragged_blocked_attention", "ragged_blocked_attention_noalloc",
    "STATIC_SCRATCH_BYTES", "ragged_batch_rebuild",
    "ragged_blocked_attention_phase", "ragged_blocked_attention_concurrent",
    "ragged_embedding_gather", "ragged_logits_gather",
    "rbkv_kv_host_bytes", "blocked_kv_offload", "blocked_kv_restore", "EXPORTED_SYMBOLS", "PHASE_ALL", "PHASE_PREFILL",
    "PHASE_DECODE", "PHASE_COMBINE", "PHASE_ATTEND",
    "OK", "ERR_INVALID_ARG", "ERR_CAPACITY", "ERR_BLOCKS", "ERR_UNSUPPORTED",
    "ERR_WORKSPACE", "ERR_DEVICE_PTR", "ERR_HIP", "ERR_HOST_MEMORY", "DTYPE_F32", "DTYPE_BF16",
]

OK, ERR_INVALID_ARG, ERR_CAPACITY, ERR_BLOCKS, ERR_UNSUPPORTED = 0, 1, 2, 3, 4
ERR_WORKSPACE, ERR_DEVICE_PTR, ERR_HIP, ERR_HOST_MEMORY = 5, 6, 7, 8
DTYPE_F32, DTYPE_BF16 = 0, 1
PHASE_ALL, PHASE_PREFILL, PHASE_DECODE, PHASE_COMBINE, PHASE_ATTEND = 0, 1, 2, 3, 4
STATIC_SCRATCH_BYTES = 64 << 20  # RBKV_STATIC_SCRATCH_BYTES

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librbkv.so")

EXPORTED_SYMBOLS = (
    "rbkv_status_string",
    "rbkv_metadata_bytes",
    "rbkv_workspace_bytes",
    "ragged_batch_finalize",
    "ragged_batch_rebuild",
    "blocked_kv_append_rotary",
    "ragged_blocked_attention",
    "ragged_blocked_attention_noalloc",
    "ragged_blocked_attention_phase",
    "ragged_blocked_attention_concurrent",
    "ragged_embedding_gather",
    "ragged_logits_gather",
    "rbkv_kv_host_bytes",
    "blocked_kv_offload",
    "blocked_kv_restore",
    # include/rbkv_state.h (bound in ragged_blocked_kv_amd.state)
    "rbkv_allocator_create",
    "rbkv_allocator_destroy",
    "rbkv_allocator_allocate",
    "rbkv_allocator_free",
    "rbkv_allocator_free_count",
    "rbkv_state_create",
    "rbkv_state_destroy",
    "rbkv_state_counts",
    "rbkv_state_sequence",
    "rbkv_state_block_ids",
    "rbkv_state_query",
    "rbkv_state_can_schedule",
    "rbkv_state_compose",
    "rbkv_state_put",
    "rbkv_state_batch",
    "rbkv_state_finalize",
    "rbkv_state_post_forward",
    "rbkv_state_flush",
    "rbkv_state_offload",
    "rbkv_state_restore",
)


class RbkvError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = int(status)
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "max_tokens", "max_seqs", "num_blocks", "block_size", "n_q_heads", "n_kv_heads",
        "head_dim", "dtype")]

    @classmethod
    def make(cls, *, max_tokens, max_seqs, num_blocks, block_size, n_q_heads, n_kv_heads,
             head_dim, dtype):
        dt = {"f32": DTYPE_F32, "bf16": DTYPE_BF16}.get(dtype, dtype)
        return cls(int(max_tokens), int(max_seqs), int(num_blocks), int(block_size),
                   int(n_q_heads), int(n_kv_heads), int(head_dim), int(dt))


_P = ctypes.POINTER(ctypes.c_int32)


class Batch(ctypes.Structure):
    _fields_ = [("shape", Shape)] + [(n, ctypes.c_int32) for n in (
        "S", "T", "n_blocks_used", "split_tiles", "n_decode_items", "n_prefill_items",
        "n_partials", "n_combine_items", "n_prefill_seqs", "prefill_qtiles_max")] + [
        (n, ctypes.c_void_p) for n in (
        "cu_seqlens", "seen", "kv_len", "block_offsets", "block_ids", "token_to_seq", "pos",
        "decode_work", "prefill_work", "combine_work")]


_lib = None


def lib():
    """The loaded librbkv (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"librbkv.so not built at {LIB_PATH}; run "
                              "`python -m ragged_blocked_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.rbkv_status_string.restype = ctypes.c_char_p
        L.rbkv_status_string.argtypes = [ctypes.c_int32]
        L.rbkv_metadata_bytes.restype = ctypes.c_int32
        L.rbkv_metadata_bytes.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_size_t),
                                          ctypes.POINTER(ctypes.c_size_t)]
        L.rbkv_workspace_bytes.restype = ctypes.c_int32
        L.rbkv_workspace_bytes.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Batch),
                                           ctypes.POINTER(ctypes.c_size_t)]
        L.ragged_batch_finalize.restype = ctypes.c_int32
        L.ragged_batch_finalize.argtypes = [
            ctypes.POINTER(Shape), ctypes.c_int32, _P, _P, ctypes.POINTER(_P), _P,
            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
            ctypes.c_void_p, ctypes.POINTER(Batch)]
        L.ragged_batch_rebuild.restype = ctypes.c_int32
        L.ragged_batch_rebuild.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Batch),
                                           ctypes.c_void_p]
        L.ragged_blocked_attention_phase.restype = ctypes.c_int32
        L.ragged_blocked_attention_phase.argtypes = [
            ctypes.POINTER(Shape), ctypes.POINTER(Batch), ctypes.c_int32, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.blocked_kv_append_rotary.restype = ctypes.c_int32
        L.blocked_kv_append_rotary.argtypes = [
            ctypes.POINTER(Shape), ctypes.POINTER(Batch), ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_double, ctypes.c_void_p]
        L.ragged_embedding_gather.restype = ctypes.c_int32
        L.ragged_embedding_gather.argtypes = [
            ctypes.POINTER(Batch), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        L.ragged_logits_gather.restype = ctypes.c_int32
        L.ragged_logits_gather.argtypes = [
            ctypes.POINTER(Batch), ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p]
        L.ragged_blocked_attention_concurrent.restype = ctypes.c_int32
        L.ragged_blocked_attention_concurrent.argtypes = [
            ctypes.POINTER(Shape), ctypes.POINTER(Batch), ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p]
        L.rbkv_kv_host_bytes.restype = ctypes.c_int32
        L.rbkv_kv_host_bytes.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_size_t)]
        for fn in (L.blocked_kv_offload, L.blocked_kv_restore):
            fn.restype = ctypes.c_int32
            fn.argtypes = [ctypes.POINTER(Shape), ctypes.c_void_p, ctypes.c_int32, _P,
                           ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.ragged_blocked_attention.restype = ctypes.c_int32
        L.ragged_blocked_attention.argtypes = [
            ctypes.POINTER(Shape), ctypes.POINTER(Batch), ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.ragged_blocked_attention_noalloc.restype = ctypes.c_int32
        L.ragged_blocked_attention_noalloc.argtypes = [
            ctypes.POINTER(Shape), ctypes.POINTER(Batch), ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().rbkv_status_string(int(status)).decode()


def check(status: int, what: str = "rbkv") -> None:
    if status != OK:
        raise RbkvError(status, what)


def _ptr(x) -> Optional[int]:
    """Raw address of a tensor / integer / None."""
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    return int(x)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return None
    if hasattr(stream, "cuda_stream"):
        return int(stream.cuda_stream)
    return int(stream)


def rbkv_metadata_bytes(shape: Shape):
    """(status, dev_bytes, host_pinned_bytes)."""
    d, h = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = lib().rbkv_metadata_bytes(ctypes.byref(shape), ctypes.byref(d), ctypes.byref(h))
    return st, d.value, h.value


def rbkv_workspace_bytes(shape: Shape, batch: Batch):
    """(status, bytes)."""
    b = ctypes.c_size_t(0)
    st = lib().rbkv_workspace_bytes(ctypes.byref(shape), ctypes.byref(batch), ctypes.byref(b))
    return st, b.value


class _HostLists:
    """Keeps the int32 host arrays alive for the duration of a finalize call.  The block
    lists are packed into one flat array and the per-sequence pointers computed from its
    offsets, so marshalling costs a few vector operations rather than one ctypes object
    per sequence."""

    def __init__(self, n_new, seen, block_lists):
        self.n_new = np.ascontiguousarray(np.asarray(n_new, dtype=np.int32))
        self.seen = np.ascontiguousarray(np.asarray(seen, dtype=np.int32))
        self.S = S = len(block_lists)
        self.lens = np.fromiter(map(len, block_lists), dtype=np.int32, count=S)
        flat = np.concatenate(block_lists, axis=None) if S else np.zeros(0, dtype=np.int32)
        if flat.dtype != np.int32:
            if flat.size and (flat.min() < -2**31 or flat.max() >= 2**31):
                raise OverflowError("block id outside the int32 range")
            flat = flat.astype(np.int32)
        self.flat = np.ascontiguousarray(flat) if flat.size else np.zeros(1, dtype=np.int32)
        offsets = np.zeros(max(S, 1), dtype=np.uintp)
        if S > 1:
            np.cumsum(self.lens[:-1], out=offsets[1:], dtype=np.uintp)
        self.addrs = offsets * np.uintp(4) + np.uintp(self.flat.ctypes.data)
        self.ptrs = self.addrs.ctypes.data_as(ctypes.POINTER(_P))


def ragged_batch_finalize(shape: Shape, n_new: Sequence[int], seen: Sequence[int],
                          block_lists: Sequence[Sequence[int]], host_pinned, host_pinned_bytes,
                          dev_meta, dev_meta_bytes, stream=None, *, S: Optional[int] = None,
                          null_lists: bool = False):
    """(status, Batch).  ``host_pinned``/``dev_meta`` are tensors or raw addresses."""
    h = _HostLists(n_new, seen, block_lists)
    S = h.S if S is None else S
    out = Batch()
    st = lib().ragged_batch_finalize(
        ctypes.byref(shape), int(S), h.n_new.ctypes.data_as(_P), h.seen.ctypes.data_as(_P),
        None if null_lists else h.ptrs, h.lens.ctypes.data_as(_P), _ptr(host_pinned),
        int(host_pinned_bytes), _ptr(dev_meta), int(dev_meta_bytes), _stream(stream),
        ctypes.byref(out))
    return st, out


def blocked_kv_append_rotary(shape: Shape, batch: Batch, qkv, kv_pool, rope_base: float,
                             stream=None) -> int:
    return lib().blocked_kv_append_rotary(ctypes.byref(shape), ctypes.byref(batch), _ptr(qkv),
                                          _ptr(kv_pool), float(rope_base), _stream(stream))


def ragged_blocked_attention(shape: Shape, batch: Batch, qkv, kv_pool, out, workspace,
                             workspace_bytes: int, stream=None) -> int:
    return lib().ragged_blocked_attention(ctypes.byref(shape), ctypes.byref(batch), _ptr(qkv),
                                          _ptr(kv_pool), _ptr(out), _ptr(workspace),
                                          int(workspace_bytes), _stream(stream))


def ragged_blocked_attention_noalloc(shape: Shape, batch: Batch, qkv, kv_pool, out,
                                     stream=None) -> int:
    return lib().ragged_blocked_attention_noalloc(ctypes.byref(shape), ctypes.byref(batch),
                                                  _ptr(qkv), _ptr(kv_pool), _ptr(out),
                                                  _stream(stream))


def ragged_batch_rebuild(shape: Shape, batch: Batch, stream=None) -> int:
    return lib().ragged_batch_rebuild(ctypes.byref(shape), ctypes.byref(batch), _stream(stream))


def ragged_blocked_attention_phase(shape: Shape, batch: Batch, phase: int, qkv, kv_pool, out,
                                   workspace, workspace_bytes: int, stream=None) -> int:
    return lib().ragged_blocked_attention_phase(
        ctypes.byref(shape), ctypes.byref(batch), int(phase), _ptr(qkv), _ptr(kv_pool),
        _ptr(out), _ptr(workspace), int(workspace_bytes), _stream(stream))


def _dtype_code(dtype) -> int:
    return {"f32": DTYPE_F32, "bf16": DTYPE_BF16}.get(dtype, dtype)


def ragged_embedding_gather(batch: Batch, token_ids, table, vocab: int, width: int, dtype,
                            out, stream=None) -> int:
    return lib().ragged_embedding_gather(ctypes.byref(batch), _ptr(token_ids), _ptr(table),
                                         int(vocab), int(width), int(_dtype_code(dtype)),
                                         _ptr(out), _stream(stream))


def ragged_logits_gather(batch: Batch, rows, width: int, dtype, out, stream=None) -> int:
    return lib().ragged_logits_gather(ctypes.byref(batch), _ptr(rows), int(width),
                                      int(_dtype_code(dtype)), _ptr(out), _stream(stream))


def rbkv_kv_host_bytes(shape: Shape, n: int):
    """(status, bytes) of the page-locked buffer that holds n offloaded blocks."""
    b = ctypes.c_size_t(0)
    st = lib().rbkv_kv_host_bytes(ctypes.byref(shape), int(n), ctypes.byref(b))
    return st, b.value


def _kv_transfer(fn, shape, kv_pool, block_ids, host, host_bytes, stream):
    ids = np.ascontiguousarray(np.asarray(block_ids, dtype=np.int32))
    return fn(ctypes.byref(shape), _ptr(kv_pool), int(ids.size), ids.ctypes.data_as(_P),
              _ptr(host), int(host_bytes), _stream(stream))


def blocked_kv_offload(shape: Shape, kv_pool, block_ids, host, host_bytes, stream=None) -> int:
    return _kv_transfer(lib().blocked_kv_offload, shape, kv_pool, block_ids, host, host_bytes,
                        stream)


def blocked_kv_restore(shape: Shape, kv_pool, block_ids, host, host_bytes, stream=None) -> int:
    return _kv_transfer(lib().blocked_kv_restore, shape, kv_pool, block_ids, host, host_bytes,
                        stream)


def _event(ev) -> Optional[int]:
    if ev is None:
        return None
    if hasattr(ev, "cuda_event"):
        return int(ev.cuda_event)
    return int(ev)


def ragged_blocked_attention_concurrent(shape: Shape, batch: Batch, qkv, kv_pool, out, workspace,
                                        workspace_bytes: int, stream, side_stream, fork_event,
                                        join_event) -> int:
    """Events may be torch.cuda.Event objects that have been recorded once (torch creates
    the underlying event on its first record) or raw hipEvent_t addresses."""
    return lib().ragged_blocked_attention_concurrent(
        ctypes.byref(shape), ctypes.byref(batch), _ptr(qkv), _ptr(kv_pool), _ptr(out),
        _ptr(workspace), int(workspace_bytes), _stream(stream), _stream(side_stream),
        _event(fork_event), _event(join_event))
