"""Python entry points with the C ABI's names (include/pa.h).

Argument marshalling only: torch tensors become `pa_tensor` descriptors,
torch's current stream becomes the launch stream, and every step of the
computation runs in libpa.so.
"""

from __future__ import annotations

import ctypes
from ctypes import byref, c_int32, c_int64
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import PA_NUM_FLAGS, PaLaunch, PaTensor, check, load

PATH_AUTO, PATH_VALU, PATH_MFMA = 0, 1, 2

_CODES = {
    torch.float32: _lib.PA_F32,
    torch.float16: _lib.PA_F16,
    torch.bfloat16: _lib.PA_BF16,
    torch.float8_e4m3fn: _lib.PA_FP8_E4M3,
    torch.int32: _lib.PA_I32,
    torch.int64: _lib.PA_I64,
}


def _desc(t: torch.Tensor, fp8: bool = False, scale: float = 1.0) -> PaTensor:
    if t.dim() > 4:
        raise ValueError("at most 4 dimensions")
    d = PaTensor()
    d.data = t.data_ptr() if t.numel() else None
    if fp8 or t.dtype == torch.float8_e4m3fn:
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError("an fp8 tensor must be uint8 or float8_e4m3fn")
        d.dtype = _lib.PA_FP8_E4M3
    else:
        if t.dtype not in _CODES:
            raise TypeError(f"unsupported dtype {t.dtype}")
        d.dtype = _CODES[t.dtype]
    d.ndim = t.dim()
    for i, (s, st) in enumerate(zip(t.shape, t.stride())):
        d.shape[i] = s
        d.stride[i] = st
    d.scale = float(scale)
    return d


def _launch(ref: torch.Tensor, workspace: Optional[torch.Tensor] = None,
            partition_tokens: int = 0, path: int = PATH_AUTO,
            stream: Optional[torch.cuda.Stream] = None,
            error_flags: Optional[torch.Tensor] = None) -> PaLaunch:
    ln = PaLaunch()
    if error_flags is not None:
        if (error_flags.dtype != torch.int32 or error_flags.numel() < PA_NUM_FLAGS
                or not error_flags.is_contiguous()):
            raise ValueError(f"error_flags must be a contiguous int32 tensor of {PA_NUM_FLAGS}")
        ln.error_flags = error_flags.data_ptr()
    if ref.is_cuda:
        s = stream if stream is not None else torch.cuda.current_stream(ref.device)
        ln.stream = s.cuda_stream
    else:
        ln.stream = None
    if workspace is not None:
        ln.workspace = workspace.data_ptr()
        ln.workspace_bytes = workspace.numel() * workspace.element_size()
    ln.partition_tokens = int(partition_tokens)
    ln.path = int(path)
    return ln


def _own_workspace(nbytes: int, device: torch.device,
                   stream: Optional[torch.cuda.Stream]) -> torch.Tensor:
    """A workspace this module allocates for one call.  torch's caching
    allocator ties a block to the stream current at allocation; the kernels
    may run on another (`stream=`), so the block is also recorded on that
    stream: it is not handed out again until the work queued there so far
    has finished, even though the tensor is dropped when the call returns."""
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if stream is not None and ws.is_cuda:
        ws.record_stream(stream)
    return ws


def _is_fp8(t: torch.Tensor, kv_dtype: Optional[str]) -> bool:
    return kv_dtype == "fp8" or t.dtype == torch.float8_e4m3fn


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor,
                      key_cache: torch.Tensor, value_cache: torch.Tensor,
                      k_scale: float = 1.0, v_scale: float = 1.0,
                      kv_dtype: Optional[str] = None,
                      stream: Optional[torch.cuda.Stream] = None,
                      error_flags: Optional[torch.Tensor] = None) -> None:
    """pa_reshape_and_cache: key/value [T, Hkv, D] into slots of the caches."""
    fp8 = _is_fp8(key_cache, kv_dtype)
    args = (_desc(key), _desc(value), _desc(slot_mapping),
            _desc(key_cache, fp8, k_scale), _desc(value_cache, fp8, v_scale))
    ln = _launch(key_cache, stream=stream, error_flags=error_flags)
    check(load().pa_reshape_and_cache(*(byref(a) for a in args), byref(ln)))


def decode_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           block_size: int, max_blocks: int, partition_tokens: int = 0) -> int:
    return check(load().pa_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                  block_size, max_blocks, partition_tokens))


SCHEDULE_NAMES = {_lib.PA_SCHEDULE_SINGLE: "single", _lib.PA_SCHEDULE_PARTITIONS: "partitions",
                  _lib.PA_SCHEDULE_BALANCED: "balanced"}


def decode_plan(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                block_size: int, max_blocks: int, partition_tokens: int = 0) -> dict:
    """pa_decode_plan: {"schedule": "single" | "partitions" | "balanced",
    "partition_tokens": int, "workspace_bytes": int}."""
    info = _lib.PaDecodePlan()
    check(load().pa_decode_plan(batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_blocks, partition_tokens, byref(info)))
    return {"schedule": SCHEDULE_NAMES[info.schedule], "partition_tokens": info.partition_tokens,
            "workspace_bytes": info.workspace_bytes}


def decode(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
           value_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
           scale: float, block_size: int, num_kv_heads: int,
           k_scale: float = 1.0, v_scale: float = 1.0, kv_dtype: Optional[str] = None,
           workspace: Optional[torch.Tensor] = None, partition_tokens: int = 0,
           path: int = PATH_AUTO, stream: Optional[torch.cuda.Stream] = None,
           error_flags: Optional[torch.Tensor] = None) -> None:
    """pa_decode.  When the plan splits and no workspace is given, one is
    allocated here (torch owns it, and it is recorded on `stream`); pass
    `workspace` to avoid that."""
    fp8 = _is_fp8(key_cache, kv_dtype)
    if workspace is None:
        need = decode_workspace_bytes(query.shape[0], query.shape[1], num_kv_heads,
                                      query.shape[2], block_size, block_tables.shape[1],
                                      partition_tokens)
        if need > 0:
            workspace = _own_workspace(need, query.device, stream)
    args = (_desc(out), _desc(query), _desc(key_cache, fp8, k_scale),
            _desc(value_cache, fp8, v_scale), _desc(block_tables), _desc(seq_lens))
    ln = _launch(query, workspace, partition_tokens, path, stream, error_flags)
    check(load().pa_decode(*(byref(a) for a in args), ctypes.c_float(scale),
                           int(block_size), int(num_kv_heads), byref(ln)))


def decode_noalloc(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                   value_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                   scale: float, block_size: int, num_kv_heads: int,
                   k_scale: float = 1.0, v_scale: float = 1.0, kv_dtype: Optional[str] = None,
                   partition_tokens: int = 0, path: int = PATH_AUTO,
                   stream: Optional[torch.cuda.Stream] = None,
                   error_flags: Optional[torch.Tensor] = None) -> None:
    """pa_decode_noalloc: pa_decode with the library's own fixed device
    scratch; nothing is allocated, here or in the library."""
    fp8 = _is_fp8(key_cache, kv_dtype)
    args = (_desc(out), _desc(query), _desc(key_cache, fp8, k_scale),
            _desc(value_cache, fp8, v_scale), _desc(block_tables), _desc(seq_lens))
    ln = _launch(query, None, partition_tokens, path, stream, error_flags)
    check(load().pa_decode_noalloc(*(byref(a) for a in args), ctypes.c_float(scale),
                                   int(block_size), int(num_kv_heads), byref(ln)))


def decode_shared_prefix_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int,
                                         head_dim: int, block_size: int, max_blocks: int,
                                         prefix_tokens: int) -> int:
    return check(load().pa_decode_shared_prefix_workspace_bytes(
        batch, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks, prefix_tokens))


def decode_shared_prefix(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                         value_cache: torch.Tensor, block_tables: torch.Tensor,
                         seq_lens: torch.Tensor, prefix_blocks: torch.Tensor, prefix_tokens: int,
                         scale: float, block_size: int, num_kv_heads: int,
                         k_scale: float = 1.0, v_scale: float = 1.0,
                         kv_dtype: Optional[str] = None,
                         workspace: Optional[torch.Tensor] = None,
                         stream: Optional[torch.cuda.Stream] = None,
                         error_flags: Optional[torch.Tensor] = None) -> None:
    """pa_decode_shared_prefix: decode of a batch whose sequences share their
    first prefix_tokens tokens (the blocks in prefix_blocks).  Without a
    workspace one is allocated here (torch owns it)."""
    fp8 = _is_fp8(key_cache, kv_dtype)
    if workspace is None:
        need = decode_shared_prefix_workspace_bytes(query.shape[0], query.shape[1], num_kv_heads,
                                                    query.shape[2], block_size,
                                                    block_tables.shape[1], prefix_tokens)
        workspace = _own_workspace(max(need, 16), query.device, stream)
    args = (_desc(out), _desc(query), _desc(key_cache, fp8, k_scale),
            _desc(value_cache, fp8, v_scale), _desc(block_tables), _desc(seq_lens),
            _desc(prefix_blocks))
    ln = _launch(query, workspace, 0, PATH_AUTO, stream, error_flags)
    check(load().pa_decode_shared_prefix(*(byref(a) for a in args), int(prefix_tokens),
                                         ctypes.c_float(scale), int(block_size),
                                         int(num_kv_heads), byref(ln)))


def prefill(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
            value_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
            query_start_loc: torch.Tensor, max_query_len: int, scale: float, block_size: int,
            num_kv_heads: int, k_scale: float = 1.0, v_scale: float = 1.0,
            kv_dtype: Optional[str] = None,
            stream: Optional[torch.cuda.Stream] = None,
            error_flags: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None) -> None:
    """pa_prefill: causal attention of the packed new rows of every sequence
    over its cached tokens (the new tokens' K/V already written).  A bf16
    query with bf16 K/V takes the library's workspace for its f16 P x V
    path; without one it is allocated here (torch owns it), and an empty
    tensor runs the bf16 product instead."""
    fp8 = _is_fp8(key_cache, kv_dtype)
    if workspace is None and query.dtype == torch.bfloat16 and key_cache.dtype == torch.bfloat16:
        need = prefill_workspace_bytes(seq_lens.shape[0], query.shape[1], query.shape[0],
                                       max_query_len)
        workspace = _own_workspace(max(need, 4), query.device, stream)
    args = (_desc(out), _desc(query), _desc(key_cache, fp8, k_scale),
            _desc(value_cache, fp8, v_scale), _desc(block_tables), _desc(seq_lens),
            _desc(query_start_loc))
    ln = _launch(query, workspace, 0, PATH_AUTO, stream, error_flags)
    check(load().pa_prefill(*(byref(a) for a in args), int(max_query_len),
                            ctypes.c_float(scale), int(block_size), int(num_kv_heads),
                            byref(ln)))


def prefill_workspace_bytes(batch: int, num_q_heads: int, num_rows: int,
                            max_query_len: int) -> int:
    return check(load().pa_prefill_workspace_bytes(batch, num_q_heads, num_rows, max_query_len))


def copy_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor, block_pairs: torch.Tensor,
                kv_dtype: Optional[str] = None, stream: Optional[torch.cuda.Stream] = None,
                error_flags: Optional[torch.Tensor] = None) -> None:
    """pa_copy_blocks: key/value_cache[dst] = key/value_cache[src] per pair."""
    fp8 = _is_fp8(key_cache, kv_dtype)
    args = (_desc(key_cache, fp8, 1.0), _desc(value_cache, fp8, 1.0), _desc(block_pairs))
    ln = _launch(key_cache, stream=stream, error_flags=error_flags)
    check(load().pa_copy_blocks(*(byref(a) for a in args), byref(ln)))


def swap_blocks(dst_key_cache: torch.Tensor, dst_value_cache: torch.Tensor,
                src_key_cache: torch.Tensor, src_value_cache: torch.Tensor,
                block_pairs: torch.Tensor, kv_dtype: Optional[str] = None,
                stream: Optional[torch.cuda.Stream] = None,
                error_flags: Optional[torch.Tensor] = None) -> None:
    """pa_swap_blocks: dst_*[dst] = src_*[src] per (src, dst) pair; either
    pair of pools may be pinned host memory."""
    fp8 = _is_fp8(dst_key_cache, kv_dtype)
    args = (_desc(dst_key_cache, fp8, 1.0), _desc(dst_value_cache, fp8, 1.0),
            _desc(src_key_cache, fp8, 1.0), _desc(src_value_cache, fp8, 1.0), _desc(block_pairs))
    dev = dst_key_cache if dst_key_cache.is_cuda else src_key_cache
    ln = _launch(dev, stream=stream, error_flags=error_flags)
    check(load().pa_swap_blocks(*(byref(a) for a in args), byref(ln)))


def build_info() -> str:
    return load().pa_build_info().decode()


class BlockAllocator:
    """pa_alloc_*: ref-counted LIFO block allocator (host)."""

    def __init__(self, num_blocks: int, free_order: Optional[Sequence[int]] = None):
        lib = load()
        arr = None
        if free_order is not None:
            fo = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            arr = fo.ctypes.data_as(ctypes.POINTER(c_int32))
        h = lib.pa_alloc_create(int(num_blocks), arr)
        if not h:
            raise _lib.PaError(_lib.PA_ERR_INVALID_ARG, _lib.last_error())
        self._h = h
        self._lib = lib

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.pa_alloc_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def allocate(self) -> int:
        out = c_int32()
        check(self._lib.pa_alloc_allocate(self._h, byref(out)))
        return out.value

    def incref(self, block: int) -> None:
        check(self._lib.pa_alloc_incref(self._h, int(block)))

    def decref(self, block: int) -> None:
        check(self._lib.pa_alloc_decref(self._h, int(block)))

    def num_free(self) -> int:
        return check(self._lib.pa_alloc_num_free(self._h))

    def num_blocks(self) -> int:
        return check(self._lib.pa_alloc_num_blocks(self._h))

    def refcount(self, block: int) -> int:
        return check(self._lib.pa_alloc_refcount(self._h, int(block)))


class BlockManager:
    """pa_bm_*: per-sequence block tables over a BlockAllocator (host)."""

    def __init__(self, allocator: BlockAllocator, block_size: int):
        self._lib = load()
        self._alloc = allocator  # keep alive
        h = self._lib.pa_bm_create(allocator.handle, int(block_size))
        if not h:
            raise _lib.PaError(_lib.PA_ERR_INVALID_ARG, _lib.last_error())
        self._h = h
        self.block_size = int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.pa_bm_destroy(h)
            self._h = None

    def add_sequence(self, seq_id: int, shared_blocks: Sequence[int] = (),
                     shared_tokens: int = 0) -> None:
        arr = np.ascontiguousarray(np.asarray(list(shared_blocks), dtype=np.int32))
        ptr = arr.ctypes.data_as(ctypes.POINTER(c_int32)) if len(arr) else None
        check(self._lib.pa_bm_add_sequence(self._h, int(seq_id), ptr, len(arr), int(shared_tokens)))

    def append_slot(self, seq_id: int):
        slot, src, dst = c_int64(), c_int32(), c_int32()
        check(self._lib.pa_bm_append_slot(self._h, int(seq_id), byref(slot), byref(src), byref(dst)))
        return slot.value, src.value, dst.value

    def fork(self, parent: int, child: int) -> None:
        check(self._lib.pa_bm_fork(self._h, int(parent), int(child)))

    def free_sequence(self, seq_id: int) -> None:
        check(self._lib.pa_bm_free_sequence(self._h, int(seq_id)))

    def seq_len(self, seq_id: int) -> int:
        return check(self._lib.pa_bm_seq_len(self._h, int(seq_id)))

    def num_blocks_of(self, seq_id: int) -> int:
        return check(self._lib.pa_bm_num_blocks_of(self._h, int(seq_id)))

    def add_sequence_cached(self, cache: "PrefixCache", seq_id: int, tokens: Sequence[int]):
        """pa_bm_add_sequence_cached: admit a sequence through the prefix
        cache.  Returns (matched tokens, slots of the remaining tokens)."""
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        slots = np.empty(max(len(tok), 1), dtype=np.int64)
        k = check(self._lib.pa_bm_add_sequence_cached(
            self._h, cache._h, int(seq_id),
            tok.ctypes.data_as(ctypes.POINTER(c_int32)) if len(tok) else None, len(tok),
            slots.ctypes.data_as(ctypes.POINTER(c_int64))))
        return int(k), slots[:len(tok) - k].copy()

    def export(self, seq_ids: Sequence[int], max_blocks: int):
        ids = np.ascontiguousarray(np.asarray(list(seq_ids), dtype=np.int64))
        tables = np.empty((len(ids), max_blocks), dtype=np.int32)
        lens = np.empty(len(ids), dtype=np.int32)
        check(self._lib.pa_bm_export(self._h, ids.ctypes.data_as(ctypes.POINTER(c_int64)),
                                     len(ids), int(max_blocks),
                                     tables.ctypes.data_as(ctypes.POINTER(c_int32)),
                                     lens.ctypes.data_as(ctypes.POINTER(c_int32))))
        return tables, lens


class PrefixCache:
    """pa_pc_*: prefix cache mapping leading full blocks of token sequences
    to the physical blocks that hold their K/V (host)."""

    def __init__(self, allocator: BlockAllocator, block_size: int):
        self._lib = load()
        self._alloc = allocator  # keep alive: the cache releases through it
        h = self._lib.pa_pc_create(allocator.handle, int(block_size))
        if not h:
            raise _lib.PaError(_lib.PA_ERR_INVALID_ARG, _lib.last_error())
        self._h = h
        self.block_size = int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.pa_pc_destroy(h)
            self._h = None

    @staticmethod
    def _ints(xs, dtype=np.int32):
        arr = np.ascontiguousarray(np.asarray(list(xs), dtype=dtype))
        return arr, (arr.ctypes.data_as(ctypes.POINTER(c_int32)) if len(arr) else None)

    def match(self, tokens: Sequence[int], max_blocks: Optional[int] = None):
        """Physical ids of the longest cached run of leading full blocks; the
        caller receives one reference on each."""
        tok, tp = self._ints(tokens)
        n = len(tok) // self.block_size if max_blocks is None else int(max_blocks)
        out = np.zeros(max(n, 1), dtype=np.int32)
        k = check(self._lib.pa_pc_match(self._h, tp, len(tok),
                                        out.ctypes.data_as(ctypes.POINTER(c_int32)), n))
        return out[:k].tolist()

    def insert(self, tokens: Sequence[int], blocks: Sequence[int]) -> int:
        tok, tp = self._ints(tokens)
        blk, bp = self._ints(blocks)
        return check(self._lib.pa_pc_insert(self._h, tp, len(tok), bp, len(blk)))

    def evict(self, max_blocks: int) -> int:
        return check(self._lib.pa_pc_evict(self._h, int(max_blocks)))

    def size(self) -> int:
        return check(self._lib.pa_pc_size(self._h))
