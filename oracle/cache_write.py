"""Writing new K/V tokens into paged cache slots (O3), and exact decoding of
stored bits to fp64.

A slot is a flat index block * block_size + offset.  Token i with slot s
goes to cache[s // block_size, s % block_size, :, :] ([P2] question 12,
appending one token: logical block = position // block_size, offset =
position % block_size, write K and V there).  Readings: a negative slot
means "skip this token"; two tokens of one call never share a slot (the
oracle refuses such a call).  Storage conversion: same dtype -> the bits are
copied; fp8 cache -> the E4M3FN quantiser of `oracle.fp8` with the per-tensor
scale.

Pins (tests/test_oracle_cache_write.py): the page's worked examples of
token -> (block, offset), and a write/read round trip against the unpaged
token stream.
"""

from __future__ import annotations

import numpy as np
import torch

from . import fp8

_INT_VIEW = {torch.float32: torch.int32, torch.float16: torch.int16,
             torch.bfloat16: torch.int16, torch.uint8: torch.uint8}


def to_f64(t: torch.Tensor, kind: str, scale: float = 1.0) -> np.ndarray:
    """Stored values -> fp64, exactly.  kind is the storage kind: 'f32',
    'f16', 'bf16' (exact in fp64) or 'fp8' (uint8 codes times scale)."""
    if kind == "fp8":
        return fp8.decode(t.numpy(), scale)
    return t.to(torch.float64).numpy()


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor,
                      slot_mapping: np.ndarray, key_cache: torch.Tensor,
                      value_cache: torch.Tensor, kind: str,
                      k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """In place.  key/value [T, Hkv, D] in the source dtype; caches
    [N, bs, Hkv, D] ('fp8' caches are uint8 tensors)."""
    bs = key_cache.shape[1]
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = np.nonzero(slots >= 0)[0]
    s = slots[keep]
    if len(np.unique(s)) != len(s):
        raise ValueError("two tokens target the same cache slot")
    if len(s) and s.max() >= key_cache.shape[0] * bs:
        raise IndexError("slot outside the cache")
    blk = torch.from_numpy(s // bs)
    off = torch.from_numpy(s % bs)
    idx = torch.from_numpy(keep)
    for src, dst, sc in ((key, key_cache, k_scale), (value, value_cache, v_scale)):
        rows = src[idx]
        if kind == "fp8":
            codes = fp8.quantize(rows.to(torch.float32).numpy(), sc)
            dst[blk, off] = torch.from_numpy(codes)
        else:
            if rows.dtype != dst.dtype:
                raise TypeError("same-dtype write expected")
            # bit copy through an integer view
            iv = _INT_VIEW[dst.dtype]
            dst.view(iv)[blk, off] = rows.view(iv)
