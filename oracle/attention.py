"""Single-query decode attention over a paged KV cache, in fp64.

What is computed (O1, the plain definition): for every sequence b and query
head h,

    out[b, h] = softmax(scale * q[b, h] . K_b^T) V_b

where K_b, V_b are the first L_b = seq_lens[b] tokens of the sequence, read
through its block table, and the K/V head is the one the query head's group
shares.  This is scaled dot-product attention ([P1] `StandardAttentionMemory`
.attention_computation; [P2] question 4, decode step with a padding mask) for
one query token attending over a cache whose tokens live in physical blocks
([P3] code block `paged_attention`).

Second route (O2): the same result reached the way the pages describe the
kernel, block by block with a running maximum and running sum that rescale
the accumulated output ([P3] `paged_attention`; [P2] question 19), and by
splitting a sequence into partitions whose (max, sum, unnormalised output)
triples are merged afterwards.  The printed `paged_attention` listing
rescales the output by the already-rescaled running sum; read here as the
intended recurrence acc <- acc * exp(m_old - m_new), l <- l * exp(m_old -
m_new) + sum(p), out = acc / l, with one (m, l, acc) state per query head.

Readings where the pages are silent:
  * the score scale is an argument (the pages divide by sqrt(head_dim));
  * q head h uses kv head h // (Hq / Hkv) ([P2] question 7, repeat_interleave
    broadcast);
  * exactly seq_lens[b] cached tokens are attended (the token just written
    by the cache write is one of them; [P1] `KVCacheEssence.definition`);
  * seq_lens[b] == 0 gives an all-zero output row;
  * block-table entries past ceil(L_b / block_size) are never read.

Pins (tests/test_oracle_attention.py): torch's scaled_dot_product_attention
in fp64 on the unpaged K/V, a pure-Python brute force on tiny shapes, closed
forms (one token, constant values, zero query), invariance under permuting
physical blocks, NaN-poisoned unused slots, and O2 == O1 to 1e-12.
paged_decode_stored (tests/test_oracle_decode_stored.py): caches built and
decoded by hand (torch's float8_e4m3fn conversion times each tensor's own
scale) against torch's scaled_dot_product_attention in fp64, fp8 with
distinct K and V scales, GQA, a zero-length row, a `pairs` subset; bit-equal
to O1 for 32- and 16-bit storage.
"""

from __future__ import annotations

from typing import Iterable, List, Optional, Sequence

import numpy as np


# --- address translation ([P1] `BlockTableDesign.implementation`,
# get_token_block; [P2] question 11, read_kv_range) ------------------------

def token_address(table_row: np.ndarray, t: np.ndarray, block_size: int):
    """Token positions -> (physical block, offset inside the block)."""
    t = np.asarray(t, dtype=np.int64)
    logical = t // block_size
    offset = t % block_size
    physical = np.asarray(table_row, dtype=np.int64)[logical]
    return physical, offset


def gather_tokens(cache: np.ndarray, table_row: np.ndarray, L: int,
                  block_size: int) -> np.ndarray:
    """The first L tokens of one sequence, in logical order: [L, Hkv, D]."""
    if L == 0:
        return cache[:0, 0]
    phys, off = token_address(table_row, np.arange(L), block_size)
    if phys.min() < 0 or phys.max() >= cache.shape[0]:
        raise IndexError("block table entry outside the physical pool")
    return cache[phys, off]


def kv_head_for(q_head: int, group: int) -> int:
    """GQA/MQA sharing: consecutive groups of query heads share one kv head."""
    return q_head // group


# --- O1: the plain definition ------------------------------------------------

def softmax_attend(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                   scale: float) -> np.ndarray:
    """softmax(scale * q K^T) V for one query vector; fp64."""
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def paged_decode(query: np.ndarray, key_cache: np.ndarray,
                 value_cache: np.ndarray, block_tables: np.ndarray,
                 seq_lens: np.ndarray, scale: float, block_size: int,
                 heads: Optional[Iterable] = None) -> np.ndarray:
    """O1.  query [B, Hq, D]; caches [N, bs, Hkv, D] fp64 (already decoded);
    returns out [B, Hq, D] fp64.  `heads` limits the work to (b, h) pairs
    (others are left as NaN)."""
    B, Hq, D = query.shape
    Hkv = key_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    g = Hq // Hkv
    want = None if heads is None else set(map(tuple, heads))
    out = np.full((B, Hq, D), np.nan) if want is not None else np.zeros((B, Hq, D))
    for b in range(B):
        L = int(seq_lens[b])
        if want is not None and not any(p[0] == b for p in want):
            continue
        if L == 0:
            for h in range(Hq):
                out[b, h] = 0.0
            continue
        Kb = gather_tokens(key_cache, block_tables[b], L, block_size)
        Vb = gather_tokens(value_cache, block_tables[b], L, block_size)
        for h in range(Hq):
            if want is not None and (b, h) not in want:
                continue
            kvh = kv_head_for(h, g)
            out[b, h] = softmax_attend(query[b, h], Kb[:, kvh, :],
                                       Vb[:, kvh, :], scale)
    return out


def paged_decode_fast(query: np.ndarray, key_cache: np.ndarray,
                      value_cache: np.ndarray, block_tables: np.ndarray,
                      seq_lens: np.ndarray, scale: float,
                      block_size: int) -> np.ndarray:
    """O1 with the heads of one kv group batched into one matrix product
    (same arithmetic per (b, h) as `paged_decode`, for larger inputs)."""
    B, Hq, D = query.shape
    Hkv = key_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    g = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        Kb = gather_tokens(key_cache, block_tables[b], L, block_size)
        Vb = gather_tokens(value_cache, block_tables[b], L, block_size)
        for kvh in range(Hkv):
            Q = query[b, kvh * g:(kvh + 1) * g]           # [g, D]
            S = scale * (Q @ Kb[:, kvh, :].T)              # [g, L]
            W = np.exp(S - S.max(axis=1, keepdims=True))
            out[b, kvh * g:(kvh + 1) * g] = (W @ Vb[:, kvh, :]) / \
                W.sum(axis=1, keepdims=True)
    return out


# --- O2: block-wise online softmax and partition merge ----------------------

def online_decode_one(q: np.ndarray, key_cache: np.ndarray,
                      value_cache: np.ndarray, table_row: np.ndarray, L: int,
                      scale: float, block_size: int, kvh: int) -> np.ndarray:
    """The pages' block loop for one (sequence, query head): per logical
    block, look up the physical block, keep only the valid tokens of a
    partly filled last block, and fold its scores into the running
    (max, sum, output) state."""
    D = q.shape[0]
    m = -np.inf
    l = 0.0
    acc = np.zeros(D)
    n_blocks = -(-L // block_size)
    for i in range(n_blocks):
        phys = int(table_row[i])
        valid = min(block_size, L - i * block_size)
        k = key_cache[phys, :valid, kvh, :]
        v = value_cache[phys, :valid, kvh, :]
        s = scale * (k @ q)
        m_new = max(m, float(s.max()))
        alpha = np.exp(m - m_new)            # 0 on the first block
        p = np.exp(s - m_new)
        l = l * alpha + p.sum()
        acc = acc * alpha + p @ v
        m = m_new
    if L == 0:
        return np.zeros(D)
    return acc / l


def partition_triple(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                     scale: float):
    """(max, sum, unnormalised output) of one partition's tokens."""
    s = scale * (K @ q)
    m = float(s.max())
    p = np.exp(s - m)
    return m, float(p.sum()), p @ V


def merge_triples(triples: Sequence) -> np.ndarray:
    """Combine per-partition triples: rescale each to the global maximum."""
    M = max(t[0] for t in triples)
    num = sum(t[2] * np.exp(t[0] - M) for t in triples)
    den = sum(t[1] * np.exp(t[0] - M) for t in triples)
    return num / den


def split_points(L: int, partition: int) -> List[int]:
    return list(range(0, L, partition)) + [L]


def partitioned_decode_one(q, Kb, Vb, scale, bounds: Sequence[int]):
    """Split [0, L) at `bounds` (sorted, starting at 0, ending at L)."""
    triples = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        if b > a:
            triples.append(partition_triple(q, Kb[a:b], Vb[a:b], scale))
    if not triples:
        return np.zeros(q.shape[0])
    return merge_triples(triples)


def paged_decode_stored(query, key_cache, value_cache, kind: str,
                        k_scale: float, v_scale: float, block_tables: np.ndarray,
                        seq_lens: np.ndarray, scale: float, block_size: int,
                        pairs: Optional[Sequence] = None) -> np.ndarray:
    """O1 on caches kept in their storage format (CPU torch tensors; fp8 as
    uint8 codes).  Each sequence's tokens are gathered in storage format and
    decoded exactly to fp64 (fp8: code value times the per-tensor scale)
    before the plain definition is applied.  `pairs` limits the work to some
    (b, h); the other rows stay NaN."""
    import torch

    from .cache_write import to_f64

    q = query.to(torch.float64).numpy()
    B, Hq, D = q.shape
    Hkv = key_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    g = Hq // Hkv
    out = np.full((B, Hq, D), np.nan)
    by_b = {}
    for b, h in (pairs if pairs is not None else [(b, h) for b in range(B) for h in range(Hq)]):
        by_b.setdefault(int(b), []).append(int(h))
    for b, hs in by_b.items():
        L = int(seq_lens[b])
        if L == 0:
            out[b, hs] = 0.0
            continue
        phys, off = token_address(block_tables[b], np.arange(L), block_size)
        if phys.min() < 0 or phys.max() >= key_cache.shape[0]:
            raise IndexError("block table entry outside the physical pool")
        pi, oi = torch.from_numpy(phys), torch.from_numpy(off)
        Kb = to_f64(key_cache[pi, oi], kind, k_scale)          # [L, Hkv, D]
        Vb = to_f64(value_cache[pi, oi], kind, v_scale)
        for h in hs:
            kvh = kv_head_for(h, g)
            out[b, h] = softmax_attend(q[b, h], Kb[:, kvh, :], Vb[:, kvh, :], scale)
    return out
