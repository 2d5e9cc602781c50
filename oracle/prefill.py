"""Causal multi-token (prefill) attention over a paged KV cache, in fp64.
TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed (O5).  A prefill call brings n_b new query tokens for each
sequence b whose K/V have already been written into the cache, so that the
cache now holds L_b = seq_lens[b] tokens of the sequence and the new ones
are the last n_b of them.  Query row i of sequence b (0 <= i < n_b) sits at
position p = L_b - n_b + i and attends, causally, to the tokens at
positions 0..p:

    out[row, h] = softmax(scale * q[row, h] . K_b[0..p]^T) V_b[0..p]

with the kv head shared by the query head's group.  With n_b == L_b this is
ordinary causal self-attention over the prompt ([P2] question 6,
`MHAWithCache`, prefill branch: lower-triangular mask, masked scores set to
-inf, softmax, times V); with n_b == 1 it is the decode step of the decode
oracle; in between, the earlier L_b - n_b tokens are context that is already
cached (a chunked prompt, or a prefix shared through the prefix cache).
The K/V are read through the block table as for decode ([P2] question 19:
outer loop over query tiles, inner loop over the logical KV blocks looked
up in the table, online softmax, normalise at the end; [P2] question 3,
section 3.3: the prefill pass stores each K/V block into the cache).

Readings where the pages are silent:
  * queries come packed, sequence after sequence, [T, Hq, D]; the rows of
    sequence b are query_start_loc[b] .. query_start_loc[b+1] - 1;
  * the new tokens' K/V are in the cache before attention is taken (the
    decode branch of the same `MHAWithCache` writes first, then reads), so
    the query at position p sees its own key;
  * the mask is aligned to the end of the sequence (row i sits at
    L_b - n_b + i), which for n_b == L_b is the printed lower-triangular
    mask;
  * a row whose position would be negative (n_b > L_b) attends no token and
    its output is zero, like a zero-length decode sequence;
  * the score scale is an argument (the printed module divides by
    sqrt(head_dim)).

Pins (tests/test_oracle_prefill.py): torch's scaled_dot_product_attention in
fp64 with is_causal on the unpaged prompt (n_b == L_b) and with an explicit
end-aligned boolean mask (chunked), the decode oracle for n_b == 1, the
last rows of a whole-prompt prefill equal to a chunked prefill over the
same tokens, the first row equal to the first value row, a pure-Python
brute force on tiny shapes, and invariance under permuting physical blocks.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .attention import gather_tokens


def row_positions(n: int, L: int) -> np.ndarray:
    """Positions of a sequence's n new rows when the cache holds L tokens."""
    return np.arange(n, dtype=np.int64) + (L - n)


def causal_attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, pos: np.ndarray,
                  scale: float) -> np.ndarray:
    """Rows Q [n, D] at positions pos over keys K, V [L, D]: each row's
    scores against keys after its position are masked out (-inf) before the
    softmax; a row that keeps no key gives zeros."""
    n = Q.shape[0]
    out = np.zeros((n, V.shape[1]))
    if n == 0 or K.shape[0] == 0:
        return out
    S = scale * (Q @ K.T)                                   # [n, L]
    keep = np.arange(K.shape[0])[None, :] <= pos[:, None]   # [n, L]
    S = np.where(keep, S, -np.inf)
    live = keep.any(axis=1)
    if not live.any():
        return out
    Sl = S[live]
    W = np.exp(Sl - Sl.max(axis=1, keepdims=True))          # masked -> 0
    out[live] = (W @ V) / W.sum(axis=1, keepdims=True)
    return out


def paged_prefill(query: np.ndarray, key_cache: np.ndarray,
                  value_cache: np.ndarray, block_tables: np.ndarray,
                  seq_lens: np.ndarray, query_start_loc: np.ndarray,
                  scale: float, block_size: int,
                  rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """O5.  query [T, Hq, D]; caches [N, bs, Hkv, D] fp64 (already decoded);
    returns out [T, Hq, D] fp64.  `rows` limits the work to some packed rows
    (the others are left as NaN)."""
    T, Hq, D = query.shape
    Hkv = key_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    g = Hq // Hkv
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    B = len(seq_lens)
    if len(qsl) != B + 1 or qsl[0] != 0 or qsl[-1] != T or np.any(np.diff(qsl) < 0):
        raise ValueError("query_start_loc must rise from 0 to the row count")
    want = None if rows is None else np.zeros(T, dtype=bool)
    if want is not None:
        want[np.asarray(rows, dtype=np.int64)] = True
    out = np.full((T, Hq, D), np.nan) if want is not None else np.zeros((T, Hq, D))
    for b in range(B):
        r0, r1 = int(qsl[b]), int(qsl[b + 1])
        n, L = r1 - r0, int(seq_lens[b])
        sel = np.arange(r0, r1) if want is None else np.nonzero(want[r0:r1])[0] + r0
        if len(sel) == 0:
            continue
        pos = row_positions(n, L)[sel - r0]
        Kb = gather_tokens(key_cache, block_tables[b], L, block_size)
        Vb = gather_tokens(value_cache, block_tables[b], L, block_size)
        for kvh in range(Hkv):
            for h in range(kvh * g, (kvh + 1) * g):
                out[sel, h] = causal_attend(query[sel, h], Kb[:, kvh, :],
                                            Vb[:, kvh, :], pos, scale)
    return out


def paged_prefill_stored(query, key_cache, value_cache, kind: str,
                         k_scale: float, v_scale: float,
                         block_tables: np.ndarray, seq_lens: np.ndarray,
                         query_start_loc: np.ndarray, scale: float,
                         block_size: int,
                         rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """O5 on caches in their storage format (CPU torch tensors; fp8 as uint8
    codes).  Only the blocks the sequences use are decoded exactly to fp64
    (fp8: code value times the per-tensor scale) before `paged_prefill`."""
    import torch

    from .cache_write import to_f64

    q = query.to(torch.float64).numpy()
    B = len(seq_lens)
    used = sorted({int(block_tables[b][i]) for b in range(B)
                   for i in range(-(-int(seq_lens[b]) // block_size))})
    if used and (used[0] < 0 or used[-1] >= key_cache.shape[0]):
        raise IndexError("block table entry outside the physical pool")
    idx = torch.tensor(used, dtype=torch.int64)
    remap = np.full(key_cache.shape[0], -1, dtype=np.int64)
    remap[used] = np.arange(len(used))
    Kc = to_f64(key_cache[idx], kind, k_scale)
    Vc = to_f64(value_cache[idx], kind, v_scale)
    tables = np.asarray(block_tables, dtype=np.int64)
    local = np.where(tables >= 0, remap[np.clip(tables, 0, key_cache.shape[0] - 1)], -1)
    return paged_prefill(q, Kc, Vc, local, seq_lens, query_start_loc, scale,
                         block_size, rows=rows)
