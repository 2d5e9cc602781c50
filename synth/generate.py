"""Seeded synthetic workloads for paged decode attention.

Everything here is input drawing: lengths, a shuffled pool of physical
block ids, block tables, queries and a stream of K/V tokens together with the
cache slot each token belongs to.  The layout conventions are the pages':
a per-sequence table of physical block ids padded with -1, one row per
sequence (page "5.KV Cache 管理 & PagedAttention", question 8, batch
organisation of block tables), and K/V pools shaped
[num_blocks, block_size, num_kv_heads, head_dim] (page
"paged-attention-and-vllm-inference", code block `paged_attention`).

Draw order (one numpy Generator per workload): lengths -> permutation of the
pool -> Q -> K tokens -> V tokens.  Normals are drawn in float32 and rounded
to the storage dtype with torch's round-to-nearest-even casts.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from .configs import WorkloadConfig

TORCH_DTYPES = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
}

# Value written into every cache slot that no token owns, so that a kernel
# reading a slot it must not use shows up as NaN.  fp8 E4M3FN has no inf; its
# NaN code with the sign bit clear is 0x7F.
FP8_POISON = 0x7F


@dataclass
class Workload:
    cfg: WorkloadConfig
    seq_lens: np.ndarray          # [B] int32
    block_tables: np.ndarray      # [B, max_blocks] int32, -1 padded
    num_blocks: int               # physical pool size
    query: torch.Tensor           # [B, Hq, D] q dtype (CPU)
    tok_key: torch.Tensor         # [T, Hkv, D] source dtype (CPU)
    tok_value: torch.Tensor       # [T, Hkv, D]
    slot_mapping: np.ndarray      # [T] int64, unique slots
    new_slots: np.ndarray         # [B] int64: slot of each sequence's last token, -1 if shared
    new_tok: np.ndarray           # [B] int64: index into the token stream (or -1)
    shared_blocks: np.ndarray     # [n_shared] int32 physical ids of the shared prefix
    token_ids: List[np.ndarray]   # per sequence: its L_b token ids (int32); the
                                  # first min(L_b, prefix) are the shared prompt's
    prompt_rows: int              # stream rows 0 .. prompt_rows-1 hold the shared
                                  # prompt's K/V, position order (0 without one)
    private_row0: np.ndarray      # [B] int64: stream row of each sequence's
                                  # first token past the shared prompt
    pool_order: np.ndarray        # [N] int32: the seeded permutation the block
                                  # ids were handed out in (first id first)
    k_scale: float                # fp8 per-tensor scales (1.0 otherwise)
    v_scale: float
    scale: float                  # score scale 1/sqrt(head_dim), as float32

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def num_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])

    def new_key(self) -> torch.Tensor:
        return _gather_rows(self.tok_key, self.new_tok)

    def new_value(self) -> torch.Tensor:
        return _gather_rows(self.tok_value, self.new_tok)

    def position_rows(self, b: int, positions: np.ndarray) -> np.ndarray:
        """Stream rows holding the K/V of sequence b at `positions`: a shared
        prompt position reads the prompt's row (the same tokens after the
        same history have the same K/V), a later one the sequence's own."""
        pos = np.asarray(positions, dtype=np.int64)
        P = self.prompt_rows
        return np.where(pos < P, pos, self.private_row0[b] + (pos - P))

    def kv_bytes_per_elem(self) -> int:
        return {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}[self.cfg.kv_dtype]

    def logical_kv_bytes(self) -> int:
        """K+V bytes summed over every sequence's valid tokens."""
        c = self.cfg
        return int(self.seq_lens.astype(np.int64).sum()) * c.num_kv_heads * \
            c.head_dim * 2 * self.kv_bytes_per_elem()

    def unique_kv_bytes(self) -> int:
        """K+V bytes of distinct cache slots read (a shared prefix counts once)."""
        c = self.cfg
        return self.unique_token_slots() * c.num_kv_heads * c.head_dim * 2 * \
            self.kv_bytes_per_elem()

    def unique_token_slots(self) -> int:
        """Distinct (block, offset) slots read over the batch."""
        bs = self.cfg.block_size
        best = {}
        for b in range(self.cfg.batch):
            L = int(self.seq_lens[b])
            for i in range(-(-L // bs)):
                blk = int(self.block_tables[b, i])
                best[blk] = max(best.get(blk, 0), min(bs, L - i * bs))
        return sum(best.values())


def _gather_rows(t: torch.Tensor, idx: np.ndarray) -> torch.Tensor:
    out = torch.zeros((len(idx),) + tuple(t.shape[1:]), dtype=t.dtype)
    ok = idx >= 0
    if ok.any():
        out[torch.from_numpy(np.nonzero(ok)[0])] = t[torch.from_numpy(idx[ok])]
    return out


def _draw_lengths(cfg: WorkloadConfig, rng: np.random.Generator) -> np.ndarray:
    kind = cfg.lengths[0]
    if kind == "fixed":
        L = np.full(cfg.batch, int(cfg.lengths[1]), dtype=np.int64)
    elif kind == "uniform":
        lo, hi = int(cfg.lengths[1]), int(cfg.lengths[2])
        L = rng.integers(lo, hi + 1, size=cfg.batch, dtype=np.int64)
    elif kind == "lognormal":
        mu, sigma, lo, hi = cfg.lengths[1:]
        L = np.clip(np.rint(np.exp(rng.normal(mu, sigma, size=cfg.batch))),
                    lo, hi).astype(np.int64)
    elif kind == "list":
        L = np.asarray(cfg.lengths[1], dtype=np.int64)
        assert L.shape == (cfg.batch,)
    else:
        raise ValueError(f"unknown length recipe {cfg.lengths!r}")
    return L.astype(np.int32)


def _normals(rng: np.random.Generator, shape, dtype: str) -> torch.Tensor:
    x = rng.standard_normal(size=int(np.prod(shape)), dtype=np.float32)
    t = torch.from_numpy(x).reshape(shape)
    return t.to(TORCH_DTYPES[dtype])


def make_workload(cfg: WorkloadConfig, seed: Optional[int] = None) -> Workload:
    """Draw one workload.  Same (cfg, seed) -> same bits, on any machine."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, Hq, Hkv, D, bs = (cfg.batch, cfg.num_q_heads, cfg.num_kv_heads,
                         cfg.head_dim, cfg.block_size)
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")

    L = _draw_lengths(cfg, rng)
    need = [-(-int(x) // bs) for x in L]

    if cfg.shared_prefix_tokens % bs:
        raise ValueError("a shared prefix must fill whole blocks")
    n_shared = cfg.shared_prefix_tokens // bs
    P = cfg.shared_prefix_tokens
    # A sequence shares the prompt's blocks that it fills completely (all of
    # them when it is longer than the prompt): a prefix cache hands out whole
    # blocks only.  The rest of its blocks are its own; when it ends inside
    # the prompt, its last, partly filled block is a private block holding
    # the prompt's K/V at those positions.
    k_shared = [min(n_shared, int(x) // bs) if int(x) < P else n_shared for x in L]
    private_need = [n - k for n, k in zip(need, k_shared)]
    if cfg.pool_blocks:
        N = int(cfg.pool_blocks)
    else:
        N = n_shared + int(math.ceil(cfg.pool_factor * sum(private_need)))
    if N < n_shared + sum(private_need):
        raise ValueError("pool too small for the drawn lengths")
    perm = rng.permutation(N).astype(np.int32)

    # Hand out blocks in permutation order: shared prefix first, then each
    # sequence's private blocks.
    shared = perm[:n_shared]
    cursor = n_shared
    max_blocks = max(max(need), 1)
    tables = np.full((B, max_blocks), -1, dtype=np.int32)
    for b in range(B):
        k = k_shared[b]
        tables[b, :k] = shared[:k]
        tables[b, k:need[b]] = perm[cursor:cursor + private_need[b]]
        cursor += private_need[b]

    query = _normals(rng, (B, Hq, D), cfg.q_dtype)

    # Token stream: the whole shared prompt once, then every sequence's
    # tokens past it in position order; these rows are drawn.  After them
    # come copies of prompt rows for the private last blocks of sequences
    # that end inside the prompt.
    slots: List[np.ndarray] = []
    if n_shared:
        pos = np.arange(P, dtype=np.int64)
        slots.append(shared[pos // bs].astype(np.int64) * bs + pos % bs)
    new_tok = np.full(B, -1, dtype=np.int64)
    new_slots = np.full(B, -1, dtype=np.int64)
    private_row0 = np.zeros(B, dtype=np.int64)
    count = sum(len(s) for s in slots)
    for b in range(B):
        start = min(P, int(L[b]))
        pos = np.arange(start, int(L[b]), dtype=np.int64)
        s = tables[b, pos // bs].astype(np.int64) * bs + pos % bs
        slots.append(s)
        private_row0[b] = count
        if len(pos):
            new_tok[b] = count + len(pos) - 1
            new_slots[b] = s[-1]
        count += len(pos)
    T = count
    copy_src: List[np.ndarray] = []
    for b in range(B):
        if int(L[b]) < P and k_shared[b] < need[b]:
            pos = np.arange(k_shared[b] * bs, int(L[b]), dtype=np.int64)
            slots.append(tables[b, pos // bs].astype(np.int64) * bs + pos % bs)
            copy_src.append(pos)
            new_tok[b] = count + len(pos) - 1
            new_slots[b] = slots[-1][-1]
            count += len(pos)
    slot_mapping = np.concatenate(slots) if slots else np.zeros(0, np.int64)

    tok_key = _normals(rng, (T, Hkv, D), cfg.src_dtype)
    tok_value = _normals(rng, (T, Hkv, D), cfg.src_dtype)
    if copy_src:
        src = torch.from_numpy(np.concatenate(copy_src))
        tok_key = torch.cat([tok_key, tok_key[src]])
        tok_value = torch.cat([tok_value, tok_value[src]])

    # token ids (for the prefix cache), from a generator of their own so the
    # draws above do not move: the shared prompt's, then each sequence's own
    trng = np.random.default_rng([cfg.seed if seed is None else seed, 0x70C5])
    prompt_ids = trng.integers(1, 32000, size=P).astype(np.int32)
    token_ids = []
    for b in range(B):
        own = trng.integers(1, 32000, size=max(0, int(L[b]) - P)).astype(np.int32)
        token_ids.append(np.concatenate([prompt_ids[:min(P, int(L[b]))], own]))

    k_scale = v_scale = 1.0
    if cfg.kv_dtype == "fp8":
        # Per-tensor calibration: the largest magnitude maps to the largest
        # finite E4M3 value (448).
        k_scale = float(np.float32(tok_key.abs().max().float().item()) / np.float32(448.0))
        v_scale = float(np.float32(tok_value.abs().max().float().item()) / np.float32(448.0))

    scale = float(np.float32(1.0) / np.float32(math.sqrt(D)))
    return Workload(cfg=cfg, seq_lens=L, block_tables=tables, num_blocks=N,
                    query=query, tok_key=tok_key, tok_value=tok_value,
                    slot_mapping=slot_mapping, new_slots=new_slots,
                    new_tok=new_tok, shared_blocks=shared.copy(), token_ids=token_ids,
                    prompt_rows=P, private_row0=private_row0, pool_order=perm,
                    k_scale=k_scale, v_scale=v_scale, scale=scale)


def empty_cache_cpu(wl: Workload) -> torch.Tensor:
    """One poisoned pool [N, bs, Hkv, D] on the CPU (fp8 pools as uint8 codes)."""
    c = wl.cfg
    shape = (wl.num_blocks, c.block_size, c.num_kv_heads, c.head_dim)
    if c.kv_dtype == "fp8":
        return torch.full(shape, FP8_POISON, dtype=torch.uint8)
    return torch.full(shape, float("nan"), dtype=TORCH_DTYPES[c.kv_dtype])


@dataclass
class PrefillRows:
    """The packed query rows of one prefill call over a drawn workload."""
    new_tokens: np.ndarray        # [B] int32 rows per sequence
    query_start_loc: np.ndarray   # [B + 1] int32
    query: torch.Tensor           # [T, Hq, D] q dtype (CPU)

    @property
    def max_query_len(self) -> int:
        return int(self.new_tokens.max()) if len(self.new_tokens) else 0

    @property
    def num_rows(self) -> int:
        return int(self.query_start_loc[-1])


def make_prefill_rows(wl: Workload, new_tokens, seed: Optional[int] = None) -> PrefillRows:
    """Rows for a prefill call: n_b new tokens per sequence, by recipe
    ("all",) (the whole sequence) | ("fixed", n) (clipped to L_b) |
    ("list", [n_b ...]) (taken as given, may exceed L_b) | ("uniform", lo, hi)
    (clipped to L_b); queries are normals rounded to the query dtype.  Drawn
    from a generator of its own, so the workload's draws are unchanged."""
    c = wl.cfg
    rng = np.random.default_rng([c.seed if seed is None else seed, 0x70F1])
    L = wl.seq_lens.astype(np.int64)
    kind = new_tokens[0]
    if kind == "all":
        n = L.copy()
    elif kind == "fixed":
        n = np.minimum(L, int(new_tokens[1]))
    elif kind == "list":
        n = np.asarray(new_tokens[1], dtype=np.int64)
        assert n.shape == L.shape
    elif kind == "uniform":
        n = np.minimum(L, rng.integers(int(new_tokens[1]), int(new_tokens[2]) + 1, size=len(L)))
    else:
        raise ValueError(f"unknown new-token recipe {new_tokens!r}")
    qsl = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    q = _normals(rng, (int(qsl[-1]), c.num_q_heads, c.head_dim), c.q_dtype)
    return PrefillRows(new_tokens=n.astype(np.int32), query_start_loc=qsl, query=q)


def shrink(cfg: WorkloadConfig, **kw) -> WorkloadConfig:
    """A copy of a config with some fields replaced (for small test cases)."""
    return dataclasses.replace(cfg, **kw)
