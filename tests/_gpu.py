"""Shared GPU-test plumbing: put a synthetic workload on the device, fill the
cache through the library, and produce the oracle's answer for the same
inputs.  Imported only by tests marked `gpu`."""

from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

import paged_kv_cache_462_amd as pa
from oracle import attention as OA
from oracle import cache_write as OW
from oracle import prefill as OP
from synth.generate import PrefillRows, Workload, empty_cache_cpu

# Tolerances: |gpu - oracle| <= atol + rtol * |oracle|, elementwise.
# 16-bit data and outputs: atol 2e-3, rtol 1e-2; fp8 KV: atol 5e-2, rtol 1e-2.
# fp32 (VALU path, fp32 throughout, hardware exp2 within 1 ulp over at most a
# few thousand tokens): atol 2e-5, rtol 1e-4.
TOL = {"f32": (2e-5, 1e-4), "f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2), "fp8": (5e-2, 1e-2)}


def tol_for(wl: Workload) -> Tuple[float, float]:
    c = wl.cfg
    return TOL["fp8"] if c.kv_dtype == "fp8" else TOL[c.q_dtype]


def say(*a):
    """Name the case being run, flushed before the GPU step."""
    print(*a, flush=True)
    sys.stdout.flush()


@dataclass
class Dev:
    query: torch.Tensor
    tables: torch.Tensor
    lens: torch.Tensor
    slots: torch.Tensor
    tok_key: torch.Tensor
    tok_value: torch.Tensor
    kc: torch.Tensor
    vc: torch.Tensor


def kv_store_dtype(wl: Workload):
    return torch.uint8 if wl.cfg.kv_dtype == "fp8" else wl.tok_key.dtype


def check_shapes(wl: Workload) -> None:
    """Host-side sanity before any launch: ids and lengths fit the pool."""
    c = wl.cfg
    assert wl.block_tables.shape == (c.batch, wl.max_blocks)
    assert (wl.seq_lens >= 0).all() and (wl.seq_lens <= wl.max_blocks * c.block_size).all()
    for b in range(c.batch):
        nb = -(-int(wl.seq_lens[b]) // c.block_size)
        row = wl.block_tables[b, :nb]
        assert (row >= 0).all() and (row < wl.num_blocks).all()
    if wl.num_tokens:
        assert wl.slot_mapping.max() < wl.num_blocks * c.block_size
        assert len(np.unique(wl.slot_mapping)) == wl.num_tokens


def to_device(wl: Workload, fill: bool = True) -> Dev:
    check_shapes(wl)
    dev = torch.device("cuda:0")
    c = wl.cfg
    shape = (wl.num_blocks, c.block_size, c.num_kv_heads, c.head_dim)
    st = kv_store_dtype(wl)
    if c.kv_dtype == "fp8":
        kc = torch.full(shape, 0x7F, dtype=st, device=dev)
    else:
        kc = torch.full(shape, float("nan"), dtype=st, device=dev)
    vc = kc.clone()
    d = Dev(query=wl.query.to(dev), tables=torch.from_numpy(wl.block_tables).to(dev),
            lens=torch.from_numpy(wl.seq_lens).to(dev),
            slots=torch.from_numpy(wl.slot_mapping).to(dev),
            tok_key=wl.tok_key.to(dev), tok_value=wl.tok_value.to(dev), kc=kc, vc=vc)
    if fill:
        gpu_write(wl, d)
    return d


def gpu_write(wl: Workload, d: Dev) -> None:
    pa.reshape_and_cache(d.tok_key, d.tok_value, d.slots, d.kc, d.vc,
                         k_scale=wl.k_scale, v_scale=wl.v_scale,
                         kv_dtype="fp8" if wl.cfg.kv_dtype == "fp8" else None)


def oracle_caches(wl: Workload):
    kc, vc = empty_cache_cpu(wl), empty_cache_cpu(wl)
    OW.reshape_and_cache(wl.tok_key, wl.tok_value, wl.slot_mapping, kc, vc,
                         wl.cfg.kv_dtype, wl.k_scale, wl.v_scale)
    return kc, vc


def gpu_decode(wl: Workload, d: Dev, partition_tokens: int = 0, path: int = 0,
               out: Optional[torch.Tensor] = None,
               error_flags: Optional[torch.Tensor] = None) -> torch.Tensor:
    c = wl.cfg
    if out is None:
        out = torch.empty_like(d.query)
    pa.decode(out, d.query, d.kc, d.vc, d.tables, d.lens, wl.scale, c.block_size,
              c.num_kv_heads, k_scale=wl.k_scale, v_scale=wl.v_scale,
              kv_dtype="fp8" if c.kv_dtype == "fp8" else None,
              partition_tokens=partition_tokens, path=path, error_flags=error_flags)
    return out


def oracle_decode(wl: Workload, kc, vc, pairs: Optional[Sequence] = None) -> np.ndarray:
    return OA.paged_decode_stored(wl.query, kc, vc, wl.cfg.kv_dtype, wl.k_scale, wl.v_scale,
                                  wl.block_tables, wl.seq_lens, wl.scale, wl.cfg.block_size,
                                  pairs)


def gpu_prefill(wl: Workload, d: Dev, rows: PrefillRows, max_query_len: Optional[int] = None,
                out: Optional[torch.Tensor] = None, qsl: Optional[torch.Tensor] = None,
                error_flags: Optional[torch.Tensor] = None) -> torch.Tensor:
    c = wl.cfg
    dev = d.kc.device
    q = rows.query.to(dev)
    if qsl is None:
        qsl = torch.from_numpy(rows.query_start_loc).to(dev)
    if out is None:
        out = torch.empty_like(q)
    mq = rows.max_query_len if max_query_len is None else max_query_len
    pa.prefill(out, q, d.kc, d.vc, d.tables, d.lens, qsl, mq, wl.scale, c.block_size,
               c.num_kv_heads, k_scale=wl.k_scale, v_scale=wl.v_scale,
               kv_dtype="fp8" if c.kv_dtype == "fp8" else None, error_flags=error_flags)
    return out


def oracle_prefill(wl: Workload, kc, vc, rows: PrefillRows,
                   subset: Optional[Sequence[int]] = None) -> np.ndarray:
    return OP.paged_prefill_stored(rows.query, kc, vc, wl.cfg.kv_dtype, wl.k_scale, wl.v_scale,
                                   wl.block_tables, wl.seq_lens, rows.query_start_loc,
                                   wl.scale, wl.cfg.block_size, rows=subset)


def sample_rows(rows: PrefillRows, n: int, seed: int = 0) -> List[int]:
    """Packed rows to check at full size: the first and last row of every
    sequence, the rows at tile boundaries of the first one, and random ones."""
    rng = np.random.default_rng(seed)
    qsl = rows.query_start_loc
    pick = set()
    for b in range(len(qsl) - 1):
        if qsl[b + 1] > qsl[b]:
            pick.update({int(qsl[b]), int(qsl[b + 1]) - 1})
    for r in (255, 256, 257, 511, 512):
        if r < qsl[1]:
            pick.add(r)
    while len(pick) < min(n, rows.num_rows):
        pick.add(int(rng.integers(rows.num_rows)))
    return sorted(pick)


def assert_close(got: torch.Tensor, ref: np.ndarray, atol: float, rtol: float,
                 pairs: Optional[Sequence] = None, what: str = "") -> Dict[str, float]:
    g = got.detach().to("cpu", torch.float64).numpy()
    if pairs is not None:
        idx = tuple(np.array(pairs).T)
        g, ref = g[idx], ref[idx]
    err = np.abs(g - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first at {tuple(i)}: "
            f"gpu={g[tuple(i)]!r} oracle={ref[tuple(i)]!r} (max err {err.max():.3e})")
    return {"max_abs": float(err.max()) if err.size else 0.0}


def sample_pairs(wl: Workload, n: int, seed: int = 0) -> List[Tuple[int, int]]:
    """Query rows to check at full size: the first and last sequence, the
    shortest and the longest, plus random ones, over random heads."""
    c = wl.cfg
    rng = np.random.default_rng(seed)
    bs = {0, c.batch - 1, int(np.argmin(wl.seq_lens)), int(np.argmax(wl.seq_lens))}
    pairs = set()
    for b in bs:
        pairs.add((b, 0))
        pairs.add((b, c.num_q_heads - 1))
    while len(pairs) < n:
        pairs.add((int(rng.integers(c.batch)), int(rng.integers(c.num_q_heads))))
    return sorted(pairs)


def caches_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Bitwise equality (NaN payloads included)."""
    iv = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[a.element_size()]
    return bool(torch.equal(a.cpu().view(iv), b.cpu().view(iv)))


# --- shared-prompt batches built through the host chain ------------------------

@dataclass
class Chain:
    alloc: object
    manager: object
    cache: object
    batch: object
    slots: np.ndarray     # [T'] int64: every K/V slot the batch writes
    rows: np.ndarray      # [T'] int64: the stream row written there


def admit_chain(wl: Workload) -> Chain:
    """The workload's tables through the library's allocator (handing out
    ids in the workload's seeded order), block manager and prefix cache:
    the shared prompt first, then every request, then the prompt's own
    sequence released."""
    c = wl.cfg
    P = c.shared_prefix_tokens
    alloc = pa.BlockAllocator(wl.num_blocks, wl.pool_order[::-1])
    mgr = pa.BlockManager(alloc, c.block_size)
    cache = pa.PrefixCache(alloc, c.block_size)
    prompt = wl.token_ids[int(np.argmax(wl.seq_lens))][:P]
    batch = pa.admit_with_shared_prompt(mgr, cache, prompt, wl.token_ids, wl.max_blocks)
    slots, rows = [], []
    for i, first, s in batch.writes:
        pos = np.arange(first, first + len(s))
        rows.append(pos if i < 0 else wl.position_rows(i, pos))
        slots.append(s)
    return Chain(alloc, mgr, cache, batch, np.concatenate(slots), np.concatenate(rows))


def chain_to_device(wl: Workload, ch: Chain) -> Dev:
    """Device buffers of the chain's batch: tables and lengths from the
    block manager, the cache filled by pa_reshape_and_cache at the chain's
    slots (pool poisoned elsewhere)."""
    c = wl.cfg
    tables, lens = ch.batch.tables, ch.batch.seq_lens
    assert tables.shape == (c.batch, wl.max_blocks)
    for b in range(c.batch):
        nb = -(-int(lens[b]) // c.block_size)
        assert (tables[b, :nb] >= 0).all() and (tables[b, :nb] < wl.num_blocks).all()
    assert len(np.unique(ch.slots)) == len(ch.slots)
    assert ch.slots.max() < wl.num_blocks * c.block_size
    dev = torch.device("cuda:0")
    shape = (wl.num_blocks, c.block_size, c.num_kv_heads, c.head_dim)
    st = kv_store_dtype(wl)
    fill = 0x7F if c.kv_dtype == "fp8" else float("nan")
    kc = torch.full(shape, fill, dtype=st, device=dev)
    vc = kc.clone()
    ri = torch.from_numpy(ch.rows)
    d = Dev(query=wl.query.to(dev), tables=torch.from_numpy(tables).to(dev),
            lens=torch.from_numpy(lens).to(dev), slots=torch.from_numpy(ch.slots).to(dev),
            tok_key=wl.tok_key[ri].to(dev), tok_value=wl.tok_value[ri].to(dev), kc=kc, vc=vc)
    gpu_write(wl, d)
    return d


def chain_oracle_caches(wl: Workload, ch: Chain):
    kc, vc = empty_cache_cpu(wl), empty_cache_cpu(wl)
    ri = torch.from_numpy(ch.rows)
    OW.reshape_and_cache(wl.tok_key[ri], wl.tok_value[ri], ch.slots, kc, vc,
                         wl.cfg.kv_dtype, wl.k_scale, wl.v_scale)
    return kc, vc


def chain_oracle_decode(wl: Workload, ch: Chain, kc, vc) -> np.ndarray:
    return OA.paged_decode_stored(wl.query, kc, vc, wl.cfg.kv_dtype, wl.k_scale, wl.v_scale,
                                  ch.batch.tables, ch.batch.seq_lens, wl.scale,
                                  wl.cfg.block_size)


# error summaries of the full-size checks, printed at the end of the session
# (tests/conftest.py) so that they show however pytest captures output
SUMMARY: List[str] = []


def err_summary(got, ref: np.ndarray, atol: float, rtol: float, what: str) -> None:
    g = got.detach().to("cpu", torch.float64).numpy() if isinstance(got, torch.Tensor) else got
    err = np.abs(g - ref)
    big = np.abs(ref) > 1e-2
    rel = f"{(err[big] / np.abs(ref[big])).max():.2e}" if big.any() else "-"
    line = (f"{what}: {err.size} outputs, max abs err {err.max():.2e}, max rel err "
            f"(|ref| > 0.01) {rel}, max err / bound {(err / (atol + rtol * np.abs(ref))).max():.3f}")
    SUMMARY.append(line)
    say(line)
