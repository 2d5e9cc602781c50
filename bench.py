#!/usr/bin/env python3
"""Paged decode attention benchmark on one MI355X.

One step = the whole decode hot path over one batch: write each sequence's
new K/V token into its cache slot (pa_reshape_and_cache), then single-query
attention of every query head over its sequence's paged K/V
(pa_decode: partition kernel, plus the merge kernel when the plan splits).
Inputs are synthetic and seeded (synth/), resident in HBM before timing.
By default the headline is the 70B-shaped GQA decode (64 sequences of 4096
tokens, 1 GiB of KV per call), with the 7B-shaped decode under "also".
Batches whose sequences share a prompt take their block tables from the
host allocator and prefix cache.

Like the layers of a model, consecutive steps use different copies of the
KV pool (enough copies that together they are several times the 256 MB
last-level cache), so no step reads K/V that an earlier step left in cache.
A back-to-back run on a single copy is reported beside it for context.

Prints ONE JSON line:
  value           KV GB/s over the whole timed step (algorithmic KV bytes of
                  the batch / step time)
  roofline        the decode call measured with HIP events (created without
                  the system-scope fence, so recording them does not flush
                  the caches between the timed launches) on the launch
                  stream, --timed-launches calls after the timed steps:
                  algorithmic KV bytes per launch / mean duration,
                  against the 8 TB/s HBM peak; `traffic` from the committed
                  rocprofv3 FETCH_SIZE/WRITE_SIZE summary when it was taken
                  from the current kernel source, else null
  cache_write     pa_reshape_and_cache timed on its own after the steps:
                  the step's new token per sequence, and a bulk write of
                  every token of the batch (GB/s over bytes read + written)
  cpu_baseline    the CPU oracle (fp64) on a bounded sample of the same
                  batch, on this host's cores, for context only
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "paged decode attention: achieved KV HBM GB/s (% of peak) and tokens/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


DECODE_SOURCES = ("pa_decode.hip", "pa_device.h", "pa_internal.h")
PREFILL_SOURCES = ("pa_prefill.hip", "pa_prefill.h", "pa_device.h", "pa_internal.h")


def kernel_source_hash(files=DECODE_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "paged_kv_cache_462_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, launch_desc: str, kernel: str = "pa_decode",
                 files=DECODE_SOURCES):
    """HBM bytes per launch from the committed counter summary
    (profiles/<kernel>_<workload>_traffic.txt, `key: value` lines), if it was
    taken on the current kernel source and launch plan."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    t = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            t[k.strip()] = v.strip()
    if t.get("kernel_source_sha") != kernel_source_hash(files) or t.get("launch") != launch_desc:
        return None
    return {"hbm_bytes_per_launch": int(t["hbm_bytes_per_launch"])}


class HipTimingEvents:
    """HIP events for timing launches on a stream, created with
    hipEventDisableSystemFence: recording one then skips the system-scope
    fence (cache write-back and invalidate) that a default event performs,
    which otherwise stalls and slows the work that follows it.  They are
    used only for elapsed times, never to synchronise with the work."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def create(self):
        ev = self.ct.c_void_p()
        self._check(self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE),
                    "hipEventCreateWithFlags")
        self.events.append(ev)
        return ev

    def record(self, ev, stream):
        self._check(self.hip.hipEventRecord(ev, self.ct.c_void_p(stream.cuda_stream)), "hipEventRecord")

    def elapsed_ms(self, a, b) -> float:
        self._check(self.hip.hipEventSynchronize(b), "hipEventSynchronize")
        ms = self.ct.c_float()
        self._check(self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b), "hipEventElapsedTime")
        return float(ms.value)

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []


def host_threads() -> dict:
    """The host cores this process may run on, and the threads the oracle's
    BLAS and torch's CPU ops use on them."""
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        pass
    import torch
    return {"cores": len(os.sched_getaffinity(0)), "blas_threads": blas,
            "torch_threads": torch.get_num_threads()}


def cpu_baseline(wl, seconds: float):
    """The oracle, unchanged, over the sequences of the batch in order (from
    the first again after the last) until the time budget is spent."""
    import numpy as np

    from oracle import attention as OA
    from oracle import cache_write as OW
    from synth.generate import empty_cache_cpu

    kc, vc = empty_cache_cpu(wl), empty_cache_cpu(wl)
    OW.reshape_and_cache(wl.tok_key, wl.tok_value, wl.slot_mapping, kc, vc,
                         wl.cfg.kv_dtype, wl.k_scale, wl.v_scale)
    c = wl.cfg
    done, t_used, kv_bytes = 0, 0.0, 0
    esz = wl.kv_bytes_per_elem()
    while True:
        b = done % c.batch
        pairs = [(b, h) for h in range(c.num_q_heads)]
        t0 = time.perf_counter()
        OA.paged_decode_stored(wl.query, kc, vc, c.kv_dtype, wl.k_scale, wl.v_scale,
                               wl.block_tables, wl.seq_lens, wl.scale, c.block_size, pairs)
        t_used += time.perf_counter() - t0
        done += 1
        kv_bytes += int(wl.seq_lens[b]) * c.num_kv_heads * c.head_dim * 2 * esz
        if t_used >= seconds:
            break
    return {
        "value": round(kv_bytes / t_used / 1e9, 4),
        "unit": "GB/s",
        **host_threads(),
        "kind": "oracle",
        "sample": f"fp64 oracle decode of {done} sequences ({done / c.batch:.1f} passes over the "
                  f"batch of {c.batch}, all {c.num_q_heads} query heads, {kv_bytes / 1e6:.1f} MB "
                  f"of KV) in {t_used:.2f} s; tokens/s {done / t_used:.2f}",
    }


HOST_LINK_PEAK_GBPS = 64.0  # PCIe 5.0 x16, one direction


def bench_swap(args) -> int:
    """Every KV block of the workload's batch swapped out to a pinned host
    pool and back in, each direction timed with HIP events on the launch
    stream; bytes = K and V of the blocks moved, against the host link."""
    import numpy as np
    import torch

    import paged_kv_cache_462_amd as pa
    from synth import get_config, make_workload

    cfg = get_config(args.config)
    wl = make_workload(cfg)
    c = wl.cfg
    dev = torch.device("cuda:0")
    fp8 = c.kv_dtype == "fp8"
    st = torch.uint8 if fp8 else wl.tok_key.dtype
    shape = (wl.num_blocks, c.block_size, c.num_kv_heads, c.head_dim)
    kc = torch.zeros(shape, dtype=st, device=dev)
    vc = torch.zeros(shape, dtype=st, device=dev)
    pa.reshape_and_cache(wl.tok_key.to(dev), wl.tok_value.to(dev),
                         torch.from_numpy(wl.slot_mapping).to(dev), kc, vc,
                         k_scale=wl.k_scale, v_scale=wl.v_scale, kv_dtype="fp8" if fp8 else None)
    used = np.unique(wl.block_tables[wl.block_tables >= 0])
    n = len(used)
    hk = torch.empty((n,) + shape[1:], dtype=st).pin_memory()
    hv = torch.empty((n,) + shape[1:], dtype=st).pin_memory()
    out_pairs = torch.from_numpy(np.stack([used, np.arange(n)], 1).astype(np.int32)).to(dev)
    in_pairs = torch.from_numpy(np.stack([np.arange(n), used], 1).astype(np.int32)).to(dev)
    kind = "fp8" if fp8 else None
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        pa.swap_blocks(hk, hv, kc, vc, out_pairs, kv_dtype=kind)
        pa.swap_blocks(kc, vc, hk, hv, in_pairs, kv_dtype=kind)
    torch.cuda.synchronize()
    t_out, t_in = [], []
    K = args.steps
    t0 = time.perf_counter()
    for _ in range(K):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        pa.swap_blocks(hk, hv, kc, vc, out_pairs, kv_dtype=kind)
        e[1].record(stream)
        pa.swap_blocks(kc, vc, hk, hv, in_pairs, kv_dtype=kind)
        e[2].record(stream)
        e[2].synchronize()
        t_out.append(e[0].elapsed_time(e[1]))
        t_in.append(e[1].elapsed_time(e[2]))
    t1 = time.perf_counter()
    nbytes = 2 * n * int(np.prod(shape[1:])) * kc.element_size()
    out_gbps = nbytes / (float(np.mean(t_out)) * 1e-3) / 1e9
    in_gbps = nbytes / (float(np.mean(t_in)) * 1e-3) / 1e9
    ms_step = (t1 - t0) * 1e3 / K
    res = {
        "metric": "KV block swap: device -> pinned host and back (GB/s per direction)",
        "value": round(2 * nbytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.kv_dtype,
        "data": "synthetic",
        "config": {"workload": c.name, "blocks": int(n), "bytes_per_direction": int(nbytes)},
        "swap_out_GBps": round(out_gbps, 2),
        "swap_in_GBps": round(in_gbps, 2),
        "roofline": {"bound": "host-link", "achieved": round(min(out_gbps, in_gbps), 2),
                     "peak": HOST_LINK_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(min(out_gbps, in_gbps) / HOST_LINK_PEAK_GBPS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)
    return 0


MFMA_PEAK_TFLOPS = 2500.0  # dense f16 / bf16 matrix cores


def prefill_flops(rows, seq_lens, Hq: int, D: int) -> int:
    """Algorithmic flops of causal prefill: per query row and head, q.k over
    the pos + 1 keys it sees (2 D flops each) and p.v over the same keys
    (2 D each); masked-out keys count nothing."""
    import numpy as np

    total = 0
    qsl = rows.query_start_loc
    for b in range(len(seq_lens)):
        n, L = int(qsl[b + 1] - qsl[b]), int(seq_lens[b])
        pos = np.arange(n, dtype=np.int64) + (L - n)
        total += int(np.maximum(pos + 1, 0).sum())
    return 4 * D * Hq * total


def cpu_baseline_prefill(wl, rows, seconds: float):
    """The prefill oracle, unchanged, on evenly spaced rows of the first
    sequence (all query heads), the row count grown until the time budget
    is spent."""
    import numpy as np
    import torch

    from oracle import cache_write as OW
    from oracle import prefill as OP
    from synth.generate import empty_cache_cpu

    kc, vc = empty_cache_cpu(wl), empty_cache_cpu(wl)
    OW.reshape_and_cache(wl.tok_key, wl.tok_value, wl.slot_mapping, kc, vc,
                         wl.cfg.kv_dtype, wl.k_scale, wl.v_scale)
    c = wl.cfg
    n0 = int(rows.query_start_loc[1])
    L0 = int(wl.seq_lens[0])
    q0 = rows.query[:n0]
    count, used, flops = 16, 0.0, 0
    while True:
        sel = np.unique(np.linspace(0, n0 - 1, min(count, n0)).astype(np.int64))
        t0 = time.perf_counter()
        OP.paged_prefill_stored(q0, kc, vc, c.kv_dtype, wl.k_scale, wl.v_scale,
                                wl.block_tables[:1], wl.seq_lens[:1], np.array([0, n0]),
                                wl.scale, c.block_size, rows=sel)
        used = time.perf_counter() - t0
        pos = sel + (L0 - n0)
        flops = 4 * c.head_dim * c.num_q_heads * int((pos + 1).sum())
        if used >= seconds / 3 or len(sel) >= n0:
            break
        count *= 4
    return {
        "value": round(flops / used / 1e12, 6),
        "unit": "TFLOP/s",
        **host_threads(),
        "kind": "oracle",
        "sample": f"fp64 prefill oracle on {len(sel)} evenly spaced rows of sequence 0 "
                  f"({n0} rows, {L0} tokens), all {c.num_q_heads} query heads, "
                  f"{flops / 1e9:.2f} GFLOP in {used:.2f} s",
    }


def bench_prefill(args) -> int:
    """One step = write the new tokens' K/V into the cache
    (pa_reshape_and_cache) and take causal attention of their query rows
    over the cache (pa_prefill).  The prefill launch is timed with HIP
    events on the launch stream; its algorithmic flops against the dense
    16-bit MFMA peak."""
    import numpy as np
    import torch

    import paged_kv_cache_462_amd as pa
    from synth import get_prefill_config, make_prefill_rows, make_workload

    name = args.config if not args.config.startswith("c") else "p1"
    cfg, news = get_prefill_config(name)
    log(f"[bench] generating {cfg.name}")
    wl = make_workload(cfg)
    rows = make_prefill_rows(wl, news)
    c = wl.cfg
    dev = torch.device("cuda:0")
    fp8 = c.kv_dtype == "fp8"
    kvd = "fp8" if fp8 else None
    shape = (wl.num_blocks, c.block_size, c.num_kv_heads, c.head_dim)
    st = torch.uint8 if fp8 else wl.tok_key.dtype
    kc = torch.zeros(shape, dtype=st, device=dev)
    vc = torch.zeros(shape, dtype=st, device=dev)
    tables = torch.from_numpy(wl.block_tables).to(dev)
    lens = torch.from_numpy(wl.seq_lens).to(dev)
    qsl = torch.from_numpy(rows.query_start_loc).to(dev)
    q = rows.query.to(dev)
    out = torch.empty_like(q)
    # the new tokens' K/V: the last n_b of each sequence in the token stream
    starts = np.concatenate([[0], np.cumsum(wl.seq_lens.astype(np.int64))])
    if cfg.shared_prefix_tokens:
        raise SystemExit("prefill workloads take no shared prefix")
    new_idx = np.concatenate([np.arange(starts[b + 1] - rows.new_tokens[b], starts[b + 1])
                              for b in range(c.batch)]).astype(np.int64)
    tok_k = wl.tok_key.to(dev)
    tok_v = wl.tok_value.to(dev)
    slots = torch.from_numpy(wl.slot_mapping).to(dev)
    pa.reshape_and_cache(tok_k, tok_v, slots, kc, vc, k_scale=wl.k_scale, v_scale=wl.v_scale,
                         kv_dtype=kvd)
    ni = torch.from_numpy(new_idx).to(dev)
    new_k, new_v, new_s = tok_k[ni].contiguous(), tok_v[ni].contiguous(), slots[ni].contiguous()
    del tok_k, tok_v
    # calibration copy for the FETCH_SIZE / WRITE_SIZE counters
    cal_src = torch.ones(1 << 26, dtype=torch.float32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    del cal_src, cal_dst
    # max_query_len sizes the grid (query-tile ranks); a smaller value makes
    # each workgroup walk several row tiles of its (sequence, head)
    mq = args.max_query_len if args.max_query_len > 0 else rows.max_query_len
    stream = torch.cuda.current_stream()

    def step_write():
        pa.reshape_and_cache(new_k, new_v, new_s, kc, vc, k_scale=wl.k_scale,
                             v_scale=wl.v_scale, kv_dtype=kvd)

    def step_attn():
        pa.prefill(out, q, kc, vc, tables, lens, qsl, mq, wl.scale, c.block_size,
                   c.num_kv_heads, k_scale=wl.k_scale, v_scale=wl.v_scale, kv_dtype=kvd)

    for _ in range(args.warmup):
        step_write()
        step_attn()
    torch.cuda.synchronize()
    K = args.steps
    timer = HipTimingEvents()
    sampled = list(range(0, K, max(1, args.time_every)))
    evs = {i: (timer.create(), timer.create()) for i in sampled}
    log(f"[bench] timing {K} prefill steps ({len(sampled)} launches event-timed)")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step_write()
        ev = evs.get(i)
        if ev:
            timer.record(ev[0], stream)
        step_attn()
        if ev:
            timer.record(ev[1], stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    att_ms = [timer.elapsed_ms(a, b) for a, b in evs.values()]
    timer.close()
    att_mean = float(np.mean(att_ms))
    flops = prefill_flops(rows, wl.seq_lens, c.num_q_heads, c.head_dim)
    achieved = flops / (att_mean * 1e-3) / 1e12
    # algorithmic bytes: the query rows and outputs once, every sequence's
    # cached K/V once
    qo_bytes = 2 * rows.num_rows * c.num_q_heads * c.head_dim * q.element_size()
    alg_bytes = qo_bytes + wl.logical_kv_bytes()
    traffic = load_traffic(c.name, "default", "pa_prefill", PREFILL_SOURCES)
    res = {
        "metric": "paged causal prefill attention: TFLOP/s (algorithmic, unmasked part) and tokens/s",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.q_dtype,
        "data": "synthetic",
        "config": {
            "workload": c.name,
            "batch": c.batch,
            "num_q_heads": c.num_q_heads,
            "num_kv_heads": c.num_kv_heads,
            "head_dim": c.head_dim,
            "block_size": c.block_size,
            "seq_lens": list(map(str, c.lengths)),
            "new_tokens": list(map(str, news)),
            "query_rows": rows.num_rows,
            "max_query_len_arg": mq,
            "q_dtype": c.q_dtype,
            "kv_dtype": c.kv_dtype,
            "flops_per_step": flops,
            "parallelism": "single GPU",
        },
        "tokens_per_s": round(rows.num_rows / (ms_step * 1e-3), 1),
        "roofline": {
            "bound": "mfma",
            "kernel": "pa_prefill",
            "achieved": round(achieved, 1),
            "peak": MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
            "traffic": (traffic["hbm_bytes_per_launch"] if traffic else None),
            "algorithmic_flops_per_launch": flops,
            "algorithmic_bytes_per_launch": alg_bytes,
            "mean_launch_ms": round(att_mean, 5),
            "median_launch_ms": round(float(np.median(att_ms)), 5),
            "event_timed_launches": len(att_ms),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (~{args.cpu_seconds}s)")
        res["cpu_baseline"] = cpu_baseline_prefill(wl, rows, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


def chain_tables(wl):
    """A shared-prompt workload's tables and K/V slots built through the
    host chain (the library's allocator handing out ids in the workload's
    seeded order, the prompt admitted and cached, every request admitted
    through the prefix cache, the prompt's own sequence released).  They
    must equal the seeded layout; returns (tables, seq_lens, slots, rows,
    prompt_blocks)."""
    import numpy as np

    import paged_kv_cache_462_amd as pa

    c = wl.cfg
    alloc = pa.BlockAllocator(wl.num_blocks, wl.pool_order[::-1])
    mgr = pa.BlockManager(alloc, c.block_size)
    cache = pa.PrefixCache(alloc, c.block_size)
    P = c.shared_prefix_tokens
    prompt = wl.token_ids[int(np.argmax(wl.seq_lens))][:P]
    batch = pa.admit_with_shared_prompt(mgr, cache, prompt, wl.token_ids, wl.max_blocks)
    if not (np.array_equal(batch.tables, wl.block_tables)
            and np.array_equal(batch.seq_lens, wl.seq_lens)):
        raise SystemExit("the host chain's tables differ from the seeded layout")
    slots, rows = [], []
    for i, first, sl in batch.writes:
        pos = np.arange(first, first + len(sl))
        rows.append(pos if i < 0 else wl.position_rows(i, pos))
        slots.append(sl)
    return (batch.tables, batch.seq_lens, np.concatenate(slots), np.concatenate(rows),
            batch.prompt_blocks)


def run_decode(name: str, args, cpu_seconds: float) -> dict:
    """One decode workload: the timed steps, the event-timed launches, the
    cache-write timings and (cpu_seconds > 0) the oracle on the host."""
    import numpy as np
    import torch

    import paged_kv_cache_462_amd as pa
    from synth import get_config, make_workload

    cfg = get_config(name)
    log(f"[bench] generating {cfg.name}")
    wl = make_workload(cfg)
    dev = torch.device("cuda:0")
    c = wl.cfg
    fp8 = c.kv_dtype == "fp8"
    kvd = "fp8" if fp8 else None
    shape = (wl.num_blocks, c.block_size, c.num_kv_heads, c.head_dim)
    st = torch.uint8 if fp8 else wl.tok_key.dtype
    kc = torch.zeros(shape, dtype=st, device=dev)
    vc = torch.zeros(shape, dtype=st, device=dev)
    q = wl.query.to(dev)
    source = "seeded layout"
    if c.shared_prefix_tokens:
        # shared-prompt batches come out of the allocator and prefix cache
        tab_np, lens_np, slots_np, rows_np, prompt_blocks_np = chain_tables(wl)
        ri = torch.from_numpy(rows_np)
        fill_k, fill_v = wl.tok_key[ri], wl.tok_value[ri]
        source = "host allocator + prefix cache"
    else:
        tab_np, lens_np, slots_np = wl.block_tables, wl.seq_lens, wl.slot_mapping
        fill_k, fill_v = wl.tok_key, wl.tok_value
        prompt_blocks_np = wl.shared_blocks
    tables = torch.from_numpy(tab_np).to(dev)
    lens = torch.from_numpy(lens_np).to(dev)
    # fill the cache once (set-up, untimed)
    pa.reshape_and_cache(fill_k.to(dev), fill_v.to(dev), torch.from_numpy(slots_np).to(dev),
                         kc, vc, k_scale=wl.k_scale, v_scale=wl.v_scale, kv_dtype=kvd)
    pool_bytes = 2 * kc.numel() * kc.element_size()
    n_layers = args.layers or max(1, -(-(3 << 30) // pool_bytes))
    layers = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(n_layers - 1)]
    # a plain copy of known size (256 MiB read + 256 MiB written): the
    # calibration kernel for the FETCH_SIZE / WRITE_SIZE counters
    cal_src = torch.ones(1 << 26, dtype=torch.float32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    del cal_src, cal_dst
    new_k = wl.new_key().to(dev)
    new_v = wl.new_value().to(dev)
    new_slots = torch.from_numpy(wl.new_slots).to(dev)
    out = torch.empty_like(q)
    shared = args.shared_prefix
    if shared and not c.shared_prefix_tokens:
        raise SystemExit(f"{c.name} has no shared prefix")
    if shared:
        ws_bytes = pa.decode_shared_prefix_workspace_bytes(
            c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim, c.block_size, wl.max_blocks,
            c.shared_prefix_tokens)
        prefix_blocks = torch.from_numpy(prompt_blocks_np.astype(np.int32)).to(dev)
    else:
        ws_bytes = pa.decode_workspace_bytes(c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                             c.block_size, wl.max_blocks, args.partition_tokens)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    plan = pa.decode_plan(c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim,
                          c.block_size, wl.max_blocks, args.partition_tokens)
    if shared:
        plan["schedule"] = "balanced+shared-prefix"
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def decode(layer):
        k_, v_ = layers[layer]
        if shared:
            pa.decode_shared_prefix(out, q, k_, v_, tables, lens, prefix_blocks,
                                    c.shared_prefix_tokens, wl.scale, c.block_size,
                                    c.num_kv_heads, k_scale=wl.k_scale, v_scale=wl.v_scale,
                                    kv_dtype=kvd, workspace=ws)
        else:
            pa.decode(out, q, k_, v_, tables, lens, wl.scale, c.block_size, c.num_kv_heads,
                      k_scale=wl.k_scale, v_scale=wl.v_scale, kv_dtype=kvd, workspace=ws,
                      partition_tokens=args.partition_tokens, path=args.path)

    def write(layer):
        k_, v_ = layers[layer]
        pa.reshape_and_cache(new_k, new_v, new_slots, k_, v_, k_scale=wl.k_scale,
                             v_scale=wl.v_scale, kv_dtype=kvd)

    log(f"[bench] {n_layers} KV pool copies of {pool_bytes / 1e6:.0f} MB; warmup {args.warmup}")
    for i in range(args.warmup):
        write(i % n_layers)
        decode(i % n_layers)
    torch.cuda.synchronize()

    # the timed steps: nothing but the steps between the two synchronisations
    K = args.steps
    log(f"[bench] timing {K} steps")
    t0 = time.perf_counter()
    for i in range(K):
        write(i % n_layers)
        decode(i % n_layers)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K

    # then the same steps again with the decode call of each between two
    # HIP events on its stream (each marker idles the GPU for a few
    # microseconds, so these steps are not the timed ones)
    timer = HipTimingEvents()
    n_ev = max(args.timed_launches, 1)
    evs = [(timer.create(), timer.create()) for _ in range(n_ev)]
    log(f"[bench] {n_ev} decode launches event-timed")
    for i, (a, b) in enumerate(evs):
        write(i % n_layers)
        timer.record(a, stream)
        decode(i % n_layers)
        timer.record(b, stream)
    torch.cuda.synchronize()
    dec_ms = [timer.elapsed_ms(a, b) for a, b in evs]
    dec_mean = float(np.mean(dec_ms))
    dec_med = float(np.median(dec_ms))

    # context: the same copy decoded back to back (part of it stays in cache)
    hot_ms = []
    for _ in range(args.hot_iters):
        a, b = timer.create(), timer.create()
        timer.record(a, stream)
        decode(0)
        timer.record(b, stream)
        hot_ms.append(timer.elapsed_ms(a, b))
    # pa_reshape_and_cache on its own, after the timed steps: the step's new
    # token per sequence, and a bulk write of every token of the batch (the
    # cache fill), each launch between two events.  A decode call is queued
    # in front of each, so the host has enqueued the write before the GPU
    # reaches it and the events time the kernel, not the host's launch.
    def timed(fn, layer):
        a, b = timer.create(), timer.create()
        decode(layer)
        timer.record(a, stream)
        fn()
        timer.record(b, stream)
        return timer.elapsed_ms(a, b)

    wr_step_ms = [timed(lambda: write(i % n_layers), (i + 1) % n_layers)
                  for i in range(args.write_iters)]
    wr_bulk_ms = []
    if args.write_iters:
        all_k, all_v = wl.tok_key.to(dev), wl.tok_value.to(dev)
        all_s = torch.from_numpy(wl.slot_mapping).to(dev)
        for i in range(3):
            k_, v_ = layers[i % n_layers]
            wr_bulk_ms.append(timed(lambda: pa.reshape_and_cache(
                all_k, all_v, all_s, k_, v_, k_scale=wl.k_scale, v_scale=wl.v_scale,
                kv_dtype=kvd), (i + 1) % n_layers))
        del all_k, all_v, all_s
    timer.close()
    hot_med = float(np.median(hot_ms)) if hot_ms else None
    # bytes a write moves per token: K and V read in the source dtype and
    # written in the cache dtype, plus its slot
    tok_bytes = 2 * c.num_kv_heads * c.head_dim * (wl.tok_key.element_size() + kc.element_size()) + 8
    cache_write = None
    if wr_step_ms:
        step_us = float(np.median(wr_step_ms)) * 1e3
        bulk_ms = float(np.median(wr_bulk_ms))
        cache_write = {
            "kernel": "pa_reshape_and_cache",
            "step_tokens": int((wl.new_slots >= 0).sum()),
            "step_median_us": round(step_us, 2),
            "bulk_tokens": wl.num_tokens,
            "bulk_median_ms": round(bulk_ms, 4),
            "bulk_GBps": round(wl.num_tokens * tok_bytes / (bulk_ms * 1e-3) / 1e9, 1),
            "bytes_per_token": tok_bytes,
        }
    del layers, kc, vc, ws
    torch.cuda.empty_cache()

    kv_unique = wl.unique_kv_bytes()
    kv_logical = wl.logical_kv_bytes()
    gbps_step = kv_unique / (ms_step * 1e-3) / 1e9
    achieved = kv_unique / (dec_mean * 1e-3) / 1e9
    launch_desc = f"schedule={plan['schedule']} partition={plan['partition_tokens']} path={args.path}"
    traffic = load_traffic(c.name, launch_desc)
    roof = {
        "bound": "hbm",
        "kernel": ("pa_decode_shared_prefix (prefix pass + decode + merge kernels)" if shared else
                   "pa_decode" + (" (decode + merge kernels)" if plan["schedule"] != "single" else "")),
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": (traffic["hbm_bytes_per_launch"] if traffic else None),
        "algorithmic_bytes_per_launch": kv_unique,
        "mean_launch_ms": round(dec_mean, 5),
        "median_launch_ms": round(dec_med, 5),
        "event_timed_launches": len(dec_ms),
        "kv_pool_copies": n_layers,
        "same_copy_back_to_back_median_ms": round(hot_med, 5) if hot_med else None,
        "same_copy_back_to_back_GBps": round(kv_unique / (hot_med * 1e-3) / 1e9, 1) if hot_med else None,
    }
    res = {
        "metric": METRIC,
        "value": round(gbps_step, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.kv_dtype,
        "data": "synthetic",
        "config": {
            "workload": c.name,
            "batch": c.batch,
            "num_q_heads": c.num_q_heads,
            "num_kv_heads": c.num_kv_heads,
            "head_dim": c.head_dim,
            "block_size": c.block_size,
            "seq_lens": list(map(str, c.lengths)),
            "sum_seq_len": int(wl.seq_lens.astype(np.int64).sum()),
            "q_dtype": c.q_dtype,
            "kv_dtype": c.kv_dtype,
            "schedule": plan["schedule"],
            "partition_tokens": plan["partition_tokens"],
            "path": {0: "auto", 1: "valu", 2: "mfma"}[args.path],
            "block_tables": source,
            "kv_bytes_unique": kv_unique,
            "kv_bytes_logical": kv_logical,
            "parallelism": "single GPU",
        },
        "pct_of_hbm_peak": round(100 * gbps_step / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(c.batch / (ms_step * 1e-3), 1),
        "roofline": roof,
        "cache_write": cache_write,
        "cpu_baseline": None,
    }
    if cpu_seconds > 0:
        log(f"[bench] cpu baseline (~{cpu_seconds}s)")
        res["cpu_baseline"] = cpu_baseline(wl, cpu_seconds)
    return res


# The 70B-shaped GQA decode is the largest single-GPU configuration (1 GiB of
# KV per call) and the headline; the 7B-shaped one rides along.
HEADLINE = "c3"
ALSO = ("c2",)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=None,
                    help="workload name or c1..c6; default: the 70B-shaped GQA decode as the "
                         "headline, with the 7B-shaped decode alongside")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--path", type=int, default=0, help="0 auto, 1 VALU, 2 MFMA")
    ap.add_argument("--layers", type=int, default=0,
                    help="KV pool copies the steps rotate through (0: enough for >= 3 GiB)")
    ap.add_argument("--hot-iters", type=int, default=20)
    ap.add_argument("--write-iters", type=int, default=20,
                    help="pa_reshape_and_cache launches timed on their own, after the steps")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="decode through pa_decode_shared_prefix (workloads with a shared prefix)")
    ap.add_argument("--timed-launches", type=int, default=40,
                    help="decode launches timed one by one with HIP events, after the timed steps")
    ap.add_argument("--time-every", type=int, default=4,
                    help="prefill: event-time the attention launch of every N-th timed step")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--max-query-len", type=int, default=0,
                    help="prefill: max_query_len passed to pa_prefill (sizes its grid; 0 = the true maximum)")
    ap.add_argument("--op", default="decode", choices=["decode", "prefill", "swap"],
                    help="decode: the decode hot path (default); prefill: causal prefill of "
                         "new tokens over the cache (--config p1 | p2); swap: the batch's KV "
                         "blocks swapped out to pinned host memory and back in (pa_swap_blocks)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the decode path shards by kv head or by sequence with no exchange inside attention, "
              "and the library has no multi-GPU launch to measure.", file=sys.stderr)
        return 2

    import torch

    import paged_kv_cache_462_amd as pa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    pa.load()
    if args.op == "swap":
        if args.config is None:
            args.config = "c2"
        return bench_swap(args)
    if args.op == "prefill":
        if args.config is None:
            args.config = "p1"
        return bench_prefill(args)
    cpu_s = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    if args.config is not None:
        print(json.dumps(run_decode(args.config, args, cpu_s)), flush=True)
        return 0
    res = run_decode(HEADLINE, args, cpu_s)
    res["also"] = {}
    for name in ALSO:
        r = run_decode(name, args, 0.0)
        res["also"][r["config"]["workload"]] = {
            k: r[k] for k in ("value", "unit", "ms_per_step", "pct_of_hbm_peak", "tokens_per_s",
                              "dtype", "config", "roofline", "cache_write")}
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
