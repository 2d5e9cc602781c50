"""Pools past 4 GiB per cache: every byte offset the kernels form must be
64-bit.  A small workload is re-paged to the top of a pool of 5 GiB per
cache (block i moves to block N - 1 - i, the table and slots follow), so
every block the kernels touch sits beyond the first 4 GiB.  The cache write
must leave the same bytes there as in the small pool, decode and prefill the
same bits (the result does not depend on where the blocks are) and the
oracle's values, and a block copy between two of the top blocks the bytes
of its source."""

import numpy as np
import pytest
import torch

import paged_kv_cache_462_amd as pa
from synth import get_config, make_prefill_rows, make_workload
from synth.generate import shrink
from tests import _gpu as G

pytestmark = pytest.mark.gpu

POOL_BYTES = 5 << 30  # per cache

# (config, prefill rows per sequence)
CASES = {
    # 70B-shaped GQA bf16, block size 16: 32 KiB blocks, 163 840 of them
    "bf16_g8": (shrink(get_config("c3"), batch=3, lengths=("list", [700, 33, 1500]), pool_blocks=0),
                [300, 33, 1]),
    # fp8 K/V with a bf16 query, block size 32, group 4: 32 KiB blocks
    "fp8_g4_bs32": (shrink(get_config("c5"), shared_prefix_tokens=0, batch=3,
                           lengths=("list", [900, 1, 64]), pool_blocks=0),
                    [512, 1, 64]),
}


def _repage_to_top(wl, n_big):
    """The same workload with block i of the pool at block n_big - 1 - i."""
    bs = wl.cfg.block_size
    big = type(wl)(**{**wl.__dict__})
    big.num_blocks = n_big
    big.block_tables = np.where(wl.block_tables >= 0, n_big - 1 - wl.block_tables, -1).astype(np.int32)
    big.slot_mapping = (n_big - 1 - wl.slot_mapping // bs) * bs + wl.slot_mapping % bs
    return big


def _bits(t):
    return t.view(torch.int16)


@pytest.mark.parametrize("name", list(CASES))
def test_pool_past_4gib(name):
    cfg, news = CASES[name]
    wl = make_workload(cfg, seed=71)
    c = wl.cfg
    block_bytes = c.block_size * c.num_kv_heads * c.head_dim * wl.kv_bytes_per_elem()
    n_big = POOL_BYTES // block_bytes
    big = _repage_to_top(wl, n_big)
    used = np.unique(wl.block_tables[wl.block_tables >= 0]).astype(np.int64)
    lowest = int(n_big - 1 - used.max())
    assert lowest * block_bytes >= 1 << 32 and n_big < 2**31
    G.say(f"large pool {name}: {n_big} blocks of {block_bytes} B per cache, "
          f"lowest block used {lowest} (byte offset {lowest * block_bytes})")

    kc, vc = G.oracle_caches(wl)
    small = G.to_device(wl)
    d = G.to_device(big)  # 2 x 5 GiB of poison, then the cache write at the top
    dev = d.kc.device
    top = torch.from_numpy(n_big - 1 - used).to(dev)
    low = torch.from_numpy(used).to(dev)
    torch.cuda.synchronize()
    assert G.caches_equal(d.kc[top], small.kc[low]) and G.caches_equal(d.vc[top], small.vc[low])
    assert G.caches_equal(d.kc[top], kc[torch.from_numpy(used)])
    assert G.caches_equal(d.vc[top], vc[torch.from_numpy(used)])

    atol, rtol = G.tol_for(wl)
    ref = G.oracle_decode(wl, kc, vc)
    for pt in (0, 512):
        a = G.gpu_decode(wl, small, partition_tokens=pt)
        b = G.gpu_decode(big, d, partition_tokens=pt)
        torch.cuda.synchronize()
        assert torch.equal(_bits(a), _bits(b)), f"decode partition_tokens={pt}"
        G.assert_close(b, ref, atol, rtol, what=f"large pool decode {name} pt={pt}")

    rows = make_prefill_rows(wl, ("list", news), seed=72)
    a = G.gpu_prefill(wl, small, rows)
    b = G.gpu_prefill(big, d, rows)
    torch.cuda.synchronize()
    assert torch.equal(_bits(a), _bits(b)), "prefill"
    G.assert_close(b, G.oracle_prefill(wl, kc, vc, rows), atol, rtol, what=f"large pool prefill {name}")

    # copy-on-write copy of the topmost used block onto the block below the
    # lowest used one
    src, dst = int(n_big - 1 - used.min()), lowest - 1
    pairs = torch.tensor([[src, dst]], dtype=torch.int32, device=dev)
    pa.copy_blocks(d.kc, d.vc, pairs, kv_dtype="fp8" if c.kv_dtype == "fp8" else None)
    torch.cuda.synchronize()
    assert G.caches_equal(d.kc[dst], d.kc[src]) and G.caches_equal(d.vc[dst], d.vc[src])
    del d, small
    torch.cuda.empty_cache()
