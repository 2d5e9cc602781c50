"""Block sizes past 16 and 32: any multiple of 16 is accepted, including
ones that are not powers of two (the kernels then take the general
slot-in-block arithmetic).  Cache write bit-exact, decode (both inner loops,
both schedules) and prefill against the fp64 oracle, on lengths that end
inside a block, exactly on a block boundary, and at zero."""

import pytest
import torch

from synth import get_config, make_prefill_rows, make_workload
from synth.generate import shrink
from tests import _gpu as G

pytestmark = pytest.mark.gpu

VALU, MFMA = 1, 2

# (base config, overrides): MHA fp16, GQA 8 bf16, fp8 K/V with a bf16 query
BASES = {
    "f16_mha": (get_config("c2"), dict(num_q_heads=8, num_kv_heads=8)),
    "bf16_g8": (get_config("c3"), dict()),
    "fp8_g4": (get_config("c5"), dict(shared_prefix_tokens=0)),
}
BLOCK_SIZES = (48, 64, 128)


def _lengths(bs):
    # inside the first block, exactly one block, a block plus one token,
    # several blocks with a ragged end, zero, and a long one
    return [7, bs, bs + 1, 5 * bs - 3, 0, 1500]


_cache = {}


def _workload(name, bs):
    key = (name, bs)
    if key not in _cache:
        base, kw = BASES[name]
        lens = _lengths(bs)
        cfg = shrink(base, batch=len(lens), lengths=("list", lens), block_size=bs, pool_blocks=0, **kw)
        wl = make_workload(cfg, seed=300 + bs)
        kc, vc = G.oracle_caches(wl)
        _cache[key] = (wl, kc, vc, G.oracle_decode(wl, kc, vc))
    return _cache[key]


@pytest.mark.parametrize("bs", BLOCK_SIZES)
@pytest.mark.parametrize("name", list(BASES))
def test_block_size_decode_and_cache_write(name, bs):
    wl, kc, vc, ref = _workload(name, bs)
    G.say(f"block size {bs} {name}: lens={wl.seq_lens.tolist()}")
    d = G.to_device(wl)
    torch.cuda.synchronize()
    assert G.caches_equal(d.kc, kc) and G.caches_equal(d.vc, vc)
    atol, rtol = G.tol_for(wl)
    paths = (VALU,) if wl.cfg.q_dtype == "f32" else (VALU, MFMA)
    for path in paths:
        for pt in (0, 512):
            out = G.gpu_decode(wl, d, partition_tokens=pt, path=path)
            torch.cuda.synchronize()
            G.assert_close(out, ref, atol, rtol, what=f"decode bs={bs} {name} path={path} pt={pt}")


@pytest.mark.parametrize("bs", BLOCK_SIZES)
@pytest.mark.parametrize("name", list(BASES))
def test_block_size_prefill(name, bs):
    wl, kc, vc, _ = _workload(name, bs)
    # chunks of every length: the whole sequence, one row, a block's worth
    news = [min(int(L), n) for L, n in zip(wl.seq_lens, [7, 1, bs, 2 * bs + 5, 0, 700])]
    rows = make_prefill_rows(wl, ("list", news), seed=301 + bs)
    G.say(f"block size {bs} {name} prefill: rows={news}")
    d = G.to_device(wl)
    out = G.gpu_prefill(wl, d, rows)
    torch.cuda.synchronize()
    atol, rtol = G.tol_for(wl)
    G.assert_close(out, G.oracle_prefill(wl, kc, vc, rows), atol, rtol, what=f"prefill bs={bs} {name}")
