"""Head shapes outside the power-of-two grid: query heads per kv head of 3,
6, 12, 16 and 32 (partly filled MFMA head tiles, two head tiles per kv head,
VALU tiles with idle heads) and odd kv-head counts (unit chunks whose last
workgroup has waves without a unit).  Decode on both inner loops and both
schedules, and prefill, against the fp64 oracle."""

import pytest
import torch

from synth import get_config, make_prefill_rows, make_workload
from synth.generate import shrink
from tests import _gpu as G

pytestmark = pytest.mark.gpu

VALU, MFMA = 1, 2
LENS = [1, 17, 300, 0, 1111, 64]
NEWS = [1, 17, 100, 0, 300, 64]

# name: (Hq, Hkv, head_dim, q dtype, kv dtype)
SHAPES = {
    "g3_hkv5_bf16": (15, 5, 128, "bf16", "bf16"),
    # 6 sequences x 4 kv heads = 24 groups: the prefill's XCD-grouped order
    "g3_hkv4_f16": (12, 4, 128, "f16", "f16"),
    "g6_hkv2_f16": (12, 2, 128, "f16", "f16"),
    "g12_hkv2_fp8": (24, 2, 128, "bf16", "fp8"),
    "g16_hkv3_bf16_d64": (48, 3, 64, "bf16", "bf16"),
    "g32_hkv2_f16": (64, 2, 128, "f16", "f16"),
    "mha7_f16_d64": (7, 7, 64, "f16", "f16"),
    "mqa6_bf16": (6, 1, 128, "bf16", "bf16"),
}

_cache = {}


def _workload(name):
    if name not in _cache:
        hq, hkv, d, qd, kd = SHAPES[name]
        base = get_config("c5") if kd == "fp8" else get_config("c3")
        cfg = shrink(base, batch=len(LENS), lengths=("list", LENS), num_q_heads=hq,
                     num_kv_heads=hkv, head_dim=d, q_dtype=qd, kv_dtype=kd,
                     block_size=16,
                     shared_prefix_tokens=0, pool_blocks=0)
        wl = make_workload(cfg, seed=400 + hq + hkv)
        kc, vc = G.oracle_caches(wl)
        _cache[name] = (wl, kc, vc)
    return _cache[name]


@pytest.mark.parametrize("name", list(SHAPES))
def test_head_shape_decode(name):
    wl, kc, vc = _workload(name)
    G.say(f"head shape {name}: Hq={wl.cfg.num_q_heads} Hkv={wl.cfg.num_kv_heads}")
    ref = G.oracle_decode(wl, kc, vc)
    d = G.to_device(wl)
    atol, rtol = G.tol_for(wl)
    for path in (VALU, MFMA):
        for pt in (0, 512):
            out = G.gpu_decode(wl, d, partition_tokens=pt, path=path)
            torch.cuda.synchronize()
            G.assert_close(out, ref, atol, rtol, what=f"decode {name} path={path} pt={pt}")


@pytest.mark.parametrize("name", list(SHAPES))
def test_head_shape_prefill(name):
    wl, kc, vc = _workload(name)
    rows = make_prefill_rows(wl, ("list", NEWS), seed=401)
    G.say(f"head shape {name} prefill")
    d = G.to_device(wl)
    out = G.gpu_prefill(wl, d, rows)
    torch.cuda.synchronize()
    atol, rtol = G.tol_for(wl)
    G.assert_close(out, G.oracle_prefill(wl, kc, vc, rows), atol, rtol, what=f"prefill {name}")
