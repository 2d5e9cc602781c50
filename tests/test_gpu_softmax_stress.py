"""Online-softmax stress on the GPU, against the fp64 oracle.

The synthetic N(0, 1) workloads move the running max of a sequence by more
than a few units (log2) only on its first tiles.  Here the keys are built so
that the max keeps moving along the whole sequence:

* growing scores: every key is c * position along one direction that every
  query shares, so each 16-token tile raises the max by a set step; steps
  below the matrix-core loop's lazy-rescale threshold (2^8) let the weights
  grow towards 2^8 before the reference moves, steps above it move the
  reference on every tile;
* heavy-tailed scores: the drawn keys scaled by 6, so the max jumps at
  random places.

Each case runs on both inner loops and under the balanced, single-pass and
fixed-partition schedules."""

import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_462_amd as pa
from synth import get_config, make_workload
from synth.generate import TORCH_DTYPES, shrink
from tests import _gpu as G

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634

CASES = {
    "c2": ("c2", [1, 15, 300, 777, 1500]),    # f16 MHA
    "c3": ("c3", [16, 513, 1200]),            # bf16, 8 query heads per kv head
    "c4": ("c4", [3000, 200]),                # bf16, 4 per kv head
    "c5": ("c5", [33, 700, 1400]),            # fp8 K/V, bf16 query
}


def _workload(name):
    base, lens = CASES[name]
    cfg = shrink(get_config(base), batch=len(lens), lengths=("list", lens),
                 shared_prefix_tokens=0)
    return make_workload(cfg, seed=31)


def _positions(wl):
    """Position in its sequence of every token of the stream."""
    bs = wl.cfg.block_size
    pos_of_slot = np.full(wl.num_blocks * bs, -1, dtype=np.int64)
    for b in range(wl.cfg.batch):
        t = np.arange(int(wl.seq_lens[b]), dtype=np.int64)
        s = wl.block_tables[b, t // bs].astype(np.int64) * bs + t % bs
        pos_of_slot[s] = t
    pos = pos_of_slot[wl.slot_mapping]
    assert (pos >= 0).all()
    return pos


def _with_keys(wl, keys_f32, query_f32=None):
    """The workload with new token keys (and queries), cast to the source
    dtype, and the fp8 key scale recomputed the way the generator does."""
    c = wl.cfg
    tok_key = keys_f32.to(TORCH_DTYPES[c.src_dtype])
    k_scale = wl.k_scale
    if c.kv_dtype == "fp8":
        k_scale = float(np.float32(tok_key.abs().max().float().item()) / np.float32(448.0))
    kw = dict(tok_key=tok_key, k_scale=k_scale)
    if query_f32 is not None:
        kw["query"] = query_f32.to(TORCH_DTYPES[c.q_dtype])
    return dataclasses.replace(wl, **kw)


def _growing(wl, step_log2):
    """Keys c * position * u (plus a little noise) and queries sqrt(D) * u,
    so the score of the token at position t is about c * t and each
    16-token tile raises it by step_log2 in log2 units."""
    c = wl.cfg
    rng = np.random.default_rng(7)
    u = rng.standard_normal(c.head_dim).astype(np.float32)
    u /= np.linalg.norm(u)
    coef = step_log2 / (16.0 * LOG2E)
    pos = torch.from_numpy(_positions(wl).astype(np.float32))
    noise = torch.from_numpy(rng.standard_normal(tuple(wl.tok_key.shape)).astype(np.float32))
    keys = pos[:, None, None] * coef * torch.from_numpy(u) + 0.05 * noise
    query = torch.from_numpy(np.broadcast_to(u * np.sqrt(c.head_dim, dtype=np.float32),
                                             tuple(wl.query.shape)).copy())
    return _with_keys(wl, keys, query)


def _heavy(wl):
    return _with_keys(wl, wl.tok_key.float() * 6.0)


def _run(wl, what):
    kc, vc = G.oracle_caches(wl)
    ref = G.oracle_decode(wl, kc, vc)
    d = G.to_device(wl)
    torch.cuda.synchronize()
    assert G.caches_equal(d.kc, kc) and G.caches_equal(d.vc, vc), f"{what}: cache write"
    atol, rtol = G.tol_for(wl)
    paths = [pa.PATH_VALU, pa.PATH_MFMA]
    for path in paths:
        for pt in (0, -1, 64):
            G.say(f"{what} path={path} partition={pt}")
            out = G.gpu_decode(wl, d, partition_tokens=pt, path=path)
            torch.cuda.synchronize()
            G.assert_close(out, ref, atol, rtol, what=f"{what} path={path} partition={pt}")


@pytest.mark.parametrize("step", [0.5, 3.0, 12.0])
@pytest.mark.parametrize("name", list(CASES))
def test_growing_scores(name, step):
    _run(_growing(_workload(name), step), f"growing scores {name} step={step}")


@pytest.mark.parametrize("name", list(CASES))
def test_heavy_tailed_scores(name):
    _run(_heavy(_workload(name)), f"heavy-tailed scores {name}")
