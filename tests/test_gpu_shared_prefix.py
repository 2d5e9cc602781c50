"""Shared-prefix decode on the GPU (pa_decode_shared_prefix through the C
ABI) against the fp64 decode oracle: the result must be plain decode's, for
sequences shorter than, equal to and longer than the shared prefix, empty
ones included, across the dtype / group / block-size / head_dim variants,
both ways of taking the prefix part (grouped work inside the decode launch
below 1024 (sequence, query head) rows per kv head, the prefix pass from
there on), and every element at the full workload sizes (c5 grouped, c6 the
pass), whose batches are built through the host allocator, block manager
and prefix cache."""

import numpy as np
import pytest
import torch

import paged_kv_cache_462_amd as pa
from synth import get_config, make_workload
from synth.generate import shrink
from tests import _gpu as G

pytestmark = pytest.mark.gpu

# (base config, shared prefix tokens, lengths)
CASES = {
    "fp8_bs32_g4": (get_config("c5"), 1024, [16, 1000, 1024, 1025, 3000, 40, 1, 0]),
    "bf16_g8": (get_config("c3"), 512, [1, 511, 512, 513, 2000, 0]),
    # MHA (group 1): the grouped work puts 16 sequences' rows in a wave, and
    # the rest of each sequence runs on the matrix-core loop as well
    "f16_mha": (shrink(get_config("c2"), num_q_heads=8, num_kv_heads=8), 256,
                [300, 256, 100, 1200, 17]),
    "bf16_g8_d64": (shrink(get_config("c3"), head_dim=64), 384, [800, 5, 384, 1000]),
    # 40 sequences x 8 heads = 320 rows per kv head: 20 row groups of the
    # grouped prefix work
    "bf16_g8_320_rows": (get_config("c3"), 256,
                         [int(x) for x in np.random.default_rng(3).integers(0, 700, 40)]),
    # 1024 rows per kv head or more: the prefix pass, in 256-row tiles (5
    # and 5, the last one partly filled)
    "bf16_g8_pass_1040_rows": (get_config("c3"), 256,
                               [int(x) for x in np.random.default_rng(4).integers(0, 700, 130)]),
    "fp8_g4_pass_1040_rows": (get_config("c5"), 512,
                              [int(x) for x in np.random.default_rng(5).integers(0, 1500, 260)]),
    "fp8_f16q_g4": (shrink(get_config("c5"), q_dtype="f16", block_size=16, shared_prefix_tokens=0),
                    160, [161, 159, 640, 1]),
    # groups that do not divide the 16 query columns: a row group holds the
    # end of one sequence's heads and the start of the next one's
    "bf16_g5_3kv": (shrink(get_config("c3"), num_q_heads=15, num_kv_heads=3), 128,
                    [5, 130, 128, 400, 0, 77, 129]),
    "fp8_g12_2kv_d64": (shrink(get_config("c5"), num_q_heads=24, num_kv_heads=2, head_dim=64,
                               shared_prefix_tokens=0), 64, [64, 63, 65, 500, 1]),
    # 205 x 5 = 1025 rows per kv head: the prefix pass with odd shapes
    "bf16_g5_3kv_pass": (shrink(get_config("c3"), num_q_heads=15, num_kv_heads=3), 256,
                         [int(x) for x in np.random.default_rng(6).integers(0, 450, 205)]),
}


def _case(name, seed=7):
    base, P, lens = CASES[name]
    cfg = shrink(base, batch=len(lens), lengths=("list", lens), shared_prefix_tokens=P,
                 pool_blocks=0)
    wl = make_workload(cfg, seed=seed)
    assert len(wl.shared_blocks) == P // cfg.block_size
    return wl, P


def _run(wl, P, d):
    c = wl.cfg
    out = torch.empty_like(d.query)
    pb = torch.from_numpy(wl.shared_blocks.astype(np.int32)).to(d.kc.device)
    pa.decode_shared_prefix(out, d.query, d.kc, d.vc, d.tables, d.lens, pb, P, wl.scale,
                            c.block_size, c.num_kv_heads, k_scale=wl.k_scale, v_scale=wl.v_scale,
                            kv_dtype="fp8" if c.kv_dtype == "fp8" else None)
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_shared_prefix_matches_decode_oracle(name):
    wl, P = _case(name)
    G.say(f"shared prefix {name}: P={P} lens={wl.seq_lens.tolist()}")
    kc, vc = G.oracle_caches(wl)
    ref = G.oracle_decode(wl, kc, vc)
    d = G.to_device(wl)
    out = _run(wl, P, d)
    torch.cuda.synchronize()
    atol, rtol = G.tol_for(wl)
    G.assert_close(out, ref, atol, rtol, what=f"shared prefix {name}")
    # and within the same bound of the plain decode kernels
    plain = G.gpu_decode(wl, d)
    torch.cuda.synchronize()
    G.assert_close(plain, ref, atol, rtol, what=f"plain decode {name}")


def test_shared_prefix_deterministic():
    wl, P = _case("bf16_g8")
    G.say("shared prefix determinism")
    d = G.to_device(wl)
    a = _run(wl, P, d)
    b = _run(wl, P, d)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name", ["c5", "c6"])
def test_prefix_cache_chain_full_size(name):
    """The full-size shared-prompt batch built through the host chain
    (allocator with the seeded order -> prompt admitted and cached ->
    every request admitted through the prefix cache -> prompt sequence
    released), its K/V written at the chain's slots by pa_reshape_and_cache,
    then pa_decode and pa_decode_shared_prefix: every output element of
    both against the decode oracle on the same tables and caches.  Prompt
    blocks carry one reference per request that fills them plus the
    cache's; releasing every request and evicting the cache frees the
    whole pool."""
    cfg = get_config(name)
    wl = make_workload(cfg)
    P = cfg.shared_prefix_tokens
    bs = cfg.block_size
    ch = G.admit_chain(wl)
    G.say(f"prefix-cache chain full {name}: B={cfg.batch} P={P} writes={len(ch.slots)}")
    fills = np.array([min(int(L), P) // bs for L in ch.batch.seq_lens])
    for j, blk in enumerate(ch.batch.prompt_blocks):
        assert ch.alloc.refcount(int(blk)) == 1 + int((fills > j).sum())
    kc, vc = G.chain_oracle_caches(wl, ch)
    d = G.chain_to_device(wl, ch)
    plain = G.gpu_decode(wl, d)
    shared = torch.empty_like(d.query)
    pb = torch.from_numpy(ch.batch.prompt_blocks.astype(np.int32)).to(d.kc.device)
    pa.decode_shared_prefix(shared, d.query, d.kc, d.vc, d.tables, d.lens, pb, P, wl.scale,
                            bs, cfg.num_kv_heads, k_scale=wl.k_scale, v_scale=wl.v_scale,
                            kv_dtype="fp8" if cfg.kv_dtype == "fp8" else None)
    torch.cuda.synchronize()
    assert G.caches_equal(d.kc, kc) and G.caches_equal(d.vc, vc)
    del d
    ref = G.chain_oracle_decode(wl, ch, kc, vc)
    atol, rtol = G.tol_for(wl)
    G.err_summary(plain, ref, atol, rtol, f"chain {name} pa_decode")
    G.err_summary(shared, ref, atol, rtol, f"chain {name} pa_decode_shared_prefix")
    G.assert_close(plain, ref, atol, rtol, what=f"chain {name} pa_decode")
    G.assert_close(shared, ref, atol, rtol, what=f"chain {name} pa_decode_shared_prefix")
    for sid in ch.batch.seq_ids:
        ch.manager.free_sequence(sid)
    ch.cache.evict(wl.num_blocks)
    assert ch.cache.size() == 0 and ch.alloc.num_free() == wl.num_blocks


def _random_case(seed):
    """A seeded shape: dtype pair, head_dim, block size, group, prefix
    length and a length mix around the prefix, with B * G on either side
    of the 1024 rows where the prefix part changes ways."""
    rng = np.random.default_rng(seed)
    q, kv = [("f16", "f16"), ("bf16", "bf16"), ("bf16", "fp8"), ("f16", "fp8")][seed % 4]
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    G = int(rng.choice([1, 2, 4, 5, 8, 16]))
    B = int(rng.integers(1, 40)) if seed % 3 else int(-(-1100 // G))  # many rows every third case
    P = bs * int(rng.integers(1, 1 + 640 // bs))
    kind = rng.integers(0, 3)
    if kind == 0:
        lens = rng.integers(0, 2 * P + 64, B)
    elif kind == 1:
        lens = P + rng.integers(-bs, 3 * bs, B)
    else:
        lens = rng.integers(0, P + 1, B)
    lens = np.maximum(lens, 0)
    lens[0] = max(int(lens[0]), P)  # the tables reach the whole prefix
    base = get_config("c5") if kv == "fp8" else get_config("c3")
    cfg = shrink(base, batch=B, num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                 q_dtype=q, kv_dtype=kv, lengths=("list", [int(x) for x in lens]),
                 shared_prefix_tokens=P, pool_blocks=0)
    return cfg, P


@pytest.mark.parametrize("seed", range(12))
def test_shared_prefix_random_shapes(seed):
    cfg, P = _random_case(seed)
    wl = make_workload(cfg, seed=700 + seed)
    G.say(f"shared prefix random {seed}: B={cfg.batch} Hq={cfg.num_q_heads} Hkv={cfg.num_kv_heads} "
          f"D={cfg.head_dim} bs={cfg.block_size} {cfg.q_dtype}/{cfg.kv_dtype} P={P} "
          f"rows={cfg.batch * cfg.num_q_heads // cfg.num_kv_heads}")
    kc, vc = G.oracle_caches(wl)
    ref = G.oracle_decode(wl, kc, vc)
    d = G.to_device(wl)
    out = _run(wl, P, d)
    torch.cuda.synchronize()
    atol, rtol = G.tol_for(wl)
    G.assert_close(out, ref, atol, rtol, what=f"shared prefix random {seed}")
