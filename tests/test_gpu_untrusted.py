"""Device-resident contents outside their contract: block ids outside the
pool (past its end, negative, the largest int32), lengths past what the
block table reaches or negative, and cache-write slots outside the cache.
The calls stay inside their buffers and give what the oracle gives on the
contents taken the documented way: an id outside the pool reads block 0, a
length is clamped to [0, max_blocks * block_size], an out-of-cache slot is
skipped.  A caller's error-flag array (the launch's error_flags) gets the
flag of every kind of content taken that way, and no other; a clean call
leaves it zero."""

import numpy as np
import pytest
import torch

import paged_kv_cache_462_amd as pa
from synth import get_config, make_prefill_rows, make_workload
from synth.generate import shrink
from tests import _gpu as G

pytestmark = pytest.mark.gpu

VALU, MFMA = 1, 2
BLOCK, LENGTH, SLOT, QSTART = (pa.PA_FLAG_BLOCK_ID, pa.PA_FLAG_LENGTH, pa.PA_FLAG_SLOT,
                               pa.PA_FLAG_QUERY_START)


def _flags():
    return torch.zeros(pa.PA_NUM_FLAGS, dtype=torch.int32, device="cuda")


def _raised(flags):
    torch.cuda.synchronize()
    return {k for k, v in enumerate(flags.tolist()) if v}
LENS = [300, 200, 150, 90, 512, 60]  # 512: the whole table, so a clamped length reads real tokens

CASES = {
    "bf16_g8": shrink(get_config("c3"), batch=len(LENS), lengths=("list", LENS), pool_blocks=0),
    "f16_mha": shrink(get_config("c2"), batch=len(LENS), lengths=("list", LENS), num_q_heads=8,
                      num_kv_heads=8, pool_blocks=0),
    "fp8_g4": shrink(get_config("c5"), batch=len(LENS), lengths=("list", LENS),
                     shared_prefix_tokens=0, pool_blocks=0),
}


def _setup(name, seed):
    wl = make_workload(CASES[name], seed=seed)
    kc, vc = G.oracle_caches(wl)
    d = G.to_device(wl)
    # block 0 is what an id outside the pool reads: give it real tokens (a
    # copy of sequence 0's first block) on both sides
    src = int(wl.block_tables[0, 0])
    kc[0], vc[0] = kc[src].clone(), vc[src].clone()
    d.kc[0], d.vc[0] = d.kc[src].clone(), d.vc[src].clone()
    # corrupt the device-resident contents
    tab = wl.block_tables.copy()
    lens = wl.seq_lens.copy()
    tab[1, 0] = wl.num_blocks + 5
    tab[2, 1] = -7
    tab[3, 0] = 2**31 - 1
    lens[4] = 10**6           # past the table's reach: clamped to max_blocks * bs
    lens[5] = -5              # negative: clamped to 0 (a zero row)
    d.tables = torch.from_numpy(tab).to(d.kc.device)
    d.lens = torch.from_numpy(lens).to(d.kc.device)
    # the contents as the kernels take them, for the oracle
    clean = type(wl)(**{**wl.__dict__})
    t2 = tab.copy()
    t2[(t2 < 0) | (t2 >= wl.num_blocks)] = 0
    clean.block_tables = t2.astype(np.int32)
    clean.seq_lens = np.clip(lens, 0, wl.max_blocks * wl.cfg.block_size).astype(np.int32)
    return wl, clean, kc, vc, d


@pytest.mark.parametrize("name", list(CASES))
def test_decode_with_bad_ids_and_lengths(name):
    wl, clean, kc, vc, d = _setup(name, 91)
    G.say(f"untrusted decode {name}: lens={d.lens.tolist()}")
    ref = G.oracle_decode(clean, kc, vc)
    assert not np.isnan(ref).any()
    atol, rtol = G.tol_for(wl)
    paths = (VALU,) if wl.cfg.q_dtype == "f32" else (VALU, MFMA)
    for path in paths:
        for pt in (0, 512):
            flags = _flags()
            out = G.gpu_decode(wl, d, partition_tokens=pt, path=path, error_flags=flags)
            torch.cuda.synchronize()
            G.assert_close(out, ref, atol, rtol, what=f"untrusted decode {name} path={path} pt={pt}")
            assert _raised(flags) == {BLOCK, LENGTH}


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_with_bad_ids_and_lengths(name):
    wl, clean, kc, vc, d = _setup(name, 92)
    rows = make_prefill_rows(wl, ("list", [100, 200, 150, 1, 250, 60]), seed=93)
    G.say(f"untrusted prefill {name}")
    ref = G.oracle_prefill(clean, kc, vc, rows)
    assert not np.isnan(ref).any()
    flags = _flags()
    out = G.gpu_prefill(wl, d, rows, error_flags=flags)
    torch.cuda.synchronize()
    atol, rtol = G.tol_for(wl)
    G.assert_close(out, ref, atol, rtol, what=f"untrusted prefill {name}")
    assert _raised(flags) == {BLOCK, LENGTH}


@pytest.mark.parametrize("name", ["bf16_g8", "fp8_g4"])
def test_cache_write_skips_slots_outside_the_cache(name):
    wl = make_workload(CASES[name], seed=94)
    G.say(f"untrusted cache write {name}")
    slots = wl.slot_mapping.copy()
    n_slots = wl.num_blocks * wl.cfg.block_size
    bad = [3, 50, 400]
    slots[bad[0]] = n_slots          # one past the end
    slots[bad[1]] = n_slots + 12345
    slots[bad[2]] = 1 << 40
    clean = slots.copy()
    clean[bad] = -1
    d = G.to_device(wl, fill=False)
    kvd = "fp8" if wl.cfg.kv_dtype == "fp8" else None
    flags = _flags()
    pa.reshape_and_cache(d.tok_key, d.tok_value, torch.from_numpy(slots).to(d.kc.device), d.kc, d.vc,
                         k_scale=wl.k_scale, v_scale=wl.v_scale, kv_dtype=kvd, error_flags=flags)
    assert _raised(flags) == {SLOT}
    wl2 = type(wl)(**{**wl.__dict__})
    wl2.slot_mapping = clean
    kc, vc = G.oracle_caches(wl2)
    assert G.caches_equal(d.kc, kc) and G.caches_equal(d.vc, vc)


@pytest.mark.parametrize("name", ["bf16_g8", "fp8_g4"])
def test_clean_calls_raise_no_flag(name):
    """Valid contents (negative cache-write slots included, which skip by
    contract): every call leaves the flags at zero."""
    wl = make_workload(CASES[name], seed=95)
    G.say(f"clean flags {name}")
    d = G.to_device(wl, fill=False)
    kvd = "fp8" if wl.cfg.kv_dtype == "fp8" else None
    slots = wl.slot_mapping.copy()
    slots[7] = -1
    flags = _flags()
    pa.reshape_and_cache(d.tok_key, d.tok_value, torch.from_numpy(slots).to(d.kc.device), d.kc, d.vc,
                         k_scale=wl.k_scale, v_scale=wl.v_scale, kv_dtype=kvd, error_flags=flags)
    for path in (VALU, MFMA):
        for pt in (0, -1, 64):
            G.gpu_decode(wl, d, partition_tokens=pt, path=path, error_flags=flags)
    rows = make_prefill_rows(wl, ("list", [100, 200, 150, 1, 250, 60]), seed=96)
    G.gpu_prefill(wl, d, rows, error_flags=flags)
    pairs = torch.tensor([[int(wl.block_tables[0, 0]), 0]], dtype=torch.int32, device="cuda")
    pa.copy_blocks(d.kc, d.vc, pairs, kv_dtype=kvd, error_flags=flags)
    assert _raised(flags) == set()


def test_prefill_flags_query_start_past_the_rows():
    """query_start_loc ending past the packed rows is clamped to them (the
    same rows as the clean call) and raises the query-start flag."""
    wl = make_workload(CASES["bf16_g8"], seed=97)
    rows = make_prefill_rows(wl, ("list", [100, 200, 150, 1, 250, 60]), seed=98)
    G.say("untrusted query_start_loc")
    d = G.to_device(wl)
    clean = G.gpu_prefill(wl, d, rows)
    qsl = rows.query_start_loc.copy()
    qsl[-1] += 5
    flags = _flags()
    out = G.gpu_prefill(wl, d, rows, qsl=torch.from_numpy(qsl).to(d.kc.device), error_flags=flags)
    assert _raised(flags) == {QSTART}
    assert torch.equal(out, clean)


def test_copy_blocks_flags_pairs_outside_the_pool():
    """A block pair naming a block outside the pool is skipped and raises the
    block-id flag; the valid pair of the same call is copied."""
    G.say("untrusted block copy")
    shape = (12, 16, 2, 128)
    kc = torch.randn(shape, dtype=torch.bfloat16, device="cuda")
    vc = torch.randn(shape, dtype=torch.bfloat16, device="cuda")
    k0, v0 = kc.clone(), vc.clone()
    pairs = torch.tensor([[1, 2], [3, 12], [-1, 4]], dtype=torch.int32, device="cuda")
    flags = _flags()
    pa.copy_blocks(kc, vc, pairs, error_flags=flags)
    assert _raised(flags) == {BLOCK}
    k0[2], v0[2] = k0[1], v0[1]
    assert torch.equal(kc, k0) and torch.equal(vc, v0)


# sequence 3 is the longest, 608 tokens: the whole table, so its length
# clamped from a value past the table's reach reads real tokens
SHARED = {
    # 6 x 8 rows per kv head: the grouped prefix work in the decode launch
    "grouped": [300, 200, 256, 608, 512, 60],
    # 130 x 8 = 1040 rows: the prefix pass
    "pass": [int(x) for x in np.random.default_rng(99).integers(0, 600, 130)],
}
SHARED["pass"][3] = 608


@pytest.mark.parametrize("way", list(SHARED))
def test_shared_prefix_with_bad_prefix_ids_and_lengths(way):
    """pa_decode_shared_prefix reads the prefix through its own block list:
    ids there outside the pool read block 0 and raise the block-id flag, as
    lengths outside the table's reach raise the length flag; the result is
    the oracle's on the contents taken that way (the prefix part of every
    sequence from the clamped list, the rest from its own table)."""
    P = 256
    lens = SHARED[way]
    cfg = shrink(get_config("c3"), batch=len(lens), lengths=("list", lens),
                 shared_prefix_tokens=P, pool_blocks=0)
    wl = make_workload(cfg, seed=90)
    bs = cfg.block_size
    assert wl.max_blocks * bs == lens[3]
    kc, vc = G.oracle_caches(wl)
    d = G.to_device(wl)
    src = int(wl.block_tables[0, 0])
    kc[0], vc[0] = kc[src].clone(), vc[src].clone()
    d.kc[0], d.vc[0] = d.kc[src].clone(), d.vc[src].clone()
    pref = wl.shared_blocks.astype(np.int64).copy()
    pref[1] = wl.num_blocks + 3
    pref[4] = -2
    lens2 = wl.seq_lens.copy()
    lens2[3] = 10**6
    lens2[5] = -1
    d.lens = torch.from_numpy(lens2).to(d.kc.device)
    G.say(f"untrusted shared prefix {way}: B={cfg.batch}")
    clean = type(wl)(**{**wl.__dict__})
    cl = np.clip(lens2, 0, wl.max_blocks * bs).astype(np.int32)
    clean.seq_lens = cl
    ids = np.where((pref < 0) | (pref >= wl.num_blocks), 0, pref)
    t2 = wl.block_tables.copy()
    for b in range(cfg.batch):
        nb = -(-min(int(cl[b]), P) // bs)
        t2[b, :nb] = ids[:nb]
    clean.block_tables = t2.astype(np.int32)
    ref = G.oracle_decode(clean, kc, vc)
    assert not np.isnan(ref).any()
    out = torch.empty_like(d.query)
    flags = _flags()
    pb = torch.from_numpy(pref.astype(np.int32)).to(d.kc.device)
    pa.decode_shared_prefix(out, d.query, d.kc, d.vc, d.tables, d.lens, pb, P, wl.scale, bs,
                            cfg.num_kv_heads, error_flags=flags)
    torch.cuda.synchronize()
    atol, rtol = G.tol_for(wl)
    G.assert_close(out, ref, atol, rtol, what=f"untrusted shared prefix {way}")
    assert _raised(flags) == {BLOCK, LENGTH}
