"""HIP path vs the CPU oracle, element by element (GPU).

Small cases span several 16-token tiles with ragged tails and run every
path / partition choice; full-size cases run in the benchmark's launch
configuration and compare every output element.  Cache writes are compared bit for
bit."""

import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_462_amd as pa
from oracle import fp8 as OF8
from synth import get_config, make_workload
from synth.generate import shrink
from tests import _gpu as G

pytestmark = pytest.mark.gpu

VALU, MFMA = pa.PATH_VALU, pa.PATH_MFMA

SMALL = {
    "c1": (get_config("c1"), None),
    "c2": (shrink(get_config("c2"), batch=6, lengths=("list", [1, 15, 16, 17, 333, 1000])), None),
    "c3": (shrink(get_config("c3"), batch=4, lengths=("list", [5, 129, 1500, 0])), None),
    "c4": (shrink(get_config("c4"), batch=2, lengths=("list", [3000, 777])), None),
    "c5": (shrink(get_config("c5"), batch=7,
                  lengths=("list", [16, 1000, 1024, 1025, 3000, 40, 1])), None),
}

_cache = {}


def _small(name):
    if name not in _cache:
        cfg = SMALL[name][0]
        wl = make_workload(cfg, seed=77)
        kc, vc = G.oracle_caches(wl)
        ref = G.oracle_decode(wl, kc, vc)
        _cache[name] = (wl, kc, vc, ref)
    return _cache[name]


@pytest.mark.parametrize("name", list(SMALL))
def test_cache_write_bit_exact_small(name):
    wl, kc, vc, _ = _small(name)
    G.say(f"cache write {name} small: T={wl.num_tokens}")
    d = G.to_device(wl)
    torch.cuda.synchronize()
    assert G.caches_equal(d.kc, kc)
    assert G.caches_equal(d.vc, vc)


def _cases():
    out = []
    for name in SMALL:
        fp32 = SMALL[name][0].q_dtype == "f32"
        paths = [VALU] if fp32 else [VALU, MFMA]
        for path in paths:
            for pt in (-1, 0, 16, 48, 512):
                out.append((name, path, pt))
    return out


@pytest.mark.parametrize("name,path,pt", _cases())
def test_decode_small(name, path, pt):
    wl, kc, vc, ref = _small(name)
    G.say(f"decode {name} small path={path} partition={pt} lens={wl.seq_lens.tolist()}")
    d = G.to_device(wl)
    out = G.gpu_decode(wl, d, partition_tokens=pt, path=path)
    torch.cuda.synchronize()
    atol, rtol = G.tol_for(wl)
    G.assert_close(out, ref, atol, rtol, what=f"{name} path={path} pt={pt}")


@pytest.mark.parametrize("name", ["c2", "c3", "c5"])
def test_block_permutation_bit_identical(name):
    wl, kc, vc, _ = _small(name)
    G.say(f"permutation {name}")
    d = G.to_device(wl)
    base = G.gpu_decode(wl, d)
    rng = np.random.default_rng(5)
    p = torch.from_numpy(rng.permutation(wl.num_blocks)).cuda()
    kc2 = torch.empty_like(d.kc)
    vc2 = torch.empty_like(d.vc)
    kc2[p] = d.kc
    vc2[p] = d.vc
    tab = d.tables.long()
    tab2 = torch.where(tab >= 0, p[tab.clamp(min=0)], tab).to(torch.int32)
    d2 = G.Dev(d.query, tab2, d.lens, d.slots, d.tok_key, d.tok_value, kc2, vc2)
    again = G.gpu_decode(wl, d2)
    twice = G.gpu_decode(wl, d)
    torch.cuda.synchronize()
    assert torch.equal(base, again)      # physical placement does not matter
    assert torch.equal(base, twice)      # and reruns are bit-identical


def test_split_matches_single():
    wl, kc, vc, ref = _small("c4")
    G.say("split vs single c4 small")
    d = G.to_device(wl)
    a = G.gpu_decode(wl, d, partition_tokens=-1).double()
    b = G.gpu_decode(wl, d, partition_tokens=512).double()
    c = G.gpu_decode(wl, d, partition_tokens=16).double()
    torch.cuda.synchronize()
    atol, rtol = G.tol_for(wl)
    for x in (b, c):
        err = (x - a).abs()
        assert bool((err <= atol + rtol * a.abs()).all())


def test_zero_and_one_token_sequences():
    cfg = shrink(get_config("c3"), batch=3, lengths=("list", [0, 1, 0]))
    wl = make_workload(cfg, seed=9)
    G.say("zero/one token c3")
    kc, vc = G.oracle_caches(wl)
    d = G.to_device(wl)
    for path in (VALU, MFMA):
        for pt in (-1, 16):
            out = G.gpu_decode(wl, d, partition_tokens=pt, path=path)
            torch.cuda.synchronize()
            assert torch.equal(out[0].float(), torch.zeros_like(out[0].float()))
            assert torch.equal(out[2].float(), torch.zeros_like(out[2].float()))
            # one token: the value row itself (bf16 in, bf16 out: exact)
            v0 = vc[wl.block_tables[1, 0], 0]            # [Hkv, D]
            want = v0.repeat_interleave(cfg.group, dim=0)
            assert torch.equal(out[1].cpu(), want)


def test_fp8_all_codes_decode_exactly():
    """Every E4M3FN code reaches the output unchanged (one-token sequences,
    V scale 1): the device's fp8 decoding equals the oracle's table."""
    cfg = shrink(get_config("c5"), batch=2, lengths=("list", [1, 1]), shared_prefix_tokens=0,
                 num_q_heads=4, num_kv_heads=1)
    wl = make_workload(cfg, seed=1)
    G.say("fp8 all codes")
    d = G.to_device(wl, fill=False)
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).reshape(2, 128)
    kc = torch.full_like(d.kc, 0x38)                 # K = 1.0 everywhere
    vc = torch.full_like(d.vc, 0x7F)
    for b in range(2):
        vc[int(wl.block_tables[b, 0]), 0, 0] = codes[b].cuda()
    d.kc, d.vc = kc, vc
    table = OF8.decode_table()
    for path in (VALU, MFMA):
        out = torch.empty_like(d.query)
        pa.decode(out, d.query, d.kc, d.vc, d.tables, d.lens, wl.scale, cfg.block_size,
                  cfg.num_kv_heads, k_scale=1.0, v_scale=1.0, kv_dtype="fp8", path=path,
                  partition_tokens=-1)
        torch.cuda.synchronize()
        got = out.double().cpu().numpy()
        for b in range(2):
            want = table[codes[b].numpy()]
            for h in range(4):
                g = got[b, h]
                assert np.array_equal(np.isnan(g), np.isnan(want))
                assert np.array_equal(g[~np.isnan(want)], want[~np.isnan(want)]), (path, b, h)


def _quant_case(values: torch.Tensor, scale: float):
    """Write `values` ([T, 1, 128]) into an fp8 cache with the given scale."""
    T = values.shape[0]
    kc = torch.full((T, 16, 1, 128), 0x7F, dtype=torch.uint8, device="cuda")
    vc = kc.clone()
    slots = torch.arange(T, dtype=torch.int64, device="cuda") * 16 + 3
    src = values.cuda()
    pa.reshape_and_cache(src, src, slots, kc, vc, k_scale=scale, v_scale=scale, kv_dtype="fp8")
    torch.cuda.synchronize()
    got = kc[:, 3, 0].cpu().numpy()
    want = OF8.quantize(values[:, 0].to(torch.float32).numpy(), scale)
    return got, want


@pytest.mark.parametrize("scale", [1.0, 0.013950892724096775, 3.0])
def test_fp8_quantiser_every_bf16_pattern(scale):
    """All 65536 bf16 bit patterns (incl. inf, NaN, subnormals) through the
    cache write, bit for bit against the oracle's quantiser."""
    G.say(f"fp8 quantiser bf16 patterns scale={scale}")
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    vals = bits.view(torch.bfloat16).reshape(512, 1, 128)
    got, want = _quant_case(vals, scale)
    bad = np.nonzero(got != want)
    assert got.shape == want.shape
    assert len(bad[0]) == 0, (got[bad][:8], want[bad][:8], vals.reshape(512, 128)[bad][:8])


def test_fp8_quantiser_fp32_edges():
    G.say("fp8 quantiser fp32 edges")
    t = OF8.decode_table()[:0x7F]
    mids = (t[:-1] + t[1:]) / 2
    v = np.concatenate([t, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        [2.0 ** -10, 2.0 ** -11, 447.9, 448.0, 449.0, 464.0, 480.0, 1e30]])
    v = np.concatenate([v, -v]).astype(np.float32)
    rng = np.random.default_rng(3)
    v = np.concatenate([v, (rng.standard_normal(128 * 400) * 60).astype(np.float32)])
    pad = (-len(v)) % 128
    v = np.concatenate([v, np.zeros(pad, np.float32)])
    vals = torch.from_numpy(v).reshape(-1, 1, 128)
    got, want = _quant_case(vals, 1.0)
    assert np.array_equal(got, want)


def test_copy_blocks_bit_exact():
    G.say("copy blocks")
    rng = np.random.default_rng(4)
    kc = torch.randn(50, 16, 8, 128, dtype=torch.bfloat16, device="cuda")
    vc = torch.randn(50, 16, 8, 128, dtype=torch.bfloat16, device="cuda")
    src = rng.choice(25, 10, replace=False)
    dst = 25 + rng.choice(25, 10, replace=False)
    pairs = torch.from_numpy(np.stack([src, dst], 1).astype(np.int32)).cuda()
    k0, v0 = kc.clone(), vc.clone()
    pa.copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    k0[torch.from_numpy(dst).cuda()] = k0[torch.from_numpy(src).cuda()]
    v0[torch.from_numpy(dst).cuda()] = v0[torch.from_numpy(src).cuda()]
    assert torch.equal(kc, k0) and torch.equal(vc, v0)


def test_fork_copy_on_write_end_to_end():
    """Host block manager + device block copy + cache write + decode, against
    the oracle's manager model, cache write and decode."""
    from oracle import attention as OA
    from oracle import cache_write as OW
    from oracle.allocator import RefCountAllocator, SequenceManager

    G.say("fork / copy-on-write")
    bs, Hkv, Hq, D, N = 16, 2, 8, 128, 64
    rng = np.random.default_rng(8)
    alloc = pa.BlockAllocator(N)
    mgr = pa.BlockManager(alloc, bs)
    m_alloc = RefCountAllocator(N)
    model = SequenceManager(m_alloc, bs)
    kc = torch.full((N, bs, Hkv, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = kc.clone()
    kc_o = torch.full((N, bs, Hkv, D), float("nan"), dtype=torch.bfloat16)
    vc_o = kc_o.clone()

    def append(seq, n):
        for _ in range(n):
            slot, src, dst = mgr.append_slot(seq)
            mslot, msrc, mdst = model.append(seq)
            assert (slot, src, dst) == (mslot, msrc, mdst)
            if src >= 0:
                pa.copy_blocks(kc, vc, torch.tensor([[src, dst]], dtype=torch.int32, device="cuda"))
                kc_o[dst] = kc_o[src]
                vc_o[dst] = vc_o[src]
            k = torch.randn(1, Hkv, D).to(torch.bfloat16)
            v = torch.randn(1, Hkv, D).to(torch.bfloat16)
            pa.reshape_and_cache(k.cuda(), v.cuda(), torch.tensor([slot], device="cuda"), kc, vc)
            OW.reshape_and_cache(k, v, np.array([slot]), kc_o, vc_o, "bf16")

    mgr.add_sequence(0)
    model.add(0)
    append(0, 37)                      # 3 blocks, last one 5/16
    mgr.fork(0, 1)
    model.fork(0, 1)
    mgr.fork(0, 2)
    model.fork(0, 2)
    append(1, 20)                      # child 1 copies the shared partial block
    append(2, 3)                       # child 2 copies it too
    append(0, 1)                       # parent's block is private again
    seqs = [0, 1, 2]
    mb = max(mgr.num_blocks_of(s) for s in seqs)
    tables, lens = mgr.export(seqs, mb)
    for i, s in enumerate(seqs):
        assert tables[i, :len(model.tables[s])].tolist() == model.tables[s]
    torch.cuda.synchronize()
    assert G.caches_equal(kc, kc_o) and G.caches_equal(vc, vc_o)
    q = torch.randn(3, Hq, D).to(torch.bfloat16)
    out = torch.empty(3, Hq, D, dtype=torch.bfloat16, device="cuda")
    pa.decode(out, q.cuda(), kc, vc, torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(),
              D ** -0.5, bs, Hkv)
    torch.cuda.synchronize()
    ref = OA.paged_decode_stored(q, kc_o, vc_o, "bf16", 1.0, 1.0, tables, lens, D ** -0.5, bs)
    G.assert_close(out, ref, 2e-3, 1e-2, what="fork/cow")


# --- full sizes, in the benchmark's launch configuration ----------------------

FULL = ["c1", "c2", "c3", "c4", "c5"]


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    """Every output of the full-size workload against the oracle (the error
    summary printed here is the one the measured-results table quotes), and
    the cache write bit for bit."""
    cfg = get_config(name)
    wl = make_workload(cfg)
    G.say(f"full {name}: B={cfg.batch} N={wl.num_blocks} T={wl.num_tokens}")
    kc, vc = G.oracle_caches(wl)
    d = G.to_device(wl)
    out = G.gpu_decode(wl, d)
    torch.cuda.synchronize()
    assert G.caches_equal(d.kc, kc)
    assert G.caches_equal(d.vc, vc)
    del d
    ref = G.oracle_decode(wl, kc, vc)
    atol, rtol = G.tol_for(wl)
    G.err_summary(out, ref, atol, rtol, f"decode full {name}")
    G.assert_close(out, ref, atol, rtol, what=f"full {name}")


# --- the balanced schedule (automatic plan) -------------------------------------

def _wide_table(wl, tokens=512):
    """The same workload with its block table padded (-1) to address at
    least `tokens` tokens, so that the automatic plan is the balanced
    schedule even for short sequences (tables reaching at most 256 tokens
    run in one pass)."""
    bs = wl.cfg.block_size
    extra = max(0, -(-tokens // bs) - wl.max_blocks)
    tables = np.pad(wl.block_tables, ((0, 0), (0, extra)), constant_values=-1)
    return dataclasses.replace(wl, block_tables=tables)


def _random_lengths(B, hi, seed, zero_frac=0.1):
    rng = np.random.default_rng(seed)
    L = rng.integers(1, hi + 1, B)
    L[rng.random(B) < zero_frac] = 0
    return [int(x) for x in L]


@pytest.mark.parametrize("name", ["c2", "c3", "c5"])
def test_balanced_many_sequences(name):
    """More sequences than workgroups, empty ones among them: every piece
    boundary pattern of the balanced schedule, against the oracle."""
    lens = _random_lengths(300, 200, seed=11)
    cfg = shrink(get_config(name), batch=300, lengths=("list", lens))
    wl = _wide_table(make_workload(cfg, seed=12))
    plan = pa.decode_plan(cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                          cfg.block_size, wl.max_blocks, 0)
    assert plan["schedule"] == "balanced"
    G.say(f"balanced many sequences {name}")
    kc, vc = G.oracle_caches(wl)
    d = G.to_device(wl)
    for path in (VALU, MFMA):
        out = G.gpu_decode(wl, d, partition_tokens=0, path=path)
        torch.cuda.synchronize()
        ref = G.oracle_decode(wl, kc, vc)
        atol, rtol = G.tol_for(wl)
        G.assert_close(out, ref, atol, rtol, what=f"balanced {name} path={path}")


@pytest.mark.parametrize("B,schedule", [(2048, "balanced"), (2049, "single")])
def test_balanced_batch_limit(B, schedule):
    """The largest batch the balanced schedule takes, and the first one past
    it (512-token partitions instead, which for these short sequences is one
    pass per sequence)."""
    lens = _random_lengths(B, 40, seed=B)
    cfg = shrink(get_config("c3"), batch=B, lengths=("list", lens))
    wl = _wide_table(make_workload(cfg, seed=13))
    plan = pa.decode_plan(cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                          cfg.block_size, wl.max_blocks, 0)
    assert plan["schedule"] == schedule
    G.say(f"balanced batch limit B={B}")
    kc, vc = G.oracle_caches(wl)
    d = G.to_device(wl)
    out = G.gpu_decode(wl, d, partition_tokens=0)
    torch.cuda.synchronize()
    pairs = G.sample_pairs(wl, 64)
    pairs += [(b, 0) for b in range(B) if lens[b] == 0][:8]
    ref = G.oracle_decode(wl, kc, vc, pairs)
    atol, rtol = G.tol_for(wl)
    G.assert_close(out, ref, atol, rtol, pairs=pairs, what=f"batch limit B={B}")


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c5"])
def test_short_context_single_pass(name):
    """Tables that reach at most 256 tokens: the automatic plan is one pass
    per sequence with no workspace, it matches the oracle, and it matches
    the balanced schedule on the same data with a wider table."""
    lens = {"c1": [100], "c2": [1, 16, 17, 255, 256, 0], "c3": [256, 5, 130],
            "c5": [32, 200, 256, 7]}[name]
    cfg = shrink(get_config(name), batch=len(lens), lengths=("list", lens))
    wl = make_workload(cfg, seed=21)
    plan = pa.decode_plan(cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                          cfg.block_size, wl.max_blocks, 0)
    assert plan["schedule"] == "single" and plan["workspace_bytes"] == 0
    wide = _wide_table(wl)
    plan = pa.decode_plan(cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                          cfg.block_size, wide.max_blocks, 0)
    assert plan["schedule"] == "balanced"
    G.say(f"short context single pass {name}")
    kc, vc = G.oracle_caches(wl)
    d = G.to_device(wl)
    a = G.gpu_decode(wl, d, partition_tokens=0)
    d.tables = torch.from_numpy(wide.block_tables).to(d.tables.device)
    b = G.gpu_decode(wide, d, partition_tokens=0)
    torch.cuda.synchronize()
    ref = G.oracle_decode(wl, kc, vc)
    atol, rtol = G.tol_for(wl)
    G.assert_close(a, ref, atol, rtol, what=f"short single {name}")
    G.assert_close(b, ref, atol, rtol, what=f"short balanced {name}")


@pytest.mark.parametrize("name", ["c2", "c4", "c5"])
def test_balanced_matches_single(name):
    """Balanced pieces merged = one pass over each whole sequence, within the
    16-bit tolerance, and reruns are bit-identical."""
    wl, kc, vc, _ = _small(name)
    G.say(f"balanced vs single {name}")
    d = G.to_device(wl)
    a = G.gpu_decode(wl, d, partition_tokens=-1).double()
    b1 = G.gpu_decode(wl, d, partition_tokens=0)
    b2 = G.gpu_decode(wl, d, partition_tokens=0)
    torch.cuda.synchronize()
    assert torch.equal(b1, b2)
    atol, rtol = G.tol_for(wl)
    err = (b1.double() - a).abs()
    assert bool((err <= atol + rtol * a.abs()).all())


def test_swap_out_and_in_bit_exact():
    """Blocks swapped out to a pinned host pool and back in are the same
    bytes; blocks not named in the pairs stay untouched."""
    G.say("swap out / in")
    rng = np.random.default_rng(6)
    shape = (40, 16, 4, 128)
    kc = torch.randn(shape, dtype=torch.bfloat16, device="cuda")
    vc = torch.randn(shape, dtype=torch.bfloat16, device="cuda")
    hk = torch.full((24,) + shape[1:], float("nan"), dtype=torch.bfloat16).pin_memory()
    hv = torch.full((24,) + shape[1:], float("nan"), dtype=torch.bfloat16).pin_memory()
    src = rng.choice(40, 12, replace=False)
    dst = rng.choice(24, 12, replace=False)
    out_pairs = torch.from_numpy(np.stack([src, dst], 1).astype(np.int32)).cuda()
    pa.swap_blocks(hk, hv, kc, vc, out_pairs)
    torch.cuda.synchronize()
    k0, v0 = kc.cpu(), vc.cpu()
    idx_s, idx_d = torch.from_numpy(src), torch.from_numpy(dst)
    assert G.caches_equal(hk[idx_d], k0[idx_s]) and G.caches_equal(hv[idx_d], v0[idx_s])
    rest = torch.from_numpy(np.setdiff1d(np.arange(24), dst))
    assert torch.isnan(hk[rest].float()).all() and torch.isnan(hv[rest].float()).all()
    # swap back in to other device blocks
    back = rng.choice(40, 12, replace=False)
    in_pairs = torch.from_numpy(np.stack([dst, back], 1).astype(np.int32)).cuda()
    kc2, vc2 = torch.zeros_like(kc), torch.zeros_like(vc)
    pa.swap_blocks(kc2, vc2, hk, hv, in_pairs)
    torch.cuda.synchronize()
    idx_b = torch.from_numpy(back).cuda()
    assert G.caches_equal(kc2[idx_b], kc[torch.from_numpy(src).cuda()])
    assert G.caches_equal(vc2[idx_b], vc[torch.from_numpy(src).cuda()])
    untouched = torch.from_numpy(np.setdiff1d(np.arange(40), back)).cuda()
    assert int(kc2[untouched].abs().sum().item()) == 0 and int(vc2[untouched].abs().sum().item()) == 0
