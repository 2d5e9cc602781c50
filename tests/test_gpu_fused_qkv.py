"""Inputs that are views into a fused QKV projection output: one row per
token of [Hq + 2 Hkv, D] values, so the query, key and value of a token sit
(Hq + 2 Hkv) * D elements apart from the next token's, and outputs written
into a wider buffer.  The decode step (write the new token's K/V, attend)
and a prefill chunk run on these strided views and must give the bits the
same calls give on contiguous copies, and the oracle's values."""

import numpy as np
import pytest
import torch

import paged_kv_cache_462_amd as pa
from synth import get_config, make_prefill_rows, make_workload
from synth.generate import shrink
from tests import _gpu as G

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_g8": shrink(get_config("c3"), batch=4, lengths=("list", [1, 17, 300, 1000]), pool_blocks=0),
    "fp8_g4": shrink(get_config("c5"), batch=4, lengths=("list", [1, 33, 260, 900]),
                     shared_prefix_tokens=0, pool_blocks=0),
}


def _fused(q, k, v):
    """[T, Hq + 2 Hkv, D] buffer holding q, k, v per token, and the three
    strided views into it."""
    T, hq, D = q.shape
    hkv = k.shape[1]
    buf = torch.empty((T, hq + 2 * hkv, D), dtype=q.dtype, device=q.device)
    buf[:, :hq] = q
    buf[:, hq:hq + hkv] = k.to(q.dtype)
    buf[:, hq + hkv:] = v.to(q.dtype)
    return buf[:, :hq], buf[:, hq:hq + hkv], buf[:, hq + hkv:]


def _kvd(wl):
    return "fp8" if wl.cfg.kv_dtype == "fp8" else None


def _bits(t):
    return t.contiguous().view(torch.int16)


@pytest.mark.parametrize("name", list(CASES))
def test_decode_step_on_fused_qkv_views(name):
    wl = make_workload(CASES[name], seed=81)
    c = wl.cfg
    assert (wl.new_tok >= 0).all()
    G.say(f"fused qkv decode {name}")
    kc_ref, vc_ref = G.oracle_caches(wl)
    dev = torch.device("cuda:0")
    # the cache holds every token but each sequence's newest one
    d = G.to_device(wl, fill=False)
    ctx_slots = wl.slot_mapping.copy()
    ctx_slots[wl.new_tok] = -1
    pa.reshape_and_cache(d.tok_key, d.tok_value, torch.from_numpy(ctx_slots).to(dev), d.kc, d.vc,
                         k_scale=wl.k_scale, v_scale=wl.v_scale, kv_dtype=_kvd(wl))
    kc0, vc0 = d.kc.clone(), d.vc.clone()
    new_k, new_v = wl.new_key().to(dev), wl.new_value().to(dev)
    new_s = torch.from_numpy(wl.new_slots).to(dev)
    q, k, v = _fused(d.query, new_k, new_v)
    assert q.stride(0) == (c.num_q_heads + 2 * c.num_kv_heads) * c.head_dim
    wide = torch.full((c.batch, 2 * c.num_q_heads, c.head_dim), float("nan"), dtype=q.dtype, device=dev)
    out = wide[:, c.num_q_heads:]
    pa.reshape_and_cache(k, v, new_s, d.kc, d.vc, k_scale=wl.k_scale, v_scale=wl.v_scale,
                         kv_dtype=_kvd(wl))
    ws = torch.empty(max(16, pa.decode_workspace_bytes(c.batch, c.num_q_heads, c.num_kv_heads,
                                                       c.head_dim, c.block_size, wl.max_blocks, 0)),
                     dtype=torch.uint8, device=dev)
    pa.decode(out, q, d.kc, d.vc, d.tables, d.lens, wl.scale, c.block_size, c.num_kv_heads,
              k_scale=wl.k_scale, v_scale=wl.v_scale, kv_dtype=_kvd(wl), workspace=ws)
    torch.cuda.synchronize()
    # the same step on contiguous copies
    kc1, vc1 = kc0, vc0
    pa.reshape_and_cache(k.contiguous(), v.contiguous(), new_s, kc1, vc1, k_scale=wl.k_scale,
                         v_scale=wl.v_scale, kv_dtype=_kvd(wl))
    out1 = torch.empty_like(d.query)
    pa.decode(out1, q.contiguous(), kc1, vc1, d.tables, d.lens, wl.scale, c.block_size,
              c.num_kv_heads, k_scale=wl.k_scale, v_scale=wl.v_scale, kv_dtype=_kvd(wl), workspace=ws)
    torch.cuda.synchronize()
    assert G.caches_equal(d.kc, kc_ref) and G.caches_equal(d.vc, vc_ref)
    assert G.caches_equal(kc1, kc_ref) and G.caches_equal(vc1, vc_ref)
    assert torch.equal(_bits(out), _bits(out1))
    assert bool(torch.isnan(wide[:, :c.num_q_heads].float()).all()), "write outside the output view"
    atol, rtol = G.tol_for(wl)
    G.assert_close(out.contiguous(), G.oracle_decode(wl, kc_ref, vc_ref), atol, rtol,
                   what=f"fused qkv decode {name}")


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_chunk_on_fused_qkv_views(name):
    wl = make_workload(CASES[name], seed=82)
    c = wl.cfg
    news = [min(int(L), n) for L, n in zip(wl.seq_lens, [1, 17, 100, 333])]
    rows = make_prefill_rows(wl, ("list", news), seed=83)
    G.say(f"fused qkv prefill {name}: rows={news}")
    kc_ref, vc_ref = G.oracle_caches(wl)
    dev = torch.device("cuda:0")
    d = G.to_device(wl, fill=False)
    # token-stream indices of the chunk (the last n_b tokens of each sequence)
    starts = np.concatenate([[0], np.cumsum(wl.seq_lens.astype(np.int64))])
    new_idx = np.concatenate([np.arange(starts[b + 1] - news[b], starts[b + 1])
                              for b in range(c.batch)]).astype(np.int64)
    ctx_slots = wl.slot_mapping.copy()
    ctx_slots[new_idx] = -1
    pa.reshape_and_cache(d.tok_key, d.tok_value, torch.from_numpy(ctx_slots).to(dev), d.kc, d.vc,
                         k_scale=wl.k_scale, v_scale=wl.v_scale, kv_dtype=_kvd(wl))
    ni = torch.from_numpy(new_idx).to(dev)
    q, k, v = _fused(rows.query.to(dev), d.tok_key[ni], d.tok_value[ni])
    pa.reshape_and_cache(k, v, d.slots[ni], d.kc, d.vc, k_scale=wl.k_scale, v_scale=wl.v_scale,
                         kv_dtype=_kvd(wl))
    T = rows.num_rows
    wide = torch.full((T, 3 * c.num_q_heads, c.head_dim), float("nan"), dtype=q.dtype, device=dev)
    out = wide[:, c.num_q_heads:2 * c.num_q_heads]
    qsl = torch.from_numpy(rows.query_start_loc).to(dev)
    pa.prefill(out, q, d.kc, d.vc, d.tables, d.lens, qsl, rows.max_query_len, wl.scale,
               c.block_size, c.num_kv_heads, k_scale=wl.k_scale, v_scale=wl.v_scale,
               kv_dtype=_kvd(wl))
    out1 = torch.empty((T, c.num_q_heads, c.head_dim), dtype=q.dtype, device=dev)
    pa.prefill(out1, q.contiguous(), d.kc, d.vc, d.tables, d.lens, qsl, rows.max_query_len,
               wl.scale, c.block_size, c.num_kv_heads, k_scale=wl.k_scale, v_scale=wl.v_scale,
               kv_dtype=_kvd(wl))
    torch.cuda.synchronize()
    assert G.caches_equal(d.kc, kc_ref) and G.caches_equal(d.vc, vc_ref)
    assert torch.equal(_bits(out), _bits(out1))
    assert bool(torch.isnan(wide[:, :c.num_q_heads].float()).all())
    assert bool(torch.isnan(wide[:, 2 * c.num_q_heads:].float()).all())
    atol, rtol = G.tol_for(wl)
    G.assert_close(out.contiguous(), G.oracle_prefill(wl, kc_ref, vc_ref, rows), atol, rtol,
                   what=f"fused qkv prefill {name}")
