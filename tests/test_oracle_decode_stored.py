"""Pins for oracle.attention.paged_decode_stored, the decode oracle on caches
kept in their storage format (the one the GPU parity tests, the smoke check
and the benchmark's CPU baseline call).

It is checked against routes that share none of its steps:
  * the cache is built here in storage format by plain loops (each token's
    row written into the slot its block-table entry names), and decoded here
    with torch's own float8_e4m3fn -> float64 conversion times the scale of
    that tensor (K with k_scale, V with v_scale), not with oracle.fp8;
  * the reference is torch's scaled_dot_product_attention in fp64 on the
    unpaged, decoded K/V of each sequence, with every query head of a group
    reading its kv head through repeat_interleave ("5.KV Cache 管理 &
    PagedAttention", question 7);
  * for 32- and 16-bit storage, where decoding is exact, the result must
    equal the plain-definition oracle O1 (already pinned) bit for bit.
Cases: f32 / f16 / bf16 storage, fp8 codes with k_scale != v_scale (so a
swapped or shared scale shows), GQA and MHA groups, a zero-length sequence
(zero row), and a `pairs` subset (the other rows stay NaN).
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A

_TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _stored_case(seed, lens, Hq, Hkv, D, bs, kind):
    """A shuffled pool in storage format plus the tokens it holds.  fp8
    caches are uint8 codes drawn from the finite codes; the rest are normals
    rounded to the storage dtype.  Unused slots are poisoned (NaN, or the
    fp8 NaN code)."""
    rng = np.random.default_rng(seed)
    B = len(lens)
    need = [-(-L // bs) for L in lens]
    N = sum(need) + 3
    perm = rng.permutation(N)
    tables = np.full((B, max(max(need), 1)), -1, dtype=np.int32)
    cur = 0
    for b in range(B):
        tables[b, :need[b]] = perm[cur:cur + need[b]]
        cur += need[b]
    if kind == "fp8":
        kc = torch.full((N, bs, Hkv, D), 0x7F, dtype=torch.uint8)
    else:
        kc = torch.full((N, bs, Hkv, D), float("nan"), dtype=_TORCH[kind])
    vc = kc.clone()
    toks_k, toks_v = [], []
    for b in range(B):
        if kind == "fp8":
            finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
            tk = torch.from_numpy(rng.choice(finite, size=(lens[b], Hkv, D)))
            tv = torch.from_numpy(rng.choice(finite, size=(lens[b], Hkv, D)))
        else:
            tk = torch.from_numpy(rng.standard_normal((lens[b], Hkv, D))).to(_TORCH[kind])
            tv = torch.from_numpy(rng.standard_normal((lens[b], Hkv, D))).to(_TORCH[kind])
        for t in range(lens[b]):
            blk = int(tables[b, t // bs])
            kc[blk, t % bs] = tk[t]
            vc[blk, t % bs] = tv[t]
        toks_k.append(tk)
        toks_v.append(tv)
    q = torch.from_numpy(rng.standard_normal((B, Hq, D))).to(
        torch.bfloat16 if kind == "fp8" else _TORCH[kind])
    return q, kc, vc, tables, np.array(lens, dtype=np.int32), toks_k, toks_v


def _decode_by_hand(t, kind, scale):
    """Stored values -> fp64: exact widening, or fp8 codes through torch's
    float8_e4m3fn type, times the tensor's scale."""
    if kind == "fp8":
        return t.view(torch.float8_e4m3fn).to(torch.float64) * scale
    return t.to(torch.float64)


def _sdpa_ref(q, toks_k, toks_v, kind, k_scale, v_scale, Hq, Hkv, scale):
    out = np.zeros((q.shape[0], Hq, q.shape[2]))
    for b in range(q.shape[0]):
        if toks_k[b].shape[0] == 0:
            continue
        K = _decode_by_hand(toks_k[b], kind, k_scale).permute(1, 0, 2)   # [Hkv, L, D]
        V = _decode_by_hand(toks_v[b], kind, v_scale).permute(1, 0, 2)
        K = K.repeat_interleave(Hq // Hkv, dim=0)
        V = V.repeat_interleave(Hq // Hkv, dim=0)
        Q = q[b].to(torch.float64)[:, None, :]
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)
        out[b] = o[:, 0, :].numpy()
    return out


@pytest.mark.parametrize("kind", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("heads", [(8, 2), (4, 4)])
def test_exact_storage_matches_o1_bitwise_and_sdpa(kind, heads):
    Hq, Hkv = heads
    D, bs = 16, 16
    q, kc, vc, tab, L, tk, tv = _stored_case(31, [37, 16, 1, 70], Hq, Hkv, D, bs, kind)
    scale = 1 / math.sqrt(D)
    got = A.paged_decode_stored(q, kc, vc, kind, 1.0, 1.0, tab, L, scale, bs)
    o1 = A.paged_decode(q.to(torch.float64).numpy(), kc.to(torch.float64).numpy(),
                        vc.to(torch.float64).numpy(), tab, L, scale, bs)
    assert np.array_equal(got, o1)
    ref = _sdpa_ref(q, tk, tv, kind, 1.0, 1.0, Hq, Hkv, scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("heads", [(8, 2), (4, 1)])
def test_fp8_codes_with_distinct_scales(heads):
    Hq, Hkv = heads
    D, bs = 16, 32
    q, kc, vc, tab, L, tk, tv = _stored_case(32, [45, 64, 3], Hq, Hkv, D, bs, "fp8")
    k_scale, v_scale = 0.0213, 1.7
    scale = 1 / math.sqrt(D)
    got = A.paged_decode_stored(q, kc, vc, "fp8", k_scale, v_scale, tab, L, scale, bs)
    ref = _sdpa_ref(q, tk, tv, "fp8", k_scale, v_scale, Hq, Hkv, scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # the scales matter: swapping them changes the answer well past rounding
    swapped = _sdpa_ref(q, tk, tv, "fp8", v_scale, k_scale, Hq, Hkv, scale)
    assert np.abs(swapped - ref).max() > 1e-3


def test_zero_length_row_and_pairs_subset():
    Hq, Hkv, D, bs = 8, 2, 16, 16
    q, kc, vc, tab, L, tk, tv = _stored_case(33, [20, 0, 33], Hq, Hkv, D, bs, "bf16")
    scale = 0.3
    full = A.paged_decode_stored(q, kc, vc, "bf16", 1.0, 1.0, tab, L, scale, bs)
    assert np.array_equal(full[1], np.zeros((Hq, D)))
    assert np.all(np.isfinite(full))
    ref = _sdpa_ref(q, tk, tv, "bf16", 1.0, 1.0, Hq, Hkv, scale)
    np.testing.assert_allclose(full, ref, rtol=1e-12, atol=1e-13)
    pairs = [(0, 7), (2, 0), (2, 5), (1, 3)]
    sub = A.paged_decode_stored(q, kc, vc, "bf16", 1.0, 1.0, tab, L, scale, bs, pairs)
    want = np.zeros((3, Hq), dtype=bool)
    for b, h in pairs:
        want[b, h] = True
        assert np.array_equal(sub[b, h], full[b, h])
    assert np.all(np.isnan(sub[~want]))


def fp8_pin():
    """The fp8 case above as a callable, for the mutant tests."""
    test_fp8_codes_with_distinct_scales((8, 2))


def gqa_pin():
    test_exact_storage_matches_o1_bitwise_and_sdpa("bf16", (8, 2))


def subset_pin():
    test_zero_length_row_and_pairs_subset()
