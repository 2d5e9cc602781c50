"""Pins for oracle.attention (O1 plain definition, O2 online / partitioned).

Independent routes: torch's scaled_dot_product_attention in fp64 on the
unpaged K/V; a pure-Python brute force on tiny shapes; closed forms; block
permutation invariance; NaN poison in slots no sequence owns."""

import itertools
import math

import numpy as np
import pytest
import torch

from oracle import attention as A


def _page(rng, dense_k, dense_v, bs, extra_blocks=2, poison=True):
    """Scatter per-sequence dense K/V ([L_b, Hkv, D]) into a shuffled pool."""
    B = len(dense_k)
    Hkv, D = dense_k[0].shape[1:]
    need = [-(-len(k) // bs) for k in dense_k]
    N = sum(need) + extra_blocks
    perm = rng.permutation(N)
    fill = np.nan if poison else 0.0
    kc = np.full((N, bs, Hkv, D), fill)
    vc = np.full((N, bs, Hkv, D), fill)
    tables = np.full((B, max(max(need), 1)), -1, dtype=np.int32)
    cur = 0
    for b in range(B):
        ids = perm[cur:cur + need[b]]
        cur += need[b]
        tables[b, :need[b]] = ids
        for t in range(len(dense_k[b])):
            kc[ids[t // bs], t % bs] = dense_k[b][t]
            vc[ids[t // bs], t % bs] = dense_v[b][t]
    return kc, vc, tables


def _case(seed, lens, Hq, Hkv, D, bs):
    rng = np.random.default_rng(seed)
    dk = [rng.standard_normal((L, Hkv, D)) for L in lens]
    dv = [rng.standard_normal((L, Hkv, D)) for L in lens]
    q = rng.standard_normal((len(lens), Hq, D))
    kc, vc, tab = _page(rng, dk, dv, bs)
    return q, dk, dv, kc, vc, tab, np.array(lens, dtype=np.int32)


def _sdpa(q, dk, dv, Hq, Hkv, scale):
    out = []
    for b in range(len(dk)):
        K = torch.from_numpy(dk[b]).permute(1, 0, 2)           # [Hkv, L, D]
        V = torch.from_numpy(dv[b]).permute(1, 0, 2)
        K = K.repeat_interleave(Hq // Hkv, dim=0)
        V = V.repeat_interleave(Hq // Hkv, dim=0)
        Q = torch.from_numpy(q[b])[:, None, :]                  # [Hq, 1, D]
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)
        out.append(o[:, 0, :].numpy())
    return np.stack(out)


@pytest.mark.parametrize("lens,Hq,Hkv,D,bs", [
    ([100], 4, 4, 64, 16),
    ([1, 17, 33, 64], 8, 2, 32, 16),
    ([5, 40, 100], 6, 1, 16, 32),
    ([77, 3], 4, 4, 8, 4),
])
def test_o1_matches_sdpa(lens, Hq, Hkv, D, bs):
    q, dk, dv, kc, vc, tab, L = _case(11, lens, Hq, Hkv, D, bs)
    scale = 1 / math.sqrt(D)
    ours = A.paged_decode(q, kc, vc, tab, L, scale, bs)
    fast = A.paged_decode_fast(q, kc, vc, tab, L, scale, bs)
    ref = _sdpa(q, dk, dv, Hq, Hkv, scale)
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(fast, ref, rtol=1e-12, atol=1e-13)


def _brute(q, dk, dv, Hq, Hkv, scale):
    """Pure-Python loops over the unpaged tokens."""
    B = len(dk)
    D = len(q[0][0])
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            kv = h * Hkv // Hq
            s = []
            for t in range(len(dk[b])):
                s.append(scale * sum(float(q[b][h][d]) * float(dk[b][t][kv][d]) for d in range(D)))
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = sum(w)
            for d in range(D):
                out[b][h][d] = sum(w[t] * float(dv[b][t][kv][d]) for t in range(len(w))) / z
    return np.array(out)


@pytest.mark.parametrize("bs", [1, 2, 3, 4])
@pytest.mark.parametrize("heads", [(1, 1), (2, 1), (4, 2)])
@pytest.mark.parametrize("D", [1, 2, 4])
def test_o1_brute_force_tiny(bs, heads, D):
    Hq, Hkv = heads
    rng = np.random.default_rng(bs * 100 + Hq * 10 + D)
    for L in range(1, 10):
        dk = [rng.standard_normal((L, Hkv, D))]
        dv = [rng.standard_normal((L, Hkv, D))]
        q = rng.standard_normal((1, Hq, D))
        ref = _brute(q, dk, dv, Hq, Hkv, 0.7)
        need = -(-L // bs)
        N = need + 2
        # every injective table into the pool when small, else 50 random ones
        if N <= 7:
            tables = list(itertools.permutations(range(N), need))
        else:
            tables = [tuple(rng.permutation(N)[:need]) for _ in range(50)]
        for ids in tables:
            kc = np.full((N, bs, Hkv, D), np.nan)
            vc = np.full((N, bs, Hkv, D), np.nan)
            for t in range(L):
                kc[ids[t // bs], t % bs] = dk[0][t]
                vc[ids[t // bs], t % bs] = dv[0][t]
            tab = np.array([ids], dtype=np.int32)
            got = A.paged_decode(q, kc, vc, tab, np.array([L]), 0.7, bs)
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_closed_forms():
    rng = np.random.default_rng(3)
    Hq, Hkv, D, bs = 4, 2, 16, 16
    # one token: output is that token's value row, exactly
    q, dk, dv, kc, vc, tab, L = _case(5, [1, 1], Hq, Hkv, D, bs)
    out = A.paged_decode(q, kc, vc, tab, L, 0.25, bs)
    for b in range(2):
        for h in range(Hq):
            assert np.array_equal(out[b, h], dv[b][0][h // (Hq // Hkv)])
    # zero query: uniform weights -> mean of the values
    q, dk, dv, kc, vc, tab, L = _case(6, [37], Hq, Hkv, D, bs)
    out = A.paged_decode(np.zeros_like(q), kc, vc, tab, L, 0.25, bs)
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], dv[0][:, h // 2].mean(axis=0), rtol=1e-13, atol=1e-14)
    # constant values: output equals that constant for any scores
    c = rng.standard_normal(D)
    dv2 = [np.broadcast_to(c, (37, Hkv, D)).copy()]
    kc2, vc2, tab2 = _page(rng, dk, dv2, bs)
    out = A.paged_decode(q, kc2, vc2, tab2, L, 0.25, bs)
    np.testing.assert_allclose(out[0], np.broadcast_to(c, (Hq, D)), rtol=1e-13)
    # identical keys: uniform weights again
    dk3 = [np.broadcast_to(dk[0][0], (37, Hkv, D)).copy()]
    kc3, vc3, tab3 = _page(rng, dk3, dv, bs)
    out = A.paged_decode(q, kc3, vc3, tab3, L, 0.25, bs)
    np.testing.assert_allclose(out[0, 0], dv[0][:, 0].mean(axis=0), rtol=1e-12, atol=1e-13)


def test_empty_sequence_gives_zeros():
    q, dk, dv, kc, vc, tab, L = _case(8, [5, 9], 2, 2, 8, 4)
    L = np.array([0, 9], dtype=np.int32)
    out = A.paged_decode(q, kc, vc, tab, L, 0.5, 4)
    assert np.array_equal(out[0], np.zeros((2, 8)))
    assert np.all(np.isfinite(out[1]))


def test_block_permutation_invariance_bit_exact():
    q, dk, dv, kc, vc, tab, L = _case(9, [50, 129, 16], 8, 4, 32, 16)
    base = A.paged_decode(q, kc, vc, tab, L, 0.3, 16)
    rng = np.random.default_rng(10)
    N = kc.shape[0]
    for _ in range(3):
        p = rng.permutation(N)               # physical id i moves to p[i]
        kc2 = np.empty_like(kc); vc2 = np.empty_like(vc)
        kc2[p] = kc; vc2[p] = vc
        tab2 = np.where(tab >= 0, p[np.maximum(tab, 0)], -1).astype(np.int32)
        got = A.paged_decode(q, kc2, vc2, tab2, L, 0.3, 16)
        assert np.array_equal(got, base)


def test_poison_is_never_read():
    q, dk, dv, kc, vc, tab, L = _case(12, [33, 7], 4, 4, 16, 16)
    out = A.paged_decode(q, kc, vc, tab, L, 0.25, 16)
    assert np.all(np.isfinite(out))          # pool is NaN outside valid slots
    assert np.isnan(kc).any()


@pytest.mark.parametrize("part", [1, 16, 512, 7])
def test_o2_partitioned_equals_o1(part):
    q, dk, dv, kc, vc, tab, L = _case(13, [1000, 1, 513], 4, 2, 32, 16)
    o1 = A.paged_decode(q, kc, vc, tab, L, 0.2, 16)
    for b in range(3):
        for h in range(4):
            Kb = dk[b][:, h // 2]
            Vb = dv[b][:, h // 2]
            got = A.partitioned_decode_one(q[b, h], Kb, Vb, 0.2, A.split_points(int(L[b]), part))
            np.testing.assert_allclose(got, o1[b, h], rtol=1e-12, atol=1e-13)


def test_o2_random_split_points_equal_o1():
    rng = np.random.default_rng(14)
    q, dk, dv, kc, vc, tab, L = _case(15, [300], 2, 1, 16, 16)
    o1 = A.paged_decode(q, kc, vc, tab, L, 0.2, 16)
    for _ in range(10):
        cuts = sorted(set(rng.integers(1, 300, size=rng.integers(1, 20)).tolist()))
        got = A.partitioned_decode_one(q[0, 1], dk[0][:, 0], dv[0][:, 0], 0.2, [0] + cuts + [300])
        np.testing.assert_allclose(got, o1[0, 1], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("bs", [16, 32, 5])
def test_o2_online_block_loop_equals_o1(bs):
    q, dk, dv, kc, vc, tab, L = _case(16, [100, 16, 1, 257], 8, 2, 32, bs)
    o1 = A.paged_decode(q, kc, vc, tab, L, 0.2, bs)
    for b in range(4):
        for h in range(8):
            got = A.online_decode_one(q[b, h], kc, vc, tab[b], int(L[b]), 0.2, bs, h // 4)
            np.testing.assert_allclose(got, o1[b, h], rtol=1e-12, atol=1e-13)


def test_page_worked_lookup():
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "block_tables.json")) as f:
        g = json.load(f)
    e = g["token_25_lookup"]
    phys, off = A.token_address(np.array(e["table"]), np.array([e["token"]]), e["block_size"])
    assert (int(phys[0]), int(off[0])) == (e["physical"], e["offset"])
    e = g["table_68_tokens"]
    phys, off = A.token_address(np.array(e["physical"]), np.arange(e["num_tokens"]), e["block_size"])
    for i, (first, last) in enumerate(e["block_contents_first_last"]):
        assert set(phys[first:last + 1].tolist()) == {e["physical"][i]}
        assert list(off[first:last + 1]) == list(range(last - first + 1))
