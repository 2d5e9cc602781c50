"""Pins for oracle.prefill (O5, causal multi-token attention over the cache).

Independent routes: torch's scaled_dot_product_attention in fp64 (is_causal
for whole prompts, an end-aligned boolean mask for chunks), the decode
oracle for one new token, a pure-Python brute force on tiny shapes, the
closed form of the first row, whole-prompt vs chunked consistency, block
permutation invariance and NaN poison in slots no sequence owns."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import prefill as P
from tests.test_oracle_attention import _page


def _case(seed, lens, news, Hq, Hkv, D, bs):
    """Dense per-sequence K/V of lens[b] tokens, paged; news[b] query rows."""
    rng = np.random.default_rng(seed)
    dk = [rng.standard_normal((L, Hkv, D)) for L in lens]
    dv = [rng.standard_normal((L, Hkv, D)) for L in lens]
    qsl = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = rng.standard_normal((int(qsl[-1]), Hq, D))
    kc, vc, tab = _page(rng, dk, dv, bs)
    return q, dk, dv, kc, vc, tab, np.array(lens, dtype=np.int32), qsl


def _sdpa_rows(q_rows, K, V, Hq, Hkv, scale, causal=False, mask=None):
    """q_rows [n, Hq, D]; K, V [L, Hkv, D] -> [n, Hq, D] via torch fp64."""
    Q = torch.from_numpy(q_rows).permute(1, 0, 2)                # [Hq, n, D]
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(
        Q, Kt, Vt, attn_mask=m, is_causal=causal, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (6, 1)])
def test_whole_prompt_matches_sdpa_causal(Hq, Hkv):
    lens = [1, 17, 40, 16]
    q, dk, dv, kc, vc, tab, sl, qsl = _case(1, lens, lens, Hq, Hkv, 16, 8)
    scale = 1 / math.sqrt(16)
    out = P.paged_prefill(q, kc, vc, tab, sl, qsl, scale, 8)
    for b, L in enumerate(lens):
        ref = _sdpa_rows(q[qsl[b]:qsl[b + 1]], dk[b], dv[b], Hq, Hkv, scale, causal=True)
        np.testing.assert_allclose(out[qsl[b]:qsl[b + 1]], ref, rtol=0, atol=1e-12)


def test_chunk_matches_sdpa_end_aligned_mask():
    lens, news = [37, 64, 5, 20], [9, 64, 1, 3]
    Hq, Hkv, D, bs = 4, 2, 8, 16
    q, dk, dv, kc, vc, tab, sl, qsl = _case(2, lens, news, Hq, Hkv, D, bs)
    out = P.paged_prefill(q, kc, vc, tab, sl, qsl, 0.3, bs)
    for b, (L, n) in enumerate(zip(lens, news)):
        # row i may see key t when t - (L - n) <= i: the causal diagonal
        # shifted to the end of the sequence
        allowed = np.tril(np.ones((n, L), dtype=bool), k=L - n)
        ref = _sdpa_rows(q[qsl[b]:qsl[b + 1]], dk[b], dv[b], Hq, Hkv, 0.3, mask=allowed)
        np.testing.assert_allclose(out[qsl[b]:qsl[b + 1]], ref, rtol=0, atol=1e-12)


def test_one_new_token_is_decode():
    lens = [1, 15, 33, 70]
    Hq, Hkv, D, bs = 8, 2, 16, 16
    q, dk, dv, kc, vc, tab, sl, qsl = _case(3, lens, [1] * 4, Hq, Hkv, D, bs)
    out = P.paged_prefill(q, kc, vc, tab, sl, qsl, 0.25, bs)
    ref = A.paged_decode(q, kc, vc, tab, sl, 0.25, bs)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_chunk_equals_tail_of_whole_prompt():
    """Causality: the last n rows of a whole-prompt prefill are the rows of
    a chunked prefill of those n tokens over the same cached sequence."""
    L, n = 53, 11
    Hq, Hkv, D, bs = 4, 4, 8, 16
    q, dk, dv, kc, vc, tab, sl, qsl = _case(4, [L], [L], Hq, Hkv, D, bs)
    whole = P.paged_prefill(q, kc, vc, tab, sl, qsl, 0.5, bs)
    part = P.paged_prefill(q[L - n:], kc, vc, tab, sl, np.array([0, n]), 0.5, bs)
    np.testing.assert_allclose(part, whole[L - n:], rtol=0, atol=1e-12)


def test_first_row_is_first_value():
    """A prompt's first token attends only to itself: weight 1 on v_0."""
    lens = [30, 2]
    q, dk, dv, kc, vc, tab, sl, qsl = _case(5, lens, lens, 4, 2, 8, 16)
    out = P.paged_prefill(q, kc, vc, tab, sl, qsl, 7.0, 16)
    for b in range(2):
        np.testing.assert_array_equal(out[qsl[b]], np.repeat(dv[b][0], 2, axis=0))


def test_brute_force_tiny():
    lens, news = [5, 3], [3, 3]
    Hq, Hkv, D, bs = 2, 1, 3, 16
    q, dk, dv, kc, vc, tab, sl, qsl = _case(6, lens, news, Hq, Hkv, D, bs)
    out = P.paged_prefill(q, kc, vc, tab, sl, qsl, 0.7, bs)
    for b in range(2):
        for i in range(news[b]):
            pos = lens[b] - news[b] + i
            for h in range(Hq):
                qq = q[qsl[b] + i, h]
                w = [math.exp(0.7 * sum(qq[d] * dk[b][t][0][d] for d in range(D)))
                     for t in range(pos + 1)]
                o = [sum(w[t] * dv[b][t][0][d] for t in range(pos + 1)) / sum(w)
                     for d in range(D)]
                np.testing.assert_allclose(out[qsl[b] + i, h], o, rtol=1e-12)


def test_more_rows_than_tokens_gives_zero_rows():
    # 4 rows over a 2-token sequence: positions -2, -1, 0, 1
    q, dk, dv, kc, vc, tab, sl, qsl = _case(7, [2], [4], 2, 2, 4, 16)
    out = P.paged_prefill(q, kc, vc, tab, sl, qsl, 1.0, 16)
    assert np.all(out[:2] == 0)
    np.testing.assert_array_equal(out[2], dv[0][0])


def test_empty_sequences_and_rows():
    lens, news = [0, 9, 4], [0, 0, 4]
    q, dk, dv, kc, vc, tab, sl, qsl = _case(8, lens, news, 2, 1, 4, 16)
    out = P.paged_prefill(q, kc, vc, tab, sl, qsl, 1.0, 16)
    assert out.shape == (4, 2, 4)
    assert np.all(np.isfinite(out))


def test_block_permutation_and_poison():
    """Same dense K/V paged two different ways (NaN in unowned slots) gives
    the same result."""
    lens, news = [45, 18], [20, 18]
    rng = np.random.default_rng(9)
    dk = [rng.standard_normal((L, 2, 8)) for L in lens]
    dv = [rng.standard_normal((L, 2, 8)) for L in lens]
    q = rng.standard_normal((38, 4, 8))
    qsl = np.array([0, 20, 38])
    sl = np.array(lens)
    r1 = P.paged_prefill(q, *_page(np.random.default_rng(10), dk, dv, 16), sl, qsl, 0.4, 16)
    r2 = P.paged_prefill(q, *_page(np.random.default_rng(11), dk, dv, 16), sl, qsl, 0.4, 16)
    assert np.all(np.isfinite(r1))
    np.testing.assert_array_equal(r1, r2)


def test_rows_subset():
    lens, news = [40, 33], [40, 10]
    q, dk, dv, kc, vc, tab, sl, qsl = _case(12, lens, news, 4, 2, 8, 16)
    full = P.paged_prefill(q, kc, vc, tab, sl, qsl, 0.3, 16)
    rows = [0, 7, 39, 40, 49]
    part = P.paged_prefill(q, kc, vc, tab, sl, qsl, 0.3, 16, rows=rows)
    np.testing.assert_array_equal(part[rows], full[rows])
    assert np.isnan(part[1]).all()


def test_stored_format_matches_fp64_route():
    from oracle import fp8
    lens, news = [33, 16], [5, 16]
    Hq, Hkv, D, bs = 4, 2, 8, 16
    q, dk, dv, kc, vc, tab, sl, qsl = _case(13, lens, news, Hq, Hkv, D, bs)
    kc0, vc0 = np.nan_to_num(kc), np.nan_to_num(vc)
    # bf16 storage: values already bf16 are exact
    kb = torch.from_numpy(kc0).to(torch.bfloat16)
    vb = torch.from_numpy(vc0).to(torch.bfloat16)
    qb = torch.from_numpy(q).to(torch.bfloat16)
    got = P.paged_prefill_stored(qb, kb, vb, "bf16", 1.0, 1.0, tab, sl, qsl, 0.35, bs)
    ref = P.paged_prefill(qb.double().numpy(), kb.double().numpy(), vb.double().numpy(),
                          tab, sl, qsl, 0.35, bs)
    np.testing.assert_array_equal(got, ref)
    # fp8 storage: codes times scale
    codes_k = torch.from_numpy(fp8.quantize(kc0, 0.05))
    codes_v = torch.from_numpy(fp8.quantize(vc0, 0.07))
    got = P.paged_prefill_stored(qb, codes_k, codes_v, "fp8", 0.05, 0.07, tab, sl, qsl, 0.35, bs)
    ref = P.paged_prefill(qb.double().numpy(), fp8.decode(codes_k.numpy(), 0.05),
                          fp8.decode(codes_v.numpy(), 0.07), tab, sl, qsl, 0.35, bs)
    np.testing.assert_array_equal(got, ref)


def test_bad_query_start_loc():
    q, dk, dv, kc, vc, tab, sl, qsl = _case(14, [4], [4], 2, 1, 4, 16)
    with pytest.raises(ValueError):
        P.paged_prefill(q, kc, vc, tab, sl, np.array([0, 3]), 1.0, 16)
    with pytest.raises(ValueError):
        P.paged_prefill(q, kc, vc, tab, sl, np.array([1, 4]), 1.0, 16)
