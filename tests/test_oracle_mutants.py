"""Plant plausible mistakes in the oracle (on the CPU) and check that the
pins catch each one.  This shows the pins constrain the oracle rather than
restate it."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import fp8
from tests import test_oracle_attention as TA
from tests import test_oracle_fp8 as TF


def _sdpa_pin():
    q, dk, dv, kc, vc, tab, L = TA._case(21, [1, 17, 40], 8, 2, 16, 16)
    ours = A.paged_decode(q, kc, vc, tab, L, 0.25, 16)
    ref = TA._sdpa(q, dk, dv, 8, 2, 0.25)
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-13)


def _online_pin():
    q, dk, dv, kc, vc, tab, L = TA._case(22, [100], 2, 1, 16, 16)
    o1 = A.paged_decode(q, kc, vc, tab, L, 0.3, 16)
    got = A.online_decode_one(q[0, 0], kc, vc, tab[0], 100, 0.3, 16, 0)
    np.testing.assert_allclose(got, o1[0, 0], rtol=1e-12, atol=1e-13)


def _merge_pin():
    q, dk, dv, kc, vc, tab, L = TA._case(23, [300], 1, 1, 8, 16)
    o1 = A.paged_decode(q, kc, vc, tab, L, 0.3, 16)
    got = A.partitioned_decode_one(q[0, 0], dk[0][:, 0], dv[0][:, 0], 0.3,
                                   A.split_points(300, 64))
    np.testing.assert_allclose(got, o1[0, 0], rtol=1e-12, atol=1e-13)


def _wrong_kv_head(h, g):
    return h % 2            # interleaved instead of grouped


def _wrong_address(table_row, t, bs):
    t = np.asarray(t, dtype=np.int64)
    return np.asarray(table_row)[t // bs], (t + 1) % bs


def _no_scale(q, K, V, scale):
    s = K @ q
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def _transposed_scores(q, K, V, scale):
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    return (w @ V[::-1]) / w.sum()


def _printed_online(q, key_cache, value_cache, table_row, L, scale, bs, kvh):
    # the listing's update, applied literally: acc *= l_rescaled * alpha
    m, l, acc = -np.inf, 0.0, np.zeros(q.shape[0])
    for i in range(-(-L // bs)):
        phys = int(table_row[i]); valid = min(bs, L - i * bs)
        s = scale * (key_cache[phys, :valid, kvh] @ q)
        m_new = max(m, float(s.max()))
        l = l * math.exp(m - m_new)
        p = np.exp(s - m_new)
        acc = acc * l * math.exp(m - m_new) + p @ value_cache[phys, :valid, kvh]
        l += p.sum(); m = m_new
    return acc / l


def _unweighted_merge(triples):
    M = max(t[0] for t in triples)
    return sum(t[2] * np.exp(t[0] - M) for t in triples) / len(triples)


@pytest.mark.parametrize("target,attr,mutant,pin", [
    (A, "kv_head_for", _wrong_kv_head, _sdpa_pin),
    (A, "token_address", _wrong_address, _sdpa_pin),
    (A, "softmax_attend", _no_scale, _sdpa_pin),
    (A, "softmax_attend", _transposed_scores, _sdpa_pin),
    (A, "online_decode_one", _printed_online, _online_pin),
    (A, "merge_triples", _unweighted_merge, _merge_pin),
])
def test_attention_mutants_are_caught(monkeypatch, target, attr, mutant, pin):
    pin()                                   # passes on the real oracle
    monkeypatch.setattr(target, attr, mutant)
    with pytest.raises((AssertionError, IndexError)):
        pin()


def _ties_away(y):
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    pos = fp8._POS
    hi = np.minimum(np.searchsorted(pos, a), 0x7E)
    lo = np.maximum(hi - 1, 0)
    code = np.where(np.abs(pos[hi] - a) <= np.abs(a - pos[lo]), hi, lo)
    code = np.where(a >= 448, 0x7E, code)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


_REAL_TABLE = fp8.decode_table


def _bias8_table():
    return _REAL_TABLE() / 2.0


def test_fp8_round_mutant_is_caught(monkeypatch):
    TF.test_round_matches_torch_on_edges()
    monkeypatch.setattr(fp8, "round_to_e4m3", _ties_away)
    with pytest.raises(AssertionError):
        TF.test_round_matches_torch_on_edges()


def test_fp8_table_mutant_is_caught(monkeypatch):
    monkeypatch.setattr(fp8, "decode_table", _bias8_table)
    with pytest.raises(AssertionError):
        TF.test_decode_table_matches_torch()


def test_prefix_cache_mutants_are_caught(monkeypatch):
    """Keying a block by its own tokens only (content hash, no history), or
    matching without taking references, fails the prefix-cache pins."""
    from oracle import prefix_cache as PC
    from tests import test_prefix_cache as TP

    TP.test_same_block_after_other_history_does_not_match()
    TP.test_page_example_block_table()

    def own_tokens(self, tokens, count):
        t = tuple(int(x) for x in tokens)
        return [t[i * self.bs:(i + 1) * self.bs] for i in range(count)]

    with monkeypatch.context() as mp:
        mp.setattr(PC.PrefixCacheModel, "_prefixes", own_tokens)
        with pytest.raises(AssertionError):
            TP.test_same_block_after_other_history_does_not_match()

    real_match = PC.PrefixCacheModel.match

    def match_without_refs(self, tokens, max_blocks=None):
        out = real_match(self, tokens, max_blocks)
        for b in out:
            self.alloc.decref(b)
        return out

    with monkeypatch.context() as mp:
        mp.setattr(PC.PrefixCacheModel, "match", match_without_refs)
        with pytest.raises(AssertionError):
            TP.test_page_example_block_table()


def _top_left_positions(n, L):
    return np.arange(n, dtype=np.int64)          # mask not shifted to the end


def _late_positions(n, L):
    return np.arange(n, dtype=np.int64) + (L - n) + 1


def _strict_causal(Q, K, V, pos, scale):
    return _real_causal(Q, K, V, pos - 1, scale)  # a row misses its own key


def _unmasked(Q, K, V, pos, scale):
    return _real_causal(Q, K, V, np.full_like(pos, K.shape[0]), scale)


from oracle import prefill as PF  # noqa: E402
from tests import test_oracle_prefill as TPF  # noqa: E402

_real_causal = PF.causal_attend


@pytest.mark.parametrize("attr,mutant", [
    ("row_positions", _top_left_positions),
    ("row_positions", _late_positions),
    ("causal_attend", _strict_causal),
    ("causal_attend", _unmasked),
])
def test_prefill_mutants_are_caught(monkeypatch, attr, mutant):
    """Each planted mask mistake fails at least one prefill pin."""
    pins = [TPF.test_chunk_matches_sdpa_end_aligned_mask,
            lambda: TPF.test_whole_prompt_matches_sdpa_causal(8, 2),
            TPF.test_first_row_is_first_value,
            TPF.test_one_new_token_is_decode]
    for pin in pins:
        pin()
    monkeypatch.setattr(PF, attr, mutant)
    failed = 0
    for pin in pins:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            failed += 1
    assert failed >= 1


# --- the storage-format decode oracle (paged_decode_stored) -----------------

from oracle import cache_write as OW  # noqa: E402
from tests import test_oracle_decode_stored as TS  # noqa: E402

_real_stored = A.paged_decode_stored


def _swapped_scales(query, kc, vc, kind, k_scale, v_scale, *rest, **kw):
    return _real_stored(query, kc, vc, kind, v_scale, k_scale, *rest, **kw)


def _k_scale_on_both(query, kc, vc, kind, k_scale, v_scale, *rest, **kw):
    return _real_stored(query, kc, vc, kind, k_scale, k_scale, *rest, **kw)


def _pairs_ignored(*args, **kw):
    if len(args) > 10:
        args = args[:10]
    kw.pop("pairs", None)
    return _real_stored(*args, **kw)


def _no_dequant_scale(t, kind, scale=1.0):
    from oracle import fp8 as F
    if kind == "fp8":
        return F.decode(t.numpy(), 1.0)
    return t.to(torch.float64).numpy()


@pytest.mark.parametrize("patch,pin", [
    ((A, "paged_decode_stored", _swapped_scales), TS.fp8_pin),
    ((A, "paged_decode_stored", _k_scale_on_both), TS.fp8_pin),
    ((A, "paged_decode_stored", _pairs_ignored), TS.subset_pin),
    ((A, "kv_head_for", _wrong_kv_head), TS.gqa_pin),
    ((OW, "to_f64", _no_dequant_scale), TS.fp8_pin),
])
def test_stored_decode_mutants_are_caught(monkeypatch, patch, pin):
    """Scales swapped, V dequantised with K's scale, the scale dropped, the
    pairs subset ignored, interleaved kv heads: each fails a pin of
    paged_decode_stored."""
    pin()
    target, attr, mutant = patch
    monkeypatch.setattr(target, attr, mutant)
    with pytest.raises((AssertionError, IndexError)):
        pin()
