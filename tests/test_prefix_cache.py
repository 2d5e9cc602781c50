"""Prefix cache: the oracle model against what the pages fix, and the
library's C++ cache against the model, operation by operation (CPU)."""

import numpy as np
import pytest

import paged_kv_cache_462_amd as pa
from oracle.allocator import BadBlock, RefCountAllocator
from oracle.prefix_cache import PrefixCacheModel

A, B, C, D, E, F, X, Y = range(1, 9)


def _order_for_first(n, firsts):
    """free_order whose first allocations (LIFO) return `firsts` in order."""
    rest = [i for i in range(n) if i not in firsts]
    return rest + list(reversed(firsts))


def _both(n, bs, free_order):
    m_alloc = RefCountAllocator(n, free_order)
    model = PrefixCacheModel(m_alloc, bs)
    c_alloc = pa.BlockAllocator(n, free_order)
    cache = pa.PrefixCache(c_alloc, bs)
    return m_alloc, model, c_alloc, cache


def test_page_example_block_table():
    """[A,B,C,D,E,F] in 2-token blocks, with [A,B] cached in block 7 and
    [C,D] (after [A,B]) in block 3: the lookup finds 7 and 3 and the table
    becomes [7, 3, new]."""
    for side in ("model", "library"):
        m_alloc, model, c_alloc, cache = _both(16, 2, _order_for_first(16, [7, 3]))
        alloc = m_alloc if side == "model" else c_alloc
        pc = model if side == "model" else cache
        first = [alloc.allocate(), alloc.allocate()]
        assert first == [7, 3]
        assert pc.insert([A, B, C, D], first) == 2
        hit = pc.match([A, B, C, D, E, F])
        assert hit == [7, 3]
        table = hit + [alloc.allocate()]       # only [E, F] needs a block
        assert table[:2] == [7, 3] and table[2] not in (7, 3)
        # owner + cache + the matcher
        assert alloc.refcount(7) == 3 and alloc.refcount(3) == 3


def test_same_block_after_other_history_does_not_match():
    for side in ("model", "library"):
        m_alloc, model, c_alloc, cache = _both(16, 2, None)
        alloc = m_alloc if side == "model" else c_alloc
        pc = model if side == "model" else cache
        blocks = [alloc.allocate(), alloc.allocate()]
        pc.insert([A, B, C, D], blocks)
        assert pc.match([X, Y, C, D]) == []      # [C, D] after [X, Y] is another prefix
        # [A, B] again, but after [X, Y]: its K/V differ, so it is a new entry
        other = [alloc.allocate(), alloc.allocate()]
        assert pc.insert([X, Y, A, B], other) == 2
        assert pc.match([X, Y, A, B]) == other
        assert pc.match([A, B, X, Y]) == [blocks[0]]
        assert pc.match([A]) == []               # no full block
        assert pc.match([A, B, C, D, E], max_blocks=1) == [blocks[0]]


def test_release_and_eviction_follow_references():
    """Question 20: a block returns to the pool once nobody references it;
    the cache never releases a block a sequence still holds."""
    for side in ("model", "library"):
        m_alloc, model, c_alloc, cache = _both(8, 2, None)
        alloc = m_alloc if side == "model" else c_alloc
        pc = model if side == "model" else cache
        seq = [alloc.allocate() for _ in range(3)]
        assert pc.insert([A, B, C, D, E, F], seq) == 3
        assert pc.evict(10) == 0                 # the sequence still holds all three
        alloc.decref(seq[2])                     # the sequence drops its last block
        assert pc.evict(10) == 1 and pc.size() == 2
        assert alloc.refcount(seq[2]) == 0
        for b in seq[:2]:
            alloc.decref(b)
        assert pc.evict(1) == 1 and pc.size() == 1   # leaves first: [C,D] before [A,B]
        assert alloc.refcount(seq[1]) == 0 and alloc.refcount(seq[0]) == 1
        assert pc.evict(5) == 1 and pc.size() == 0
        assert (alloc.num_free() if side == "model" else alloc.num_free()) == 8


def test_insert_rejects_free_block():
    m_alloc, model, c_alloc, cache = _both(8, 2, None)
    with pytest.raises(BadBlock):
        model.insert([A, B], [3])
    with pytest.raises(pa.PaError):
        cache.insert([A, B], [3])


@pytest.mark.parametrize("seed", range(12))
def test_library_matches_model(seed):
    rng = np.random.default_rng(seed)
    n, bs = 96, int(rng.choice([1, 2, 4]))
    order = [int(x) for x in rng.permutation(n)]
    m_alloc, model, c_alloc, cache = _both(n, bs, order)
    held = {"m": [], "c": []}          # references the test itself holds
    stems = [list(rng.integers(0, 5, size=int(rng.integers(0, 4 * bs + 1)))) for _ in range(6)]
    for step in range(400):
        op = rng.integers(0, 10)
        if op < 4:      # a new prompt: match, allocate the rest, cache it
            toks = list(stems[rng.integers(len(stems))]) + list(rng.integers(0, 3, size=int(rng.integers(0, 3 * bs + 1))))
            hm = model.match(toks)
            hc = cache.match(toks)
            assert hm == hc, (step, toks)
            need = -(-len(toks) // bs) - len(hm) if toks else 0
            if m_alloc.num_free() < need:
                for b in hm:
                    m_alloc.decref(b)
                    c_alloc.decref(b)
                continue
            new_m = [m_alloc.allocate() for _ in range(need)]
            new_c = [c_alloc.allocate() for _ in range(need)]
            assert new_m == new_c
            table = hm + new_m
            assert model.insert(toks, table) == cache.insert(toks, table)
            held["m"].append(table)
        elif op < 7 and held["m"]:   # a sequence ends: drop its references
            i = int(rng.integers(len(held["m"])))
            for b in held["m"].pop(i):
                m_alloc.decref(b)
                c_alloc.decref(b)
        else:
            k = int(rng.integers(0, 6))
            assert model.evict(k) == cache.evict(k)
        assert model.size() == cache.size()
        assert [m_alloc.refcount(b) for b in range(n)] == [c_alloc.refcount(b) for b in range(n)]
        assert m_alloc.num_free() == c_alloc.num_free()
