"""Pins for oracle.allocator: the page's allocation order and error cases,
and conservation / reference-count invariants over random operations."""

import numpy as np
import pytest

from oracle.allocator import BadBlock, OutOfBlocks, RefCountAllocator, SequenceManager


def test_lifo_order_and_exhaustion():
    a = RefCountAllocator(4)
    assert [a.allocate() for _ in range(4)] == [3, 2, 1, 0]     # pop from the end
    with pytest.raises(OutOfBlocks):
        a.allocate()
    a.decref(2)
    a.decref(0)
    assert a.allocate() == 0                                     # last freed first


def test_bad_ids_and_underflow():
    a = RefCountAllocator(3)
    with pytest.raises(BadBlock):
        a.decref(3)
    with pytest.raises(BadBlock):
        a.incref(-1)
    b = a.allocate()
    a.decref(b)
    with pytest.raises(BadBlock):
        a.decref(b)                                              # double free
    with pytest.raises(BadBlock):
        a.incref(b)


def test_free_order():
    a = RefCountAllocator(5, free_order=[4, 0, 3, 1, 2])
    assert [a.allocate() for _ in range(5)] == [2, 1, 3, 0, 4]
    with pytest.raises(ValueError):
        RefCountAllocator(3, free_order=[0, 0, 1])


def _check_invariants(a, m):
    held = {}
    for t in m.tables.values():
        for b in t:
            held[b] = held.get(b, 0) + 1
    for b in range(a.n):
        assert a.ref[b] == held.get(b, 0)
    assert a.num_free() + len(held) == a.n
    assert sorted(a.free) == sorted(set(range(a.n)) - set(held))
    for s, t in m.tables.items():
        assert len(t) == -(-m.lens[s] // m.bs) or (len(t) >= -(-m.lens[s] // m.bs))


def test_random_sequences_conserve_blocks():
    rng = np.random.default_rng(0)
    for trial in range(20):
        a = RefCountAllocator(40)
        m = SequenceManager(a, 4)
        nxt = 0
        for _ in range(400):
            op = rng.integers(0, 4)
            try:
                if op == 0 or not m.tables:
                    m.add(nxt); nxt += 1
                elif op == 1:
                    s = int(rng.choice(list(m.tables)))
                    slot, cs, cd = m.append(s)
                    L = m.lens[s] - 1
                    assert slot == m.tables[s][L // 4] * 4 + L % 4
                    if cs >= 0:
                        assert a.refcount(cd) == 1
                elif op == 2:
                    s = int(rng.choice(list(m.tables)))
                    m.fork(s, nxt); nxt += 1
                else:
                    s = int(rng.choice(list(m.tables)))
                    m.free(s)
            except OutOfBlocks:
                pass
            _check_invariants(a, m)


def test_cow_on_shared_partial_block():
    a = RefCountAllocator(8)
    m = SequenceManager(a, 4)
    m.add(0)
    for _ in range(6):
        m.append(0)                      # blocks [7, 6], last one half full
    m.fork(0, 1)
    assert a.refcount(7) == 2 and a.refcount(6) == 2
    slot, src, dst = m.append(1)         # writes into shared block 6 -> copy
    assert (src, dst) == (6, 5) and slot == 5 * 4 + 2
    assert m.tables[1] == [7, 5] and m.tables[0] == [7, 6]
    assert a.refcount(6) == 1 and a.refcount(5) == 1
    slot, src, dst = m.append(0)         # parent's block 6 is private again
    assert (src, dst) == (-1, -1) and slot == 6 * 4 + 2


def test_shared_prefix_refcounts():
    a = RefCountAllocator(16)
    prefix = [a.allocate() for _ in range(2)]     # 2 full blocks of 4
    m = SequenceManager(a, 4)
    for s in range(3):
        m.add(s, prefix, 8)
    assert [a.refcount(b) for b in prefix] == [4, 4]
    slot, src, dst = m.append(0)                   # position 8: new private block
    assert src == -1 and m.tables[0][:2] == prefix and len(m.tables[0]) == 3
    for s in range(3):
        m.free(s)
    assert [a.refcount(b) for b in prefix] == [1, 1]
