"""Python model of the prefix cache (test infrastructure only).

What is modelled: a map from token prefixes to the physical blocks holding
their K/V, block by block ("KV Cache 优化与内存管理深度解析：PagedAttention
原理与实践", `HashBasedCaching`: the prefix lookup walk-through, where
[A,B,C,D,E,F] in 2-token blocks finds blocks 7 and 3 and needs one new
block; "5.KV Cache 管理 & PagedAttention", question 20: match, take
references, allocate the rest, release at zero).  Reading where the pages
offer several keys: block i's key is the whole token prefix through the end
of block i (their prefix-hash option), since a block's K/V depend on every
earlier token.  Here the key is literally that tuple of tokens: no hashing.

Reference counts go through the allocator model: one reference per cached
block for the cache, one more per returned block for whoever matched.  Every
block a match or insert walks past is stamped with the next value of a
counter; eviction releases the least recently stamped entry that has no
cached one-block extension and that nobody else references, repeatedly.

Pins (tests/test_prefix_cache.py): the pages' worked example, the prefix
reading (equal blocks after different histories do not match), reference
counts, and the C++ cache against this model over random operations.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

from .allocator import BadBlock, RefCountAllocator


class PrefixCacheModel:
    def __init__(self, alloc: RefCountAllocator, block_size: int):
        self.alloc = alloc
        self.bs = int(block_size)
        self.entries: Dict[Tuple[int, ...], List[int]] = {}  # prefix -> [block, stamp]
        self.clock = 0

    def _prefixes(self, tokens: Sequence[int], count: int):
        t = tuple(int(x) for x in tokens)
        return [t[:(i + 1) * self.bs] for i in range(count)]

    def match(self, tokens: Sequence[int], max_blocks: Optional[int] = None) -> List[int]:
        full = len(tokens) // self.bs
        limit = full if max_blocks is None else min(full, int(max_blocks))
        out = []
        for key in self._prefixes(tokens, limit):
            if key not in self.entries:
                break
            self.clock += 1
            self.entries[key][1] = self.clock
            out.append(self.entries[key][0])
        for b in out:
            self.alloc.incref(b)
        return out

    def insert(self, tokens: Sequence[int], blocks: Sequence[int]) -> int:
        count = min(len(tokens) // self.bs, len(blocks))
        for i in range(count):
            if self.alloc.refcount(blocks[i]) <= 0:
                raise BadBlock("a block to cache is not allocated")
        added = 0
        for i, key in enumerate(self._prefixes(tokens, count)):
            if key not in self.entries:
                self.alloc.incref(blocks[i])
                self.entries[key] = [int(blocks[i]), 0]
                added += 1
            self.clock += 1
            self.entries[key][1] = self.clock
        return added

    def _has_extension(self, key: Tuple[int, ...]) -> bool:
        n = len(key) + self.bs
        return any(len(k) == n and k[:len(key)] == key for k in self.entries)

    def evict(self, max_blocks: int) -> int:
        freed = 0
        while freed < max_blocks:
            cands = [k for k, (b, _) in self.entries.items()
                     if not self._has_extension(k) and self.alloc.refcount(b) == 1]
            if not cands:
                break
            victim = min(cands, key=lambda k: self.entries[k][1])
            self.alloc.decref(self.entries.pop(victim)[0])
            freed += 1
        return freed

    def size(self) -> int:
        return len(self.entries)
