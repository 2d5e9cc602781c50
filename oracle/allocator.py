"""Python model of the host-side block allocator and sequence block manager.

Allocator ([P2] question 9): a stack of free physical block ids; allocating
pops the most recently pushed id (the initial stack is 0..N-1, so the first
allocation returns N-1, or the caller supplies the initial order), an empty
stack is an out-of-blocks error (9.1), and with sharing each block carries a
reference count: allocation sets it to 1, sharing increments it, releasing
decrements it and the block returns to the stack at zero (9.4).  Readings
where the page has no guard: incref or decref of a block that is not
allocated, and any id outside [0, N), are errors.

Sequence manager: a sequence owns a list of physical ids (its block table)
and a length.  Appending a token allocates a new block when the length is a
multiple of the block size ([P2] question 12, append_token), and returns the
slot block * bs + offset the new token goes to.  Forking shares every block
of the parent with one more reference each; appending into a shared block
that still has free slots first copies it to a fresh block (copy-on-write,
[P2] question 18, COWBlockManager.write_token).  A shared prefix is attached
by incref'ing existing blocks ([P2] question 20, allocate_with_prefix).

Pins (tests/test_oracle_allocator.py): the page's allocation order and error
cases, conservation (free + allocated == N) and reference counts equal to the
number of tables that hold each block, over random operation sequences.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple


class OutOfBlocks(Exception):
    pass


class BadBlock(Exception):
    pass


class RefCountAllocator:
    def __init__(self, num_blocks: int, free_order: Optional[Sequence[int]] = None):
        self.n = int(num_blocks)
        if free_order is None:
            self.free = list(range(self.n))
        else:
            self.free = [int(x) for x in free_order]
            if sorted(self.free) != list(range(self.n)):
                raise ValueError("free_order must be a permutation of 0..N-1")
        self.ref = [0] * self.n

    def allocate(self) -> int:
        if not self.free:
            raise OutOfBlocks(f"all {self.n} blocks are in use")
        blk = self.free.pop()
        self.ref[blk] = 1
        return blk

    def _check(self, blk: int) -> None:
        if blk < 0 or blk >= self.n:
            raise BadBlock(f"block {blk} outside [0, {self.n})")
        if self.ref[blk] == 0:
            raise BadBlock(f"block {blk} is not allocated")

    def incref(self, blk: int) -> None:
        self._check(blk)
        self.ref[blk] += 1

    def decref(self, blk: int) -> None:
        self._check(blk)
        self.ref[blk] -= 1
        if self.ref[blk] == 0:
            self.free.append(blk)

    def num_free(self) -> int:
        return len(self.free)

    def refcount(self, blk: int) -> int:
        if blk < 0 or blk >= self.n:
            raise BadBlock(f"block {blk} outside [0, {self.n})")
        return self.ref[blk]


class SequenceManager:
    def __init__(self, alloc: RefCountAllocator, block_size: int):
        self.a = alloc
        self.bs = int(block_size)
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}

    def add(self, seq: int, shared_blocks: Sequence[int] = (), shared_tokens: int = 0) -> None:
        if seq in self.tables:
            raise ValueError("sequence exists")
        if shared_tokens > len(shared_blocks) * self.bs:
            raise ValueError("shared tokens exceed the shared blocks")
        for b in shared_blocks:
            self.a._check(int(b))
        for b in shared_blocks:
            self.a.incref(int(b))
        self.tables[seq] = [int(b) for b in shared_blocks]
        self.lens[seq] = int(shared_tokens)

    def append(self, seq: int) -> Tuple[int, int, int]:
        """-> (slot, cow_src, cow_dst); cow_* are -1 when no copy is needed."""
        t = self.tables[seq]
        L = self.lens[seq]
        cow_src = cow_dst = -1
        if L % self.bs == 0 and L // self.bs == len(t):
            t.append(self.a.allocate())
        else:
            i = L // self.bs
            blk = t[i]
            if self.a.refcount(blk) > 1:
                new = self.a.allocate()
                self.a.decref(blk)
                t[i] = new
                cow_src, cow_dst = blk, new
        i = L // self.bs
        slot = t[i] * self.bs + L % self.bs
        self.lens[seq] = L + 1
        return slot, cow_src, cow_dst

    def fork(self, parent: int, child: int) -> None:
        if child in self.tables:
            raise ValueError("sequence exists")
        for b in self.tables[parent]:
            self.a.incref(b)
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]

    def free(self, seq: int) -> None:
        for b in self.tables.pop(seq):
            self.a.decref(b)
        del self.lens[seq]
