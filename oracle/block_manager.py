"""Reference block allocator: free pool, block tables, refcounts, fork, CoW.

What the pages fix:
  * KV is cut into fixed-size blocks handed out one at a time from a shared
    physical pool, anywhere in memory ([youngju] "블록 테이블: 논리적으로 연속,
    물리적으로 흩어짐"; [ttlab] "블록과 블록 표").
  * A sequence writes into its current block; when that block is full it takes
    one free block and extends its block table; when a request finishes, the
    blocks nobody else references go back to the free pool ([icarus]
    "Block Table 如何工作").
  * Several sequences may point at the same physical block, counted by a
    reference count; a shared block is copied only when one of them has to
    write into it, i.e. copy-on-write ([icarus] "支持块级共享"; [ttlab]
    "블록을 함께 쓰기").

Readings where the pages leave a choice (each listed in the design notes):
  * Which free block: the free pool is a FIFO queue seeded with a given order;
    allocation pops from the front.  Freed blocks are pushed at the back, the
    sequence's blocks taken from its last logical block to its first (the
    tail-first order [ttlab] "4. 프리픽스 캐시" gives for its cached-block
    queue).
  * Who copies when k sharers write: each writer copies while the block's
    refcount is above one; the last remaining holder writes in place.
  * Running out of blocks fails the whole request and leaves the allocator
    exactly as it was.

Processing is token by token, in the order the text describes, with a
snapshot taken before each request for the all-or-nothing failure.
"""

import copy
from collections import deque


class OutOfBlocks(Exception):
    pass


class BlockManager:
    def __init__(self, num_blocks, block_size, free_order):
        free_order = [int(b) for b in free_order]
        if sorted(free_order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the block ids")
        if block_size < 1:
            raise ValueError("block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.free = deque(free_order)
        self.ref = [0] * self.num_blocks
        self.table = {}
        self.length = {}

    # -- sequences ---------------------------------------------------------
    def add_seq(self, seq):
        if seq in self.table:
            raise KeyError(f"sequence {seq} exists")
        self.table[seq] = []
        self.length[seq] = 0

    def fork(self, parent, child):
        """child shares every block of parent (parallel sampling / beam search)."""
        if parent not in self.table or child in self.table:
            raise KeyError("fork needs an existing parent and a new child")
        self.table[child] = list(self.table[parent])
        self.length[child] = self.length[parent]
        for b in self.table[child]:
            self.ref[b] += 1

    def free_seq(self, seq):
        """Drop a finished sequence; blocks whose count reaches 0 rejoin the pool."""
        blocks = self.table.pop(seq)
        del self.length[seq]
        for b in reversed(blocks):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    # -- growth ------------------------------------------------------------
    def _take_free(self):
        if not self.free:
            raise OutOfBlocks()
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def append_slots(self, seq, n):
        """Reserve slots for the next n tokens of ``seq``.

        Returns (slots, cow_pairs): slot = physical block * block_size + offset
        for each new token in order, and the (source, destination) block pairs
        whose contents must be copied before the new tokens are written.
        Raises OutOfBlocks with no state change when the pool runs dry.
        """
        if seq not in self.table:
            raise KeyError(f"no sequence {seq}")
        snapshot = (copy.copy(self.free), list(self.ref), list(self.table[seq]), self.length[seq])
        slots, pairs = [], []
        try:
            tab = self.table[seq]
            for p in range(self.length[seq], self.length[seq] + n):
                j = p // self.block_size
                if j == len(tab):
                    tab.append(self._take_free())
                elif self.ref[tab[j]] > 1:
                    old = tab[j]
                    new = self._take_free()
                    self.ref[old] -= 1
                    tab[j] = new
                    pairs.append((old, new))
                slots.append(tab[j] * self.block_size + p % self.block_size)
        except OutOfBlocks:
            self.free, self.ref, self.table[seq], self.length[seq] = snapshot
            raise
        self.length[seq] += n
        return slots, pairs

    # -- inspection ----------------------------------------------------------
    def block_table(self, seq):
        return list(self.table[seq])

    def seq_len(self, seq):
        return self.length[seq]

    def refcount(self, b):
        return self.ref[b]

    def num_free(self):
        return len(self.free)

    def free_list(self):
        return list(self.free)

    def sequences(self):
        return sorted(self.table)
