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

Automatic prefix caching ([ttlab] "4. 프리픽스 캐시"; [icarus] "支持块级共享":
full KV blocks are hashed so a later request with the same prefix reuses the
computed K/V):
  * every full block gets a key = hash(the previous block's key, this block's
    token ids, extra information such as a cache salt); through the previous
    key, one key stands for the whole prefix up to that block, so equal
    tokens after different prefixes get different keys;
  * only full blocks are cached;
  * a finished request's blocks are not wiped: they wait in the free queue
    with their contents and keys ("empty but still holding content"), queued
    tail first, and the least recently used is evicted when a block is
    needed;
  * the hash is sha256.
Readings where the pages leave a choice (listed in the design notes): the
first block's previous key is 32 zero bytes; the hashed bytes are the
previous key, the block's token ids as little-endian int32 and the extra
information as one little-endian uint64; a block whose key is already cached
under another block stays uncached; a cache hit takes the block out of the
free queue wherever it sits; a sequence appended without token ids
(append_slots) is no longer keyed.

Processing is token by token, in the order the text describes, with a
snapshot taken before each request for the all-or-nothing failure.
"""

import copy
import hashlib
import struct
from collections import deque

ROOT_KEY = bytes(32)


def block_key(prev_key, tokens, extra):
    """Key of one full block: sha256(previous key, token ids, extra)."""
    data = prev_key + struct.pack(f"<{len(tokens)}i", *[int(t) for t in tokens]) + struct.pack("<Q", int(extra))
    return hashlib.sha256(data).digest()


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
        # prefix cache: key -> block, block -> key, and per sequence the
        # keying state: (extra, key of its last full block, token ids of its
        # partly filled block), or None once it is no longer keyed
        self.cache = {}
        self.key_of = {}
        self.keyed = {}

    # -- sequences ---------------------------------------------------------
    def add_seq(self, seq, extra=0):
        if seq in self.table:
            raise KeyError(f"sequence {seq} exists")
        self.table[seq] = []
        self.length[seq] = 0
        self.keyed[seq] = (int(extra), ROOT_KEY, [])

    def add_seq_prefix(self, seq, tokens, extra=0):
        """A new sequence for a prompt: its table starts with the cached
        blocks of the prompt's longest cached prefix of full blocks.  Returns
        the number of prompt tokens those blocks hold; the caller appends the
        rest with append_tokens."""
        self.add_seq(seq, extra)
        bs = self.block_size
        prev = ROOT_KEY
        for j in range(len(tokens) // bs):
            key = block_key(prev, tokens[j * bs:(j + 1) * bs], extra)
            b = self.cache.get(key)
            if b is None:
                break
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
            self.table[seq].append(b)
            self.length[seq] += bs
            prev = key
        self.keyed[seq] = (int(extra), prev, [])
        return self.length[seq]

    def blocks_needed(self, seq, n):
        """Free blocks append_slots(seq, n) would take: the new logical blocks
        it reaches, and one more when its partly filled last block is
        shared (copy-on-write)."""
        bs, tab, ln = self.block_size, self.table[seq], self.length[seq]
        if n <= 0:
            return 0
        fresh = -(-(ln + n) // bs) - len(tab)
        cow = 1 if ln % bs and self.ref[tab[-1]] > 1 else 0
        return fresh + cow

    def admit_cost(self, tokens, extra=0):
        """Free-queue blocks that admitting a prompt takes: its cached prefix
        blocks that wait in the free queue, and a fresh block for each block
        of the rest."""
        bs = self.block_size
        prev, hits, waiting = ROOT_KEY, 0, 0
        for j in range(len(tokens) // bs):
            key = block_key(prev, tokens[j * bs:(j + 1) * bs], extra)
            b = self.cache.get(key)
            if b is None:
                break
            hits += 1
            waiting += self.ref[b] == 0
            prev = key
        return waiting + -(-len(tokens) // bs) - hits

    def prefix_lookup(self, tokens, extra=0):
        """Prompt tokens a new request would find cached (no state change)."""
        bs = self.block_size
        prev, hit = ROOT_KEY, 0
        for j in range(len(tokens) // bs):
            key = block_key(prev, tokens[j * bs:(j + 1) * bs], extra)
            if key not in self.cache:
                break
            hit += bs
            prev = key
        return hit

    def fork(self, parent, child):
        """child shares every block of parent (parallel sampling / beam search)."""
        if parent not in self.table or child in self.table:
            raise KeyError("fork needs an existing parent and a new child")
        self.table[child] = list(self.table[parent])
        self.length[child] = self.length[parent]
        for b in self.table[child]:
            self.ref[b] += 1
        st = self.keyed[parent]
        self.keyed[child] = None if st is None else (st[0], st[1], list(st[2]))

    def free_seq(self, seq):
        """Drop a finished sequence; blocks whose count reaches 0 rejoin the pool."""
        blocks = self.table.pop(seq)
        del self.length[seq]
        del self.keyed[seq]
        for b in reversed(blocks):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    # -- growth ------------------------------------------------------------
    def _take_free(self):
        if not self.free:
            raise OutOfBlocks()
        b = self.free.popleft()
        if b in self.key_of:  # evict: its contents are about to be overwritten
            del self.cache[self.key_of.pop(b)]
        self.ref[b] = 1
        return b

    def append_slots(self, seq, n):
        """Reserve slots for the next n tokens of ``seq``.

        Returns (slots, cow_pairs): slot = physical block * block_size + offset
        for each new token in order, and the (source, destination) block pairs
        whose contents must be copied before the new tokens are written.
        Raises OutOfBlocks with no state change when the pool runs dry.
        Without token ids the sequence's later blocks cannot be keyed.
        """
        slots, pairs = self._append(seq, n, None)
        self.keyed[seq] = None
        return slots, pairs

    def append_tokens(self, seq, tokens):
        """append_slots for the given token ids; every block the append fills
        is keyed and, unless its key is already cached, cached."""
        return self._append(seq, len(tokens), [int(t) for t in tokens])

    def _append(self, seq, n, tokens):
        if seq not in self.table:
            raise KeyError(f"no sequence {seq}")
        snapshot = (copy.copy(self.free), list(self.ref), list(self.table[seq]), self.length[seq],
                    dict(self.cache), dict(self.key_of), self.keyed[seq])
        slots, pairs = [], []
        st = self.keyed[seq]
        if tokens is not None and st is not None:
            st = (st[0], st[1], list(st[2]))
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
                if tokens is not None and st is not None:
                    extra, prev, part = st
                    part.append(tokens[p - self.length[seq]])
                    if len(part) == self.block_size:  # block j is full: key it
                        key = block_key(prev, part, extra)
                        if key not in self.cache:
                            self.cache[key] = tab[j]
                            self.key_of[tab[j]] = key
                        st = (extra, key, [])
        except OutOfBlocks:
            (self.free, self.ref, self.table[seq], self.length[seq], self.cache, self.key_of,
             self.keyed[seq]) = snapshot
            raise
        self.length[seq] += n
        if tokens is not None:
            self.keyed[seq] = st
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

    def num_cached(self):
        return len(self.cache)

    def block_key_of(self, b):
        """The block's cache key, or None if it is not cached."""
        return self.key_of.get(b)
