"""Pins of the oracle allocator: printed examples, closed forms, invariants, brute force."""

import itertools
import math

import numpy as np
import pytest

from oracle.block_manager import BlockManager, OutOfBlocks
from oracle.pool import Pool


def identity_order(n):
    return list(range(n))


def test_600_tokens_take_38_blocks(golden):
    g = golden["block_count_600"]["printed"]
    bm = BlockManager(64, g["block_size"], identity_order(64))
    bm.add_seq(0)
    slots, pairs = bm.append_slots(0, g["tokens"])
    assert len(bm.block_table(0)) == g["blocks"]
    assert len(bm.block_table(0)) * g["block_size"] == g["slots"]
    assert g["slots"] < g["reserved_tokens"]
    assert pairs == [] and len(set(slots)) == g["tokens"]


@pytest.mark.parametrize("key", ["block_table_youngju", "block_table_icarus"])
def test_printed_block_tables(golden, key):
    """A request that grows to four blocks, handed the physical blocks in the
    printed order, ends up with exactly the printed table, and its slots
    address the printed physical blocks in logical order."""
    phys = golden[key]["printed"]["physical"]
    n = max(phys) + 5
    order = phys + [b for b in range(n) if b not in phys]
    bs = 16
    bm = BlockManager(n, bs, order)
    bm.add_seq("A")
    slots = []
    for _ in range(4 * bs):  # token by token, as a decode would grow it
        s, _ = bm.append_slots("A", 1)
        slots += s
    assert bm.block_table("A") == phys
    assert [s // bs for s in slots[::bs]] == phys
    assert [s % bs for s in slots] == list(range(bs)) * 4


def test_capacity_22048_tokens_holds_34_requests(golden):
    g = golden["capacity_22048"]
    p, dv = g["printed"], g["derived"]
    bs = p["block_size"]
    n_blocks = p["kv_tokens"] // bs
    assert n_blocks == dv["num_blocks"] and n_blocks * bs == p["kv_tokens"]
    bm = BlockManager(n_blocks, bs, identity_order(n_blocks))
    fitted = 0
    while True:
        bm.add_seq(fitted)
        try:
            bm.append_slots(fitted, p["request_in"] + p["request_out"])
        except OutOfBlocks:
            break
        fitted += 1
    assert fitted == dv["fits_exactly"] == p["about_fits"]
    assert len(bm.block_table(0)) == dv["blocks_per_request"]


def test_waste_illustration(golden):
    g = golden["waste_illustration"]
    bs = g["derived"]["block_size"]
    bm = BlockManager(256, bs, identity_order(256))
    for i, used in enumerate(g["printed"]["used"]):
        bm.add_seq(i)
        bm.append_slots(i, used)
        nb = len(bm.block_table(i))
        assert nb == g["derived"]["blocks"][i]
        assert nb * bs - used == g["derived"]["paged_waste"][i]
        assert g["printed"]["reserved"] - used == g["derived"]["reserved_waste"][i]


def test_self_check_two_requests(golden):
    g = golden["self_check_two_requests"]
    bs = g["derived"]["block_size"]
    bm = BlockManager(400, bs, identity_order(400))
    for i, used in enumerate(g["printed"]["used"]):
        bm.add_seq(i)
        bm.append_slots(i, used)
    blocks = [len(bm.block_table(i)) for i in range(2)]
    assert blocks == g["derived"]["blocks"]
    assert sum(blocks) == g["derived"]["total_blocks"]
    assert sum(blocks) * bs == g["derived"]["paged_slots"]
    assert 2 * g["printed"]["max_tokens"] == g["derived"]["reserved_slots"]
    assert bm.num_free() == 400 - sum(blocks)


@pytest.mark.parametrize("bs", [1, 3, 8, 16, 32])
def test_block_count_and_waste_bound(bs):
    rng = np.random.default_rng(bs)
    bm = BlockManager(45000, bs, rng.permutation(45000))
    for i in range(60):
        n = int(rng.integers(0, 700))
        bm.add_seq(i)
        # grow in random pieces, like prefill followed by decode steps
        left = n
        while left:
            k = int(min(left, rng.integers(1, 50)))
            bm.append_slots(i, k)
            left -= k
        nb = len(bm.block_table(i))
        assert nb == math.ceil(n / bs)
        waste = nb * bs - n
        assert 0 <= waste <= bs - 1


def _check_invariants(bm):
    used = {}
    for s in bm.sequences():
        tab = bm.block_table(s)
        assert len(tab) == math.ceil(bm.seq_len(s) / bm.block_size)
        for b in tab:
            used[b] = used.get(b, 0) + 1
    # refcount recomputed from the tables
    for b in range(bm.num_blocks):
        assert bm.refcount(b) == used.get(b, 0)
    free = bm.free_list()
    assert len(set(free)) == len(free)
    assert set(free) == {b for b in range(bm.num_blocks) if used.get(b, 0) == 0}
    assert sum(bm.refcount(b) for b in range(bm.num_blocks)) == sum(len(bm.block_table(s)) for s in bm.sequences())


class TokenWorld:
    """Allocator + a pool that stores token ids, next to the plain logical history.

    Each write stores a fresh unique id; a sequence's gathered ids must always
    equal the list of ids it (or its ancestors before a fork) wrote -- the
    semantic statement of paging plus copy-on-write.
    """

    def __init__(self, n, bs, order):
        self.bm = BlockManager(n, bs, order)
        self.pool = Pool(1, 1, n, bs, 1, "f32", fill_bits=0xFFFFFFFF)
        self.hist = {}
        self.next_id = 1

    def add(self, s):
        self.bm.add_seq(s)
        self.hist[s] = []

    def fork(self, p, c):
        self.bm.fork(p, c)
        self.hist[c] = list(self.hist[p])

    def free(self, s):
        self.bm.free_seq(s)
        del self.hist[s]

    def append(self, s, n):
        slots, pairs = self.bm.append_slots(s, n)
        self.pool.copy_blocks(pairs)
        ids = list(range(self.next_id, self.next_id + n))
        self.next_id += n
        rows = np.array(ids, dtype=np.uint32).reshape(n, 1, 1)
        self.pool.append(0, rows, rows, slots)
        self.hist[s] += ids
        return slots, pairs

    def check(self):
        _check_invariants(self.bm)
        live_slots = {}
        for s in self.bm.sequences():
            tab = self.bm.block_table(s)
            L = self.bm.seq_len(s)
            got = self.pool.k[0, 0, [tab[p // self.bm.block_size] for p in range(L)],
                              [p % self.bm.block_size for p in range(L)], 0].tolist() if L else []
            assert got == self.hist[s], (s, got, self.hist[s])
            # a block held by exactly one sequence is that sequence's alone
            for b in tab:
                if self.bm.refcount(b) == 1:
                    assert live_slots.setdefault(b, s) == s


def test_random_ops_keep_history_and_invariants():
    rng = np.random.default_rng(2024)
    for trial in range(40):
        n = int(rng.integers(4, 40))
        bs = int(rng.choice([1, 2, 3, 4, 16]))
        w = TokenWorld(n, bs, rng.permutation(n))
        live = []
        nxt = 0
        for _ in range(120):
            op = rng.random()
            if op < 0.2 or not live:
                w.add(nxt)
                live.append(nxt)
                nxt += 1
            elif op < 0.35:
                c = nxt
                nxt += 1
                w.fork(live[int(rng.integers(len(live)))], c)
                live.append(c)
            elif op < 0.5:
                w.free(live.pop(int(rng.integers(len(live)))))
            else:
                s = live[int(rng.integers(len(live)))]
                k = int(rng.integers(1, 3 * bs + 2))
                before = (w.bm.free_list(), [w.bm.refcount(b) for b in range(n)],
                          {q: w.bm.block_table(q) for q in live}, {q: w.bm.seq_len(q) for q in live})
                try:
                    w.append(s, k)
                except OutOfBlocks:
                    after = (w.bm.free_list(), [w.bm.refcount(b) for b in range(n)],
                             {q: w.bm.block_table(q) for q in live}, {q: w.bm.seq_len(q) for q in live})
                    assert before == after
            w.check()


def test_cow_copies_only_the_written_shared_block():
    bs = 4
    w = TokenWorld(32, bs, identity_order(32))
    w.add(0)
    w.append(0, 10)  # blocks 0,1,2 ; block 2 half full
    for c in (1, 2, 3):
        w.fork(0, c)
    assert [w.bm.refcount(b) for b in (0, 1, 2)] == [4, 4, 4]
    got_pairs = []
    for s in (0, 1, 2, 3):
        _, pairs = w.append(s, 1)
        got_pairs.append(pairs)
        w.check()
    # writers 0,1,2 copy the shared partial block; the last holder writes in place
    assert got_pairs == [[(2, 3)], [(2, 4)], [(2, 5)], []]
    assert [w.bm.refcount(b) for b in (0, 1, 2)] == [4, 4, 1]
    # full shared blocks are never copied
    for s in (0, 1):
        _, pairs = w.append(s, 2)
        assert pairs == []
    w.check()


def test_free_returns_blocks_tail_first_at_the_back():
    bm = BlockManager(10, 2, identity_order(10))
    bm.add_seq(0)
    bm.append_slots(0, 5)  # blocks 0,1,2
    bm.add_seq(1)
    bm.append_slots(1, 2)  # block 3
    bm.free_seq(0)
    assert bm.free_list() == [4, 5, 6, 7, 8, 9, 2, 1, 0]
    bm.fork(1, 2)
    bm.free_seq(1)
    assert bm.refcount(3) == 1 and 3 not in bm.free_list()
    bm.free_seq(2)
    assert bm.free_list()[-1] == 3


def _brute_ops(n_seq_max=3):
    ops = [("add",), ("append", 1), ("append", 2), ("fork",), ("free",)]
    return ops


@pytest.mark.parametrize("n_blocks,bs", [(3, 1), (4, 2), (5, 3)])
def test_brute_force_small_pools(n_blocks, bs):
    """Every sequence of up to 5 ops on every free order of a tiny pool keeps
    the token history and every invariant, and a failing append changes nothing."""
    ops = _brute_ops()
    count = 0
    orders = list(itertools.permutations(range(n_blocks)))
    if len(orders) > 24:  # relabelings of one another; a fixed sample suffices
        orders = [orders[i] for i in np.random.default_rng(n_blocks).choice(len(orders), 8, replace=False)]
    for order in orders:
        for seq_ops in itertools.product(range(len(ops)), repeat=5):
            w = TokenWorld(n_blocks, bs, list(order))
            live = []
            nxt = 0
            for oi in seq_ops:
                op = ops[oi]
                if op[0] == "add":
                    w.add(nxt)
                    live.append(nxt)
                    nxt += 1
                elif not live:
                    continue
                elif op[0] == "append":
                    s = live[-1]
                    snap = (w.bm.free_list(), [w.bm.refcount(b) for b in range(n_blocks)], w.bm.block_table(s))
                    try:
                        w.append(s, op[1])
                    except OutOfBlocks:
                        assert snap == (w.bm.free_list(), [w.bm.refcount(b) for b in range(n_blocks)],
                                        w.bm.block_table(s))
                elif op[0] == "fork":
                    w.fork(live[0], nxt)
                    live.append(nxt)
                    nxt += 1
                elif op[0] == "free":
                    w.free(live.pop(0))
                w.check()
                count += 1
    assert count > 1000
