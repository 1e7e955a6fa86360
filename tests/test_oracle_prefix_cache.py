"""The oracle's automatic prefix cache against what the pages fix ([ttlab]
"llm-kv-cache-02-serving-engine-kv", section "4. 프리픽스 캐시"; [icarus]
"PagedAttention", section "支持块级共享"):

  * a block's key hashes the previous block's key, the block's token ids and
    the extra information, so equal tokens after different prefixes get
    different keys and a key stands for the whole prefix;
  * only full blocks are cached (the page's 3,000-token prefix with 32-token
    tails: later requests find 2,992 tokens);
  * a finished request's blocks wait in the free queue tail first and the
    least recently used is evicted first;
  * reused blocks hold exactly the K/V of the same prefix: checked on a
    token-identity pool, where every sequence must gather its own token ids.
"""

import hashlib
import struct

import numpy as np
import pytest

from oracle.block_manager import ROOT_KEY, BlockManager, OutOfBlocks, block_key


def test_key_is_sha256_of_previous_key_tokens_and_extra():
    toks = list(range(100, 116))
    want = hashlib.sha256(bytes(32) + b"".join(struct.pack("<i", t) for t in toks) + struct.pack("<Q", 7)).digest()
    assert block_key(ROOT_KEY, toks, 7) == want
    assert len(want) == 32


def test_equal_tokens_after_different_prefixes_get_different_keys():
    bs = 16
    a = [1] * bs + [5] * bs
    b = [2] * bs + [5] * bs
    bm = BlockManager(8, bs, range(8))
    for s, toks in ((0, a), (1, b)):
        bm.add_seq(s)
        bm.append_tokens(s, toks)
    k0 = [bm.block_key_of(x) for x in bm.block_table(0)]
    k1 = [bm.block_key_of(x) for x in bm.block_table(1)]
    assert k0[1] != k1[1]  # the same 16 tokens, different prefixes
    assert bm.num_cached() == 4
    # the same prompt again reuses both blocks of sequence 0
    assert bm.add_seq_prefix(2, a) == 2 * bs
    assert bm.block_table(2) == bm.block_table(0)
    # a different salt (extra information) finds nothing
    assert bm.prefix_lookup(a, extra=1) == 0
    assert bm.prefix_lookup(a[:bs] + [9] * bs) == bs


def test_only_full_blocks_page_prefix_workload():
    """3,000 shared tokens + 32 unique ones per request, block size 16: the
    first request caches its 189 full blocks; a later request finds the 187
    blocks that lie entirely inside the shared 3,000 tokens (2,992 tokens)
    and computes 40."""
    bs, N = 16, 600
    rng = np.random.default_rng(0)
    prefix = [int(x) for x in rng.integers(0, 50000, 3000)]
    bm = BlockManager(N, bs, rng.permutation(N))
    tails = [[int(x) for x in rng.integers(0, 50000, 32)] for _ in range(4)]
    assert bm.add_seq_prefix(0, prefix + tails[0]) == 0
    bm.append_tokens(0, prefix + tails[0])
    assert bm.num_cached() == 3032 // bs == 189
    for i in (1, 2, 3):
        hit = bm.add_seq_prefix(i, prefix + tails[i])
        assert hit == 2992 == (3000 // bs) * bs
        bm.append_tokens(i, (prefix + tails[i])[hit:])
        assert bm.block_table(i)[:187] == bm.block_table(0)[:187]
        assert bm.block_table(i)[187] != bm.block_table(0)[187]
    for b in bm.block_table(0)[:187]:
        assert bm.refcount(b) == 4


def test_freed_blocks_wait_tail_first_and_lru_is_evicted_first():
    bs, N = 4, 6
    bm = BlockManager(N, bs, range(N))
    prompt = list(range(16))  # 4 full blocks
    bm.add_seq_prefix(0, prompt)
    bm.append_tokens(0, prompt)
    blocks = bm.block_table(0)
    assert blocks == [0, 1, 2, 3] and bm.free_list() == [4, 5]
    bm.free_seq(0)
    # kept with their keys, queued from the last logical block to the first
    assert bm.free_list() == [4, 5, 3, 2, 1, 0] and bm.num_cached() == 4
    assert bm.prefix_lookup(prompt) == 16
    # three fresh blocks: the two never-used ones, then the tail block of the
    # finished request, whose key is evicted
    bm.add_seq(1)
    bm.append_tokens(1, [99] * 12)
    assert bm.block_table(1) == [4, 5, 3]
    assert bm.block_key_of(3) is not None  # block 3 was refilled and keyed as sequence 1's third block
    assert bm.prefix_lookup(prompt) == 12
    # the same prompt again: its first three blocks come back out of the queue
    assert bm.add_seq_prefix(2, prompt) == 12
    assert bm.block_table(2) == [0, 1, 2] and bm.free_list() == []
    assert [bm.refcount(b) for b in range(N)] == [1, 1, 1, 1, 1, 1]


def test_hits_on_live_blocks_share_them():
    bs = 8
    bm = BlockManager(10, bs, range(10))
    p = list(range(20))
    bm.add_seq_prefix(0, p)
    bm.append_tokens(0, p)
    assert bm.add_seq_prefix(1, p) == 16
    assert [bm.refcount(b) for b in bm.block_table(0)] == [2, 2, 1]
    # the second request's own partial block gets the remaining 4 tokens
    slots, pairs = bm.append_tokens(1, p[16:])
    assert pairs == [] and bm.block_table(1)[:2] == bm.block_table(0)[:2]


def test_append_without_token_ids_stops_keying():
    bs = 4
    bm = BlockManager(8, bs, range(8))
    bm.add_seq(0)
    bm.append_tokens(0, [1, 2, 3, 4])
    bm.append_slots(0, 4)
    bm.append_tokens(0, [9, 9, 9, 9])
    assert bm.num_cached() == 1


def test_failed_append_changes_nothing():
    bs = 4
    bm = BlockManager(3, bs, range(3))
    bm.add_seq_prefix(0, list(range(8)))
    bm.append_tokens(0, list(range(8)))
    bm.free_seq(0)
    before = (bm.free_list(), bm.num_cached(), [bm.block_key_of(b) for b in range(3)])
    bm.add_seq(1)
    with pytest.raises(OutOfBlocks):
        bm.append_tokens(1, list(range(100, 116)))  # 4 blocks > 3
    assert before == (bm.free_list(), bm.num_cached(), [bm.block_key_of(b) for b in range(3)])


def _check_identity(bm, pool, want):
    """Every live sequence gathers exactly its own token ids; refcounts and
    the free queue agree with the tables; every cached block is either in use
    or waiting in the free queue."""
    bs = bm.block_size
    refs = [0] * bm.num_blocks
    for s, toks in want.items():
        tab = bm.block_table(s)
        assert bm.seq_len(s) == len(toks)
        got = [pool.get(tab[p // bs] * bs + p % bs) for p in range(len(toks))]
        assert got == toks, f"sequence {s} gathers other tokens"
        for b in tab:
            refs[b] += 1
    assert refs == [bm.refcount(b) for b in range(bm.num_blocks)]
    free = bm.free_list()
    assert len(set(free)) == len(free)
    assert sorted(free) == [b for b in range(bm.num_blocks) if refs[b] == 0]
    for b in range(bm.num_blocks):
        k = bm.block_key_of(b)
        if k is not None:
            assert bm.cache[k] == b


@pytest.mark.parametrize("seed", range(8))
def test_identity_pool_fuzz(seed):
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([1, 2, 4, 16]))
    N = int(rng.integers(12, 60))
    bm = BlockManager(N, bs, rng.permutation(N))
    bases = [[int(x) for x in rng.integers(0, 5, 6 * bs)] for _ in range(3)]
    pool, want, nxt, synth = {}, {}, 0, -1

    def write(slots, toks, pairs):
        for src, dst in pairs:
            for o in range(bs):
                if src * bs + o in pool:
                    pool[dst * bs + o] = pool[src * bs + o]
        for sl, t in zip(slots, toks):
            pool[int(sl)] = t

    for _ in range(300):
        x = rng.random()
        live = list(want)
        if x < 0.25 or not live:
            base = bases[int(rng.integers(3))]
            prompt = base[:int(rng.integers(0, len(base) + 1))] + [int(t) for t in rng.integers(0, 5, int(rng.integers(0, 3 * bs)))]
            extra = int(rng.integers(0, 2))
            hit = bm.add_seq_prefix(nxt, prompt, extra)
            assert hit % bs == 0 and hit <= len(prompt)
            want[nxt] = prompt[:hit]
            try:
                slots, pairs = bm.append_tokens(nxt, prompt[hit:])
                write(slots, prompt[hit:], pairs)
                want[nxt] = prompt
            except OutOfBlocks:
                bm.free_seq(nxt)
                del want[nxt]
            nxt += 1
        elif x < 0.35:
            p = live[int(rng.integers(len(live)))]
            bm.fork(p, nxt)
            want[nxt] = list(want[p])
            nxt += 1
        elif x < 0.55:
            s = live[int(rng.integers(len(live)))]
            bm.free_seq(s)
            del want[s]
        elif x < 0.9:
            s = live[int(rng.integers(len(live)))]
            toks = [int(t) for t in rng.integers(0, 5, int(rng.integers(1, bs + 2)))]
            try:
                slots, pairs = bm.append_tokens(s, toks)
                write(slots, toks, pairs)
                want[s] += toks
            except OutOfBlocks:
                pass
        else:
            s = live[int(rng.integers(len(live)))]
            k = int(rng.integers(1, bs + 1))
            try:
                slots, pairs = bm.append_slots(s, k)
                toks = list(range(synth, synth - k, -1))  # ids no prompt uses
                synth -= k
                write(slots, toks, pairs)
                want[s] += toks
            except OutOfBlocks:
                pass
        _check_identity(bm, pool, want)


# ------------------------------------------------ admission queries (oracle only)
# blocks_needed and admit_cost are what a scheduler compares with the free
# block count before it admits, lets wait or preempts ([icarus] "改善调度与回收";
# [ttlab] "5. KV 자리가 모자라면").  Their pin is their effect: the query must
# equal the free blocks the operation then takes, and the operation must fail
# exactly when the query exceeds the free count.

def test_admission_queries_closed_forms():
    """Hand-worked cases at block size 4: a fresh sequence, a partly filled
    last block, a shared partly filled block (copy-on-write costs one more),
    a shared full block (no copy), and a prompt whose cached prefix waits in
    the free queue or is held by a live sequence."""
    bm = BlockManager(16, 4, list(range(16)))
    bm.add_seq(0)
    assert bm.blocks_needed(0, 0) == 0
    assert bm.blocks_needed(0, 1) == 1
    assert bm.blocks_needed(0, 9) == 3          # ceil(9 / 4)
    bm.append_slots(0, 6)                       # blocks 0, 1; block 1 half full
    assert bm.blocks_needed(0, 2) == 0          # fits in block 1
    assert bm.blocks_needed(0, 3) == 1
    bm.fork(0, 1)                               # block 1 shared, half full
    assert bm.blocks_needed(1, 1) == 1          # copy-on-write of block 1
    assert bm.blocks_needed(1, 3) == 2          # the copy + one new block
    bm.append_slots(0, 2)                       # seq 0 copies block 1, fills its copy
    bm.add_seq(2)
    bm.append_slots(2, 8)
    bm.fork(2, 3)                               # seq 3 shares two full blocks
    assert bm.blocks_needed(3, 1) == 1          # a new block, no copy
    # prefix cache: keyed sequence 4 with 8 tokens = 2 full cached blocks
    prompt = list(range(100, 108))
    bm.add_seq_prefix(4, prompt)
    bm.append_tokens(4, prompt)
    free0 = bm.num_free()
    assert bm.admit_cost(prompt + [1, 2, 3]) == 1          # both blocks live: only the tail block
    assert bm.admit_cost([9] + prompt) == 3                # no hit: ceil(9 / 4)
    bm.free_seq(4)                                         # its blocks wait in the free queue
    assert bm.num_free() == free0 + 2
    assert bm.admit_cost(prompt + [1, 2, 3]) == 3          # two waiting hits + the tail block
    assert bm.admit_cost(prompt[:4]) == 1                  # one waiting hit, nothing else


@pytest.mark.parametrize("seed", range(6))
def test_admission_queries_equal_their_effect(seed):
    """Random admits, forks, frees and appends with token ids: before each
    admission or append, its query equals the drop in free blocks that
    follows, and the operation runs out of blocks exactly when the query is
    larger than the free count (then nothing changes)."""
    rng = np.random.default_rng(500 + seed)
    bs = int(rng.choice([1, 2, 4, 8]))
    N = int(rng.integers(6, 40))
    bm = BlockManager(N, bs, rng.permutation(N))
    bases = [[int(x) for x in rng.integers(0, 5, 5 * bs)] for _ in range(3)]
    live, nxt, checked = [], 0, 0
    for _ in range(400):
        x = rng.random()
        if x < 0.3 or not live:
            base = bases[int(rng.integers(3))]
            prompt = base[:int(rng.integers(0, len(base) + 1))] + \
                [int(t) for t in rng.integers(0, 5, int(rng.integers(0, 3 * bs)))]
            cost, free = bm.admit_cost(prompt), bm.num_free()
            hit = bm.add_seq_prefix(nxt, prompt)
            try:
                bm.append_tokens(nxt, prompt[hit:])
                assert cost <= free and free - bm.num_free() == cost
                live.append(nxt)
            except OutOfBlocks:
                assert cost > free
                bm.free_seq(nxt)  # give back the hit blocks it took
            checked += 1
            nxt += 1
        elif x < 0.4:
            p = live[int(rng.integers(len(live)))]
            bm.fork(p, nxt)
            live.append(nxt)
            nxt += 1
        elif x < 0.55:
            bm.free_seq(live.pop(int(rng.integers(len(live)))))
        else:
            s = live[int(rng.integers(len(live)))]
            n = int(rng.integers(0, 2 * bs + 2))
            need, free = bm.blocks_needed(s, n), bm.num_free()
            before = bm.block_table(s)
            try:
                bm.append_tokens(s, [int(t) for t in rng.integers(0, 5, n)])
                assert need <= free and free - bm.num_free() == need
            except OutOfBlocks:
                assert need > free and bm.block_table(s) == before and bm.num_free() == free
            checked += 1
    assert checked > 150
