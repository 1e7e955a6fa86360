"""The library's prefix cache (pa_bm_add_seq_prefix, pa_bm_append_tokens,
pa_bm_prefix_lookup and the key-keeping free queue) against the oracle:
bit-exact tables, slots, copy-on-write pairs, refcounts, free queue order,
hit counts and block keys.  Host code only: runs without a GPU."""

import hashlib

import numpy as np
import pytest

from oracle.block_manager import BlockManager as OracleBM, OutOfBlocks as OracleOOB
from paged_kv_cache_140_amd import BlockManager as LibBM, OutOfBlocks as LibOOB, pa_sha256


def test_sha256_fips_180_4_examples():
    # the examples of the SHA-256 specification (NIST FIPS 180-4 example set)
    assert pa_sha256(b"abc").hex() == "ba7816bf8f01cfea414140de5dae2223b00361a396177a9cb410ff61f20015ad"
    assert pa_sha256(b"").hex() == "e3b0c44298fc1c149afbf4c8996fb92427ae41e4649b934ca495991b7852b855"
    assert pa_sha256(b"abcdbcdecdefdefgefghfghighijhijkijkljklmklmnlmnomnopnopq").hex() == \
        "248d6a61d20638b8e5c026930c3e6039a33ce45964ff2167f6ecedd419db06c1"
    assert pa_sha256(b"a" * 1000000).hex() == "cdc76e5c9914fb9281a1c7e284d73e67f1809a48a497200e046d39ccc7112cd0"


def test_sha256_every_padding_boundary():
    rng = np.random.default_rng(0)
    for n in list(range(0, 200)) + [1000, 4096 + 55]:
        data = rng.integers(0, 256, n, dtype=np.uint8).tobytes()
        assert pa_sha256(data) == hashlib.sha256(data).digest(), n


def _same(o, l, live):
    assert o.free_list() == l.free_list()
    assert o.num_cached() == l.num_cached()
    for b in range(o.num_blocks):
        assert o.refcount(b) == l.refcount(b)
        assert o.block_key_of(b) == l.block_key_of(b), b
    for s in live:
        assert o.block_table(s) == l.block_table(s)
        assert o.seq_len(s) == l.seq_len(s)


@pytest.mark.parametrize("seed", range(10))
def test_prefix_cache_ops_bit_exact(seed):
    rng = np.random.default_rng(1000 + seed)
    bs = int(rng.choice([1, 2, 4, 8, 16]))
    N = int(rng.integers(8, 70))
    order = rng.permutation(N)
    o, l = OracleBM(N, bs, order), LibBM(N, bs, order)
    bases = [[int(x) for x in rng.integers(-3, 4, 6 * bs)] for _ in range(3)]
    live, nxt = [], 0
    for _ in range(300):
        x = rng.random()
        if x < 0.25 or not live:
            base = bases[int(rng.integers(3))]
            prompt = base[:int(rng.integers(0, len(base) + 1))] + \
                [int(t) for t in rng.integers(-3, 4, int(rng.integers(0, 3 * bs)))]
            extra = int(rng.choice([0, 1, 2**63 + 5]))
            assert o.prefix_lookup(prompt, extra) == l.prefix_lookup(prompt, extra)
            cost = o.admit_cost(prompt, extra)
            assert cost == l.admit_cost(prompt, extra)
            free_before = o.num_free()
            ho, hl = o.add_seq_prefix(nxt, prompt, extra), l.add_seq_prefix(nxt, prompt, extra)
            assert ho == hl
            live.append(nxt)
            try:
                so, po = o.append_tokens(nxt, prompt[ho:])
                ok = True
            except OracleOOB:
                ok = False
            assert ok == (cost <= free_before)
            if ok:
                assert free_before - o.num_free() == cost
                sl, pl = l.append_tokens(nxt, prompt[ho:])
                assert list(sl) == so and pl == po
            else:
                with pytest.raises(LibOOB):
                    l.append_tokens(nxt, prompt[ho:])
            nxt += 1
        elif x < 0.33:
            p = live[int(rng.integers(len(live)))]
            o.fork(p, nxt)
            l.fork(p, nxt)
            live.append(nxt)
            nxt += 1
        elif x < 0.5:
            s = live.pop(int(rng.integers(len(live))))
            o.free_seq(s)
            l.free_seq(s)
        elif x < 0.85:
            s = live[int(rng.integers(len(live)))]
            toks = [int(t) for t in rng.integers(-3, 4, int(rng.integers(0, 2 * bs + 2)))]
            need = o.blocks_needed(s, len(toks))
            assert need == l.blocks_needed(s, len(toks))
            free_before = o.num_free()
            try:
                so, po = o.append_tokens(s, toks)
                ok = True
            except OracleOOB:
                ok = False
            assert ok == (need <= free_before)
            if ok:
                assert free_before - o.num_free() == need
                sl, pl = l.append_tokens(s, toks)
                assert list(sl) == so and pl == po
            else:
                with pytest.raises(LibOOB):
                    l.append_tokens(s, toks)
        elif x < 0.93:
            s = live[int(rng.integers(len(live)))]
            k = int(rng.integers(0, bs + 2))
            try:
                so, po = o.append_slots(s, k)
                ok = True
            except OracleOOB:
                ok = False
            if ok:
                sl, pl = l.append_slots(s, k)
                assert list(sl) == so and pl == po
            else:
                with pytest.raises(LibOOB):
                    l.append_slots(s, k)
        else:
            # a batch that the library must apply all or nothing (evicted keys
            # included); the oracle applies it entry by entry when it fits
            m = int(rng.integers(1, min(4, len(live)) + 1))
            seqs = [live[int(i)] for i in rng.integers(len(live), size=m)]
            ks = [int(rng.integers(0, 2 * bs + 2)) for _ in seqs]
            free_before, cached_before = l.free_list(), l.num_cached()
            keys_before = [l.block_key_of(b) for b in range(N)]
            try:
                sl, pl = l.append_slots_batch(seqs, ks)
                ok = True
            except LibOOB:
                ok = False
            if ok:
                so, po = [], []
                for s, k in zip(seqs, ks):
                    a, b = o.append_slots(s, k)
                    so += a
                    po += b
                assert list(sl) == so and [tuple(p) for p in pl.tolist()] == po
            else:
                assert l.free_list() == free_before and l.num_cached() == cached_before
                assert [l.block_key_of(b) for b in range(N)] == keys_before
        _same(o, l, live)


def test_failed_batch_restores_evicted_keys():
    bs = 4
    l = LibBM(6, bs, range(6))
    p = list(range(16))
    l.add_seq_prefix(0, p)
    l.append_tokens(0, p)
    l.free_seq(0)
    l.add_seq(1)
    l.add_seq(2)
    assert l.num_cached() == 4 and l.free_list() == [4, 5, 3, 2, 1, 0]
    # the first entry takes blocks 4, 5, 3 (evicting block 3's key); the
    # second needs 4 more: the whole batch fails and block 3 is cached again
    with pytest.raises(LibOOB):
        l.append_slots_batch([1, 2], [12, 16])
    assert l.free_list() == [4, 5, 3, 2, 1, 0] and l.num_cached() == 4
    assert l.prefix_lookup(p) == 16
