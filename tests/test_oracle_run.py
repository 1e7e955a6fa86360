"""The oracle's scenario driver: paged view == logical view, and the workload
facts the configs promise (block counts, copy-on-write pairs, pool fit)."""

import numpy as np
import pytest

from oracle.run import OracleRun
from pa_inputs import build_scenario


def _run(cid, seed=0, **over):
    scn = build_scenario(cid, seed, **over)
    r = OracleRun(scn)
    r.run_setup()
    return scn, r


def test_config1_paged_equals_logical_and_uses_12_blocks():
    scn, r = _run(1)
    assert list(scn.ctx) == [1, 16, 17, 100]
    used_before = 64 - r.bm.num_free()
    assert used_before == 1 + 1 + 2 + 7
    res = r.run_step(scn.steps[0])
    assert 64 - r.bm.num_free() == 12
    assert res.decode_lengths == [2, 17, 18, 101]
    assert res.pairs == []
    logical = [r.logical_kv(s) for s in range(4)]
    from oracle import attention, run as orun

    q = orun.widen(scn.steps[0].q, "f32")
    for i in range(4):
        ref = attention.attend(q[i], *logical[i], scn.cfg["scale"])
        np.testing.assert_array_equal(res.decode_out[i], ref)


def test_config2_shapes_and_fit():
    scn, r = _run(2)
    ctx = scn.ctx
    assert ctx.min() >= 512 and ctx.max() <= 640 and len(ctx) == 32
    res = r.run_step(scn.steps[0], decode_rows=[0, 31])
    assert np.all(np.isfinite(res.decode_out[[0, 31]]))
    assert len(res.slots) == 32 and len(set(res.slots)) == 32


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_config3_churn_then_fit(bs):
    scn = build_scenario(3, 0, bs=bs)
    r = OracleRun(scn, with_data=False)
    r.run_setup()
    assert r.bm.num_blocks == 64 * (2048 // bs + 1)
    # churn scattered the free list: the real sequences do not get ascending ids
    t0 = r.bm.block_table(0)
    assert t0 != sorted(t0)
    res = r.run_step(scn.steps[0])
    assert len(res.slots) == 64


def test_config4_copy_on_write_pairs_small():
    """Scaled-down config 4: 2 prompts x 3 samples, 40-token prefix (block 2 of 16
    tokens half full), tail of 5: every sample but the last copies the block."""
    scn = build_scenario(4, 0, prompts=2, samples=3, prefix=40, tail=5, steps=2, num_blocks=64)
    r = OracleRun(scn)
    r.run_setup()
    shared = [r.bm.block_table(0)[2], r.bm.block_table(3)[2]]
    assert [r.bm.refcount(b) for b in shared] == [3, 3]
    tail = r.run_step(scn.steps[0])
    assert [s for s, _ in tail.pairs] == [shared[0], shared[0], shared[1], shared[1]]
    assert r.bm.block_table(2)[2] == shared[0] and r.bm.block_table(5)[2] == shared[1]
    assert [r.bm.refcount(b) for b in shared] == [1, 1]
    for st in scn.steps[1:]:
        res = r.run_step(st)
        assert res.pairs == []
        for i, seq in enumerate(st.decode_seqs):
            from oracle import attention, run as orun

            ref = attention.attend(orun.widen(st.q, "bf16")[i], *r.logical_kv(seq), scn.cfg["scale"])
            np.testing.assert_array_equal(res.decode_out[i], ref)


def test_config4_full_bookkeeping():
    """Full config 4 allocator only: 56 copy-on-write pairs, 1,752 blocks used."""
    scn = build_scenario(4, 0)
    r = OracleRun(scn, with_data=False)
    r.run_setup()
    assert r.bm.num_free() == 2048 - 8 * 188
    assert all(r.bm.refcount(b) == 8 for b in r.bm.block_table(0))
    tail = r.run_step(scn.steps[0])
    assert len(tail.pairs) == 56
    for st in scn.steps[1:]:
        r.run_step(st)
    assert 2048 - r.bm.num_free() == 1752
    assert r.results[-1].decode_lengths == [3048] * 64


def test_config5_bookkeeping_and_chunk_rows():
    scn = build_scenario(5, 0)
    assert scn.ctx.min() >= 1024 and scn.ctx.max() <= 32768 and len(scn.ctx) == 63
    r = OracleRun(scn, with_data=False)  # allocator only (the full pool is GPU-sized)
    r.run_setup()
    slots, pairs = r.bookkeeping(scn.steps[0])
    assert len(slots) == 63 + 1024 and pairs == []
    assert r.bm.seq_len(63) == 3500 + 1024
    assert len(r.bm.block_table(63)) == -(-4524 // 16)


def test_beam_search_paged_equals_logical_every_step():
    """Beam search: beams fork from forks and copy the shared partly filled
    block on write at every depth; at each step every beam's paged decode
    equals attention over its own logical K/V rows, bit for bit."""
    from oracle import attention
    from oracle.run import widen

    scn = build_scenario(6, 0, prompts=2, prompt_len=40, steps=12, d=64)
    r = OracleRun(scn)
    r.run_setup()
    forks = pairs = 0
    for st in scn.steps:
        forks += sum(op[0] == "fork" for op in st.ops)
        res = r.run_step(st)
        pairs += len(res.pairs)
        q = widen(st.q, "bf16")
        for i, seq in enumerate(st.decode_seqs):
            np.testing.assert_array_equal(res.decode_out[i], attention.attend(q[i], *r.logical_kv(seq),
                                                                              scn.cfg["scale"]))
        # each prompt keeps exactly ``beam`` live beams
        assert len(st.decode_seqs) == 2 * 4
    assert forks > 0 and pairs > 0
