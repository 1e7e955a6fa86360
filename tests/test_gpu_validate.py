"""Validate mode: every entry point checks the device indices it trusts
before it launches anything, and returns PA_EINVAL (nothing enqueued) on a
bad one.  Valid inputs give the same bits with the mode on.

The pool tensors hold 16 blocks more than the library is told, and every bad
block id used here lies in that margin, so even a check that let one through
would only read inside the allocation."""

import numpy as np
import pytest
import torch

from gpu_util import bits, say

pytestmark = pytest.mark.gpu

N, BS, H_KV, H_Q, D = 64, 16, 2, 8, 128


@pytest.fixture
def world():
    from paged_kv_cache_140_amd import KVPool, pa_set_validate

    pool = KVPool(1, H_KV, N + 16, BS, D, "bf16")  # allocation with a margin
    pool.k.normal_()
    pool.v.normal_()
    pool.num_blocks = N  # what the library is told
    old = pa_set_validate(True)
    try:
        yield pool
    finally:
        pa_set_validate(old)


def _expect_einval(fn, *a):
    from paged_kv_cache_140_amd import PAError
    from paged_kv_cache_140_amd._lib import PA_EINVAL

    with pytest.raises(PAError) as ei:
        fn(*a)
    assert ei.value.status == PA_EINVAL


def test_validate_rejects_bad_indices_before_launch(world):
    from paged_kv_cache_140_amd import (decode_workspace, pa_cache_append, pa_copy_blocks, pa_decode,
                                        pa_decode_append, pa_mixed_batch, pa_prefill_chunk)

    pool = world
    say("validate mode: bad indices")
    dev = "cuda"
    tab = torch.arange(0, 8, dtype=torch.int32, device=dev).reshape(2, 4)
    lens = torch.tensor([50, 64], dtype=torch.int32, device=dev)
    q = torch.randn(2, H_Q, D, device=dev).to(torch.bfloat16)
    out = torch.full_like(q, float("nan"))
    # a visible block id past the pool; a context past max_ctx
    bad = tab.clone()
    bad[1, 3] = N + 3
    _expect_einval(pa_decode, pool, 0, out, q, bad, lens, 64, 0.1)
    _expect_einval(pa_decode, pool, 0, out, q, tab, torch.tensor([50, 65], dtype=torch.int32, device=dev), 64, 0.1)
    # an entry past a sequence's visible blocks is not looked at
    ok = tab.clone()
    ok[0, 3] = N + 5  # sequence 0 sees blocks 0..3 (50 tokens): entry 3 is visible -> rejected
    _expect_einval(pa_decode, pool, 0, out, q, ok, lens, 64, 0.1)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all(), "a rejected call wrote its output"
    # appends: a repeated slot, a slot past the pool
    kv = torch.randn(3, H_KV, D, device=dev).to(torch.bfloat16)
    _expect_einval(pa_cache_append, pool, 0, kv, kv, torch.tensor([5, 9, 5], dtype=torch.int32, device=dev))
    _expect_einval(pa_cache_append, pool, 0, kv, kv, torch.tensor([5, 9, N * BS], dtype=torch.int32, device=dev))
    # copy pairs: a destination reused, a destination that is also a source, an id past the pool
    for pairs in ([[1, 2], [3, 2]], [[1, 2], [2, 4]], [[1, N + 2]]):
        _expect_einval(pa_copy_blocks, pool, torch.tensor(pairs, dtype=torch.int32, device=dev))
    # fused append: a slot that is not position ctx - 1 of its row
    nk = torch.randn(2, H_KV, D, device=dev).to(torch.bfloat16)
    slot_ok = [int(tab[0, 49 // BS]) * BS + 49 % BS, int(tab[1, 63 // BS]) * BS + 63 % BS]
    _expect_einval(pa_decode_append, pool, 0, out, q, nk, nk,
                   torch.tensor([slot_ok[0] + 1, slot_ok[1]], dtype=torch.int32, device=dev), tab, lens, 64, 0.1)
    # prefill and the mixed batch: a chunk table entry past the pool
    pq = torch.randn(40, H_Q, D, device=dev).to(torch.bfloat16)
    pout = torch.full_like(pq, float("nan"))
    ptab = torch.arange(10, 20, dtype=torch.int32, device=dev)
    pbad = ptab.clone()
    pbad[4] = N + 1
    _expect_einval(pa_prefill_chunk, pool, 0, pout, pq, pbad, 100, 0.1)
    ws = decode_workspace(pool, 2, H_Q, 64)
    _expect_einval(pa_mixed_batch, pool, 0, out, q, bad, lens, 64, pout, pq, [(40, 100)], ptab.view(1, -1), 0.1, 0,
                   ws)
    _expect_einval(pa_mixed_batch, pool, 0, out, q, tab, lens, 64, pout, pq, [(40, 100)], pbad.view(1, -1), 0.1, 0,
                   ws)
    torch.cuda.synchronize()
    assert torch.isnan(pout.float()).all() and torch.isnan(out.float()).all()


def test_validate_passes_valid_calls_unchanged(world):
    from paged_kv_cache_140_amd import pa_decode, pa_prefill_chunk, pa_set_validate

    pool = world
    say("validate mode: valid calls")
    dev = "cuda"
    tab = torch.tensor([[7, 3, 9, 1], [2, 8, 4, 6]], dtype=torch.int32, device=dev)
    lens = torch.tensor([50, 64], dtype=torch.int32, device=dev)
    q = torch.randn(2, H_Q, D, device=dev).to(torch.bfloat16)
    pq = torch.randn(40, H_Q, D, device=dev).to(torch.bfloat16)
    ptab = torch.arange(10, 20, dtype=torch.int32, device=dev)
    outs = []
    for on in (True, False):
        pa_set_validate(on)
        out, pout = torch.empty_like(q), torch.empty_like(pq)
        pa_decode(pool, 0, out, q, tab, lens, 64, 0.1)
        pa_prefill_chunk(pool, 0, pout, pq, ptab, 100, 0.1)
        torch.cuda.synchronize()
        outs.append((bits(out), bits(pout)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
