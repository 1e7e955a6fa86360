"""KV memory use, paged against max-length reservation, pinned by the pages'
numbers: the three-request illustration (320 / 96 / 1,180 tokens of 2,048
reserved), the 20.4-38.2% of KV memory that held tokens in prior systems,
waste below one block per request, and 22,048 tokens of KV holding 34
requests of 640 tokens."""

import numpy as np
import pytest

from oracle import capacity
from oracle.block_manager import BlockManager
from pa_inputs import gen
from pa_inputs.configs import config


def _paged(lengths, bs):
    N = sum(-(-n // bs) for n in lengths)
    bm = BlockManager(N, bs, range(N))
    for i, n in enumerate(lengths):
        bm.add_seq(i)
        bm.append_slots(i, int(n))
    return bm


def test_page_illustration():
    lengths, max_len = [320, 96, 1180], 2048
    tokens = sum(lengths)
    reserved = capacity.utilisation(tokens, capacity.reserved_slots(lengths, max_len))
    assert abs(reserved - 1596 / 6144) < 1e-12
    assert 0.204 <= reserved <= 0.382  # the pages' range for reservation-based systems
    bm = _paged(lengths, 16)
    assert capacity.waste_per_request(bm, range(3)) == [0, 0, 4]
    assert capacity.paged_slots(bm, range(3)) == 1600
    assert capacity.utilisation(tokens, capacity.paged_slots(bm, range(3))) > 0.99


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_lognormal_lengths_waste_below_one_block(bs):
    """The 13B-shaped workload's lengths (lognormal, median 400): each request
    wastes 0 .. bs-1 slots (mean near (bs-1)/2); a 2,048-token reservation
    holds tokens in about a quarter of its slots, inside the pages' range."""
    cfg = config(3, bs=bs)
    lengths = [int(x) for x in gen.lengths(cfg, 0)]
    bm = _paged(lengths, bs)
    waste = capacity.waste_per_request(bm, range(len(lengths)))
    assert all(0 <= w < bs for w in waste)
    assert abs(np.mean(waste) - (bs - 1) / 2) < bs / 4
    tokens = sum(lengths)
    paged = capacity.utilisation(tokens, capacity.paged_slots(bm, range(len(lengths))))
    reserved = capacity.utilisation(tokens, capacity.reserved_slots(lengths, 2048))
    assert paged >= 1 - bs / min(lengths) and 0.204 <= reserved <= 0.382


def test_active_requests_in_the_page_pool():
    """22,048 tokens of KV: 34 requests of 512 + 128 tokens paged at block 16
    (the page's figure), 10 when each reserves 2,048."""
    per_request = -(-640 // 16) * 16
    assert capacity.n_active(22048, per_request) == 34
    assert capacity.n_active(22048, 2048) == 10


def test_shared_blocks_count_once():
    bm = BlockManager(8, 4, range(8))
    bm.add_seq(0)
    bm.append_slots(0, 10)
    bm.fork(0, 1)
    assert capacity.paged_slots(bm, [0, 1]) == 12
