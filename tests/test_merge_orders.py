"""CPU model of the XCD-aware orders (csrc/pa_common.h merge_row; the split
branch of prefill_chunk_kernel in csrc/pa_prefill.hip): every merge
workgroup takes a distinct row and every (item, split) of a split prefill
runs exactly once, and with H_kv a multiple of 8 a KV head's rows and
workgroups all sit on the XCD its index picks (workgroup L runs on XCD
L mod 8)."""

import itertools

import pytest


def merge_row(L, H_q, H_kv):
    G = H_q // H_kv
    g = L % H_kv
    rest = L // H_kv
    return (rest // G) * H_q + g * G + rest % G


def split_item(L, ntiles, H_kv):
    rest = L // H_kv
    return (L % H_kv) * ntiles + rest % ntiles, rest // ntiles


@pytest.mark.parametrize("B,H_q,H_kv", [(1, 8, 8), (3, 32, 8), (64, 40, 40), (5, 64, 8), (7, 12, 3), (4, 16, 1)])
def test_merge_row_is_a_permutation_keeping_heads_on_their_xcd(B, H_q, H_kv):
    rows = [merge_row(L, H_q, H_kv) for L in range(B * H_q)]
    assert sorted(rows) == list(range(B * H_q))
    G = H_q // H_kv
    for L, row in enumerate(rows):
        g = (row % H_q) // G
        assert L % H_kv == g
        if H_kv % 8 == 0:
            assert L % 8 == g % 8


@pytest.mark.parametrize("ntiles,H_kv,splits", list(itertools.product([1, 2, 7], [1, 8, 40], [2, 5, 12])))
def test_split_prefill_order_runs_each_item_and_split_once(ntiles, H_kv, splits):
    seen = [split_item(L, ntiles, H_kv) for L in range(ntiles * H_kv * splits)]
    assert sorted(seen) == sorted(itertools.product(range(ntiles * H_kv), range(splits)))
    if H_kv % 8 == 0:
        for L, (item, _) in enumerate(seen):
            assert L % 8 == (item // ntiles) % 8  # the item's KV head picks the XCD, as in the merge


def test_a_plausible_mistake_is_caught():
    """Swapping the two inner indices of merge_row breaks the XCD pairing."""
    def wrong(L, H_q, H_kv):
        G = H_q // H_kv
        rest = L // H_kv
        return (rest // G) * H_q + (rest % G) * H_kv + L % H_kv
    rows = [wrong(L, 32, 8) for L in range(3 * 32)]
    assert sorted(rows) == list(range(96))  # still a permutation
    assert any(L % 8 != (row % 32) // 4 for L, row in enumerate(rows))  # but heads leave their XCD
