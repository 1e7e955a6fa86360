"""Pins of the oracle's pool writes ([icarus] "Block Table 如何工作" for the
slot a new token goes to; [icarus] "支持块级共享" and [ttlab] "블록을 함께
쓰기" for copy-on-write duplicating a whole block): checked element by element
against positions written out by hand on a pool whose every element is
distinct."""

import numpy as np

from oracle.pool import Pool

L, H, N, BS, D = 3, 2, 6, 4, 5


def _numbered_pool():
    """K element (l, h, b, o, e) holds its own flat index; V holds 10^6 more."""
    p = Pool(L, H, N, BS, D, "f32", fill_bits=0)
    idx = np.arange(L * H * N * BS * D, dtype=np.uint32).reshape(p.k.shape)
    p.k[...] = idx
    p.v[...] = idx + 10**6
    return p, idx


def test_copy_duplicates_every_layer_head_and_both_tensors():
    p, idx = _numbered_pool()
    p.copy_blocks([(1, 4)])
    for layer in range(L):
        for h in range(H):
            for b in range(N):
                src = 1 if b == 4 else b  # block 4 now holds block 1; the rest are untouched
                assert np.array_equal(p.k[layer, h, b], idx[layer, h, src])
                assert np.array_equal(p.v[layer, h, b], idx[layer, h, src] + 10**6)


def test_copies_apply_in_order():
    p, idx = _numbered_pool()
    p.copy_blocks([(0, 2), (2, 5), (3, 0)])
    assert np.array_equal(p.k[:, :, 5], idx[:, :, 0])  # through block 2, which held block 0 by then
    assert np.array_equal(p.k[:, :, 2], idx[:, :, 0])
    assert np.array_equal(p.k[:, :, 0], idx[:, :, 3])
    assert np.array_equal(p.v[:, :, 5], idx[:, :, 0] + 10**6)


def test_append_writes_slot_block_and_offset():
    p = Pool(2, H, N, BS, D, "f32", fill_bits=0)
    rows = np.arange(4 * H * D, dtype=np.uint32).reshape(4, H, D) + 1
    # slot 9 = block 2, offset 1; slot 3 = block 0, offset 3; -1 = no write;
    # slot 9 again: the later row wins
    p.append(1, rows, rows + 100, [9, 3, -1, 9])
    want_k = np.zeros_like(p.k)
    want_k[1, :, 2, 1] = rows[3]
    want_k[1, :, 0, 3] = rows[1]
    assert np.array_equal(p.k, want_k)
    want_v = np.zeros_like(p.v)
    want_v[1, :, 2, 1] = rows[3] + 100
    want_v[1, :, 0, 3] = rows[1] + 100
    assert np.array_equal(p.v, want_v)
