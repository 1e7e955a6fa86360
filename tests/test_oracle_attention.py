"""Pins of the oracle's attention: torch's float64 scaled_dot_product_attention,
closed forms, permutation invariance of the physical blocks, softmax rows."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention, encoding
from oracle.block_manager import BlockManager
from oracle.pool import Pool


def _paged_world(rng, lengths, H_kv, d, bs, dtype, n_blocks=None, order=None):
    """Scatter contiguous per-sequence K/V into a pool through the allocator.

    Returns the pool, block tables and the contiguous K/V (float64, exactly
    the values the pool holds)."""
    need = sum(-(-n // bs) for n in lengths)
    n_blocks = n_blocks or need + 7
    order = rng.permutation(n_blocks) if order is None else order
    bm = BlockManager(n_blocks, bs, order)
    pool = Pool(1, H_kv, n_blocks, bs, d, dtype)
    kc, vc = [], []
    for i, n in enumerate(lengths):
        bm.add_seq(i)
        slots, _ = bm.append_slots(i, n)
        k = rng.standard_normal((n, H_kv, d)).astype(np.float32)
        v = rng.standard_normal((n, H_kv, d)).astype(np.float32)
        pool.append(0, encoding.encode(k, dtype), encoding.encode(v, dtype), slots)
        kc.append(encoding.decode(encoding.encode(k, dtype), dtype))
        vc.append(encoding.decode(encoding.encode(v, dtype), dtype))
    tables = [bm.block_table(i) for i in range(len(lengths))]
    return pool, tables, kc, vc


def _sdpa(q, k, v, scale, causal=False):
    """torch SDPA in float64 on CPU. q [H_q][Lq][d], k/v [H_kv][Lk][d]."""
    G = q.shape[0] // k.shape[0]
    out = F.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        is_causal=causal, scale=scale, enable_gqa=G > 1)
    return out[0].numpy()


@pytest.mark.parametrize("H_q,H_kv,d,bs,dtype", [
    (4, 4, 64, 16, "f32"), (16, 8, 128, 16, "bf16"), (8, 1, 32, 8, "f16"), (6, 2, 16, 3, "bf16"),
    (40, 40, 128, 32, "bf16"),
])
def test_paged_decode_equals_sdpa_on_contiguous(H_q, H_kv, d, bs, dtype):
    rng = np.random.default_rng(H_q * 1000 + d + bs)
    lengths = [1, bs - 1 if bs > 1 else 1, bs, bs + 1, 5 * bs + 3, 100]
    pool, tables, kc, vc = _paged_world(rng, lengths, H_kv, d, bs, dtype)
    q = rng.standard_normal((len(lengths), H_q, d))
    scale = float(np.float32(1 / np.sqrt(d)))
    got = attention.decode(pool, 0, q, tables, lengths, scale)
    for i, n in enumerate(lengths):
        ref = _sdpa(q[i][:, None, :], kc[i].transpose(1, 0, 2), vc[i].transpose(1, 0, 2), scale)[:, 0, :]
        np.testing.assert_allclose(got[i], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("ctx_before,T,G", [(0, 7, 1), (13, 5, 2), (37, 33, 4), (64, 16, 8)])
def test_prefill_chunk_equals_last_rows_of_causal_sdpa(ctx_before, T, G):
    """A chunk after ctx_before cached tokens equals the last T rows of full
    causal attention over all ctx_before + T positions."""
    rng = np.random.default_rng(ctx_before * 7 + T)
    H_kv, d, bs = 2, 32, 16
    H_q = H_kv * G
    n = ctx_before + T
    pool, tables, kc, vc = _paged_world(rng, [n], H_kv, d, bs, "bf16")
    q_all = rng.standard_normal((n, H_q, d))
    scale = 0.3
    got = attention.prefill_chunk(pool, 0, q_all[ctx_before:], tables[0], ctx_before, scale)
    ref = _sdpa(q_all.transpose(1, 0, 2), kc[0].transpose(1, 0, 2), vc[0].transpose(1, 0, 2), scale, causal=True)
    np.testing.assert_allclose(got, ref.transpose(1, 0, 2)[ctx_before:], rtol=0, atol=1e-12)


def test_permuting_physical_blocks_changes_nothing():
    rng = np.random.default_rng(5)
    lengths = [3, 17, 40, 64]
    bs, H_kv, d = 8, 2, 16
    pool, tables, _, _ = _paged_world(rng, lengths, H_kv, d, bs, "bf16", n_blocks=30)
    q = rng.standard_normal((len(lengths), 4, d))
    base = attention.decode(pool, 0, q, tables, lengths, 0.25)
    for trial in range(5):
        perm = rng.permutation(pool.N)  # physical block b moves to perm[b]
        p2 = Pool(1, H_kv, pool.N, bs, d, "bf16")
        p2.k[:, :, perm] = pool.k
        p2.v[:, :, perm] = pool.v
        t2 = [[int(perm[b]) for b in t] for t in tables]
        got = attention.decode(p2, 0, q, t2, lengths, 0.25)
        assert np.array_equal(got, base)


def test_closed_forms():
    rng = np.random.default_rng(11)
    H_kv, d, bs = 2, 16, 4
    lengths = [1, 9]
    pool, tables, kc, vc = _paged_world(rng, lengths, H_kv, d, bs, "f32")
    q = rng.standard_normal((2, 4, d))
    out = attention.decode(pool, 0, q, tables, lengths, 0.7)
    # one visible token: the output is that token's V row, exactly
    for h in range(4):
        assert np.array_equal(out[0, h], vc[0][0, h // 2])
    # scale 0: every visible token weighs the same -> mean of the visible V
    out0 = attention.decode(pool, 0, q, tables, lengths, 0.0)
    for h in range(4):
        np.testing.assert_allclose(out0[1, h], vc[1][:, h // 2].mean(axis=0), rtol=0, atol=1e-14)
    # one dominant logit: the output is (to within e^-huge) that token's V row
    k = np.zeros((1, 9, d))
    k[0, 4, 0] = 1.0
    qd = np.zeros((1, d))
    qd[0, 0] = 1.0
    v = rng.standard_normal((1, 9, d))
    o = attention.attend(qd, k, v, 800.0)
    np.testing.assert_allclose(o[0], v[0, 4], rtol=0, atol=1e-300)
    # a sequence with nothing visible writes zeros
    assert np.array_equal(attention.attend(q[0], np.zeros((2, 0, d)), np.zeros((2, 0, d)), 1.0), np.zeros((4, d)))


def test_softmax_rows_sum_to_one_and_large_logits_are_safe():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((6, 8)) * 50
    k = rng.standard_normal((3, 200, 8)) * 50
    p = attention.softmax_weights(q, k, 1.0)
    assert np.all(np.isfinite(p))
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p >= 0)


def test_unused_slots_are_never_read():
    """The pool starts NaN-filled; gathers through the tables never touch the
    unused tail of a last block or any free block."""
    rng = np.random.default_rng(21)
    lengths = [5, 16, 33]
    pool, tables, kc, vc = _paged_world(rng, lengths, 2, 8, 16, "bf16", n_blocks=12)
    assert np.isnan(encoding.decode(pool.k, "bf16")).any()
    out = attention.decode(pool, 0, rng.standard_normal((3, 2, 8)), tables, lengths, 0.5)
    assert np.all(np.isfinite(out))


def test_gqa_group_mapping_is_contiguous():
    """Query heads h = g*G .. g*G+G-1 read KV head g (checked against torch's
    enable_gqa by giving each KV head a distinct constant V)."""
    d, G, H_kv = 4, 3, 2
    k = np.zeros((H_kv, 5, d))
    v = np.zeros((H_kv, 5, d))
    v[0] += 1.0
    v[1] += 2.0
    q = np.ones((G * H_kv, d))
    out = attention.attend(q, k, v, 1.0)
    ref = _sdpa(q[:, None, :], k, v, 1.0)[:, 0, :]
    np.testing.assert_array_equal(out, ref)
    assert out[:G].max() == 1.0 and out[G:].min() == 2.0
