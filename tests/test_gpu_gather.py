"""pa_gather_checksum (pa_decode's walk and loads without the arithmetic, the
benchmark's access-pattern ceiling) reads exactly the visible K/V: the XOR
of each (sequence, KV head)'s per-wave checksums equals, bit for bit, the
XOR of the K and V dwords of its visible tokens gathered through the block
table on the CPU (context lengths that fill whole 16-token units), for
single-partition and split plans, at 4 and 8 waves per workgroup (the
library's own choices for one partition and for a split)."""

import numpy as np
import pytest
import torch

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H_q,H_kv,d,bs,lengths,part_blocks", [
    (16, 8, 128, 16, [512, 640, 16, 576], None),
    (40, 40, 128, 16, [1024, 32, 2048], None),
    (64, 8, 128, 16, [4096, 1024, 32768], None),
    (16, 8, 128, 32, [640, 64, 96], 3),
    (32, 8, 64, 8, [160, 48, 992], 5),
    # a split plan that the device runs unsplit (40 balanced long contexts):
    # the empty partition slots' checksums are written as 0
    (16, 8, 128, 16, [4096 + 16 * (i % 5) for i in range(40)], None),
])
@pytest.mark.parametrize("waves", [4, 8])
def test_gather_checksum_reads_every_visible_token_once(H_q, H_kv, d, bs, lengths, part_blocks, waves, tune):
    import paged_kv_cache_140_amd as pa

    tune(decode_waves=waves)
    if part_blocks:
        tune(decode_part_blocks=part_blocks)
    rng = np.random.default_rng(sum(lengths) + d)
    need = sum(-(-n // bs) for n in lengths)
    N = need + 5
    order = rng.permutation(N)
    tables, pos = [], 0
    for n in lengths:
        nb = -(-n // bs)
        tables.append(order[pos:pos + nb])
        pos += nb
    pool = pa.KVPool(1, H_kv, N, bs, d, "bf16")
    bits_k = rng.integers(0, 1 << 16, size=pool.k.shape, dtype=np.uint16)
    bits_v = rng.integers(0, 1 << 16, size=pool.v.shape, dtype=np.uint16)
    pool.k.view(torch.int16).copy_(torch.from_numpy(bits_k.view(np.int16)))
    pool.v.view(torch.int16).copy_(torch.from_numpy(bits_v.view(np.int16)))
    maxb = max(len(t) for t in tables)
    tab = np.zeros((len(lengths), maxb), dtype=np.int32)
    for i, t in enumerate(tables):
        tab[i, :len(t)] = t
    say("gather checksum", H_q, H_kv, d, bs, lengths, part_blocks, waves)
    cs = pa.pa_gather_checksum(pool, 0, H_q, torch.from_numpy(tab).cuda(),
                               torch.tensor(lengths, dtype=torch.int32).cuda(), max(lengths))
    torch.cuda.synchronize()
    W = waves  # the decode plan's waves per workgroup
    got = cs.cpu().numpy().view(np.uint32).reshape(len(lengths), -1, H_kv, W)  # [B][P][H_kv][W]
    got = np.bitwise_xor.reduce(np.bitwise_xor.reduce(got, axis=3), axis=1)  # [B][H_kv]
    for i, n in enumerate(lengths):
        blocks = tab[i, :-(-n // bs)]
        for g in range(H_kv):
            k = bits_k[0, g, blocks].reshape(-1, d)[:n]
            v = bits_v[0, g, blocks].reshape(-1, d)[:n]
            want = np.bitwise_xor.reduce(np.ascontiguousarray(k).view(np.uint32).ravel()) ^ \
                np.bitwise_xor.reduce(np.ascontiguousarray(v).view(np.uint32).ravel())
            assert got[i, g] == want, (i, g)
