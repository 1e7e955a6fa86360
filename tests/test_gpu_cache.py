"""pa_cache_append and pa_copy_blocks against the oracle: pools bit-exact,
including NaN-poisoned slots the writes must not touch."""

import numpy as np
import pytest
import torch

from gpu_util import bits, say
from oracle import encoding
from oracle.block_manager import BlockManager as OracleBM
from oracle.pool import Pool
from oracle.run import OracleRun
from pa_inputs import build_scenario

pytestmark = pytest.mark.gpu


def _pools_equal(gpu_pool, oracle_pool):
    assert np.array_equal(bits(gpu_pool.k), oracle_pool.k)
    assert np.array_equal(bits(gpu_pool.v), oracle_pool.v)


@pytest.mark.parametrize("cid,over", [(1, {}), (2, {}), (4, dict(prompts=2, samples=4, prefix=100, tail=7, steps=3,
                                                                   num_blocks=80))])
def test_append_and_copy_on_workloads(cid, over):
    from paged_kv_cache_140_amd.runner import DeviceRun

    scn = build_scenario(cid, 0, **over)
    say("append/copy", cid, over)
    orc = OracleRun(scn)
    orc.run_setup()
    gpu = DeviceRun(scn)
    gpu.run_setup()
    torch.cuda.synchronize()
    _pools_equal(gpu.pool, orc.pool)
    for st in scn.steps:
        ores = orc.run_step(st, decode_rows=[])
        si = gpu.prepare(st)
        assert list(si.host_slots) == ores.slots
        assert [tuple(p) for p in si.host_pairs.tolist()] == ores.pairs
        gpu.launch(si, do_decode=False, do_prefill=False)
        torch.cuda.synchronize()
        _pools_equal(gpu.pool, orc.pool)


@pytest.mark.parametrize("dtype,d,bs,L,H", [("bf16", 128, 16, 3, 8), ("f32", 64, 8, 2, 4), ("f16", 64, 32, 1, 5),
                                            ("bf16", 64, 8, 2, 3)])
def test_append_random_slots_and_skips(dtype, d, bs, L, H):
    from paged_kv_cache_140_amd import KVPool, pa_cache_append

    rng = np.random.default_rng(d + bs + L)
    N = 64
    say("append random", dtype, d, bs, L, H)
    op = Pool(L, H, N, bs, d, dtype)
    gp = KVPool(L, H, N, bs, d, dtype)
    gp.k.fill_(float("nan"))
    gp.v.fill_(float("nan"))
    for layer in range(L):
        for T in (0, 1, 7, 300):
            slots = rng.choice(N * bs, size=T, replace=False).astype(np.int32)
            if T > 2:
                slots[::3] = -1  # skipped rows
            k = rng.standard_normal((T, H, d)).astype(np.float32)
            v = rng.standard_normal((T, H, d)).astype(np.float32)
            op.append(layer, encoding.encode(k, dtype), encoding.encode(v, dtype), slots)
            from paged_kv_cache_140_amd.runner import to_device

            pa_cache_append(gp, layer, to_device(k, dtype, "cuda"), to_device(v, dtype, "cuda"),
                            torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    _pools_equal(gp, op)


@pytest.mark.parametrize("dtype,d,bs,L,H,n", [("bf16", 128, 16, 1, 8, 56), ("bf16", 128, 32, 4, 2, 9),
                                              ("f32", 64, 8, 2, 3, 1), ("f16", 64, 16, 3, 1, 20)])
def test_copy_blocks_bit_exact(dtype, d, bs, L, H, n):
    from paged_kv_cache_140_amd import KVPool, pa_copy_blocks

    rng = np.random.default_rng(n + bs)
    N = 3 * n + 5
    say("copy", dtype, d, bs, L, H, n)
    op = Pool(L, H, N, bs, d, dtype)
    rand = rng.integers(0, 2**16 if dtype != "f32" else 2**32, size=op.k.shape, dtype=np.uint64)
    op.k[...] = rand.astype(op.k.dtype)
    op.v[...] = (rand[::-1]).astype(op.v.dtype)
    gp = KVPool(L, H, N, bs, d, dtype)
    view = torch.int32 if dtype == "f32" else torch.int16
    gp.k.view(view).copy_(torch.from_numpy(op.k.view(np.int32 if dtype == "f32" else np.int16)))
    gp.v.view(view).copy_(torch.from_numpy(op.v.view(np.int32 if dtype == "f32" else np.int16)))
    blocks = rng.permutation(N)
    pairs = np.stack([blocks[:n], blocks[n:2 * n]], axis=1).astype(np.int32)  # disjoint src / dst
    op.copy_blocks(pairs)
    pa_copy_blocks(gp, torch.from_numpy(pairs).cuda())
    pa_copy_blocks(gp, torch.zeros((0, 2), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    _pools_equal(gp, op)


def test_cow_then_append_keeps_sharers_intact():
    """Fork, copy-on-write, append: every sequence still gathers its own history
    (GPU pool compared with the oracle pool, bit for bit)."""
    from paged_kv_cache_140_amd import BlockManager, KVPool, pa_cache_append, pa_copy_blocks
    from paged_kv_cache_140_amd.runner import to_device

    rng = np.random.default_rng(77)
    N, bs, H, d = 40, 16, 2, 128
    order = rng.permutation(N)
    ob, lb = OracleBM(N, bs, order), BlockManager(N, bs, order)
    op, gp = Pool(1, H, N, bs, d, "bf16"), KVPool(1, H, N, bs, d, "bf16")
    gp.k.fill_(float("nan"))
    gp.v.fill_(float("nan"))
    say("cow sequence")

    def write(seq, n):
        so, po = ob.append_slots(seq, n)
        sl, pl = lb.append_slots(seq, n)
        assert list(sl) == so and pl == po
        k = rng.standard_normal((n, H, d)).astype(np.float32)
        v = rng.standard_normal((n, H, d)).astype(np.float32)
        op.copy_blocks(po)
        op.append(0, encoding.encode(k, "bf16"), encoding.encode(v, "bf16"), so)
        if pl:
            pa_copy_blocks(gp, torch.tensor(pl, dtype=torch.int32, device="cuda"))
        pa_cache_append(gp, 0, to_device(k, "bf16", "cuda"), to_device(v, "bf16", "cuda"),
                        torch.from_numpy(np.asarray(sl, dtype=np.int32)).cuda())

    for s in (0,):
        ob.add_seq(s)
        lb.add_seq(s)
    write(0, 37)
    for c in (1, 2, 3):
        ob.fork(0, c)
        lb.fork(0, c)
    for s in (2, 0, 3, 1):
        write(s, 5)
    write(1, 20)
    torch.cuda.synchronize()
    _pools_equal(gp, op)
