"""Automatic prefix caching end to end: a later request reuses the blocks
that hold an earlier request's K/V for the same prefix and computes only the
rest ([ttlab] "llm-kv-cache-02-serving-engine-kv", section "4. 프리픽스 캐시";
[icarus] "PagedAttention", section "支持块级共享").  The page's workload: a
3,000-token shared prefix, 32 unique tokens per request, block size 16.

The reused request's prefill chunk (its last 40 positions: 8 prefix tokens of
the partly shared block + 32 tail tokens) and its next decode step run in the
HIP kernels over a table whose first 187 blocks belong to the first request;
the oracle attends over the request's whole K/V laid out contiguously."""

import numpy as np
import pytest
import torch

from gpu_util import TOL, bits, f64, max_abs_err, say
from oracle import attention, encoding
from oracle.block_manager import BlockManager as OracleBM
from oracle.pool import Pool
from oracle.run import widen

pytestmark = pytest.mark.gpu

BS, H_KV, H_Q, D, N = 16, 8, 32, 128, 700


def _kv(rng, n):
    return (rng.standard_normal((n, H_KV, D)).astype(np.float32),
            rng.standard_normal((n, H_KV, D)).astype(np.float32))


@pytest.mark.parametrize("first_alive", [True, False], ids=["first-request-live", "first-request-freed"])
def test_prefix_hit_prefill_and_decode_match_oracle(first_alive):
    from paged_kv_cache_140_amd import (BlockManager, KVPool, decode_workspace, pa_cache_append, pa_decode,
                                        pa_prefill_chunk, prefill_workspace)
    from paged_kv_cache_140_amd.runner import to_device

    rng = np.random.default_rng(3000)
    order = rng.permutation(N)
    prefix = [int(x) for x in rng.integers(0, 150000, 3000)]
    tails = [[int(x) for x in rng.integers(0, 150000, 32)] for _ in range(2)]
    pk, pv = _kv(rng, 3000)  # the shared prefix's K/V (equal prefixes, equal K/V)
    tk = [_kv(rng, 32) for _ in range(2)]
    scale = float(np.float32(1 / np.sqrt(D)))

    ob, lb = OracleBM(N, BS, order), BlockManager(N, BS, order)
    op = Pool(1, H_KV, N, BS, D, "bf16")
    gp = KVPool(1, H_KV, N, BS, D, "bf16")
    gp.k.fill_(float("nan"))
    gp.v.fill_(float("nan"))

    def append(seq, toks, k, v):
        so, po = ob.append_tokens(seq, toks)
        sl, pl = lb.append_tokens(seq, toks)
        assert list(sl) == so and pl == po == []
        op.append(0, encoding.encode(k, "bf16"), encoding.encode(v, "bf16"), so)
        pa_cache_append(gp, 0, to_device(k, "bf16", "cuda"), to_device(v, "bf16", "cuda"),
                        torch.from_numpy(np.asarray(sl, dtype=np.int32)).cuda())

    # first request: nothing cached, the whole prompt is computed
    say("prefix cache: first request")
    prompt0 = prefix + tails[0]
    assert ob.add_seq_prefix(0, prompt0) == lb.add_seq_prefix(0, prompt0) == 0
    append(0, prompt0, np.concatenate([pk, tk[0][0]]), np.concatenate([pv, tk[0][1]]))
    assert lb.num_cached() == ob.num_cached() == 189
    shared = lb.block_table(0)[:187]
    if not first_alive:
        ob.free_seq(0)
        lb.free_seq(0)
    before = bits(gp.k[0, :, shared]), bits(gp.v[0, :, shared])

    # second request: 187 cached blocks found, 40 positions computed
    prompt1 = prefix + tails[1]
    hit = lb.add_seq_prefix(1, prompt1)
    assert hit == ob.add_seq_prefix(1, prompt1) == 2992
    assert lb.block_table(1) == shared
    k1 = np.concatenate([pk[2992:], tk[1][0]])
    v1 = np.concatenate([pv[2992:], tk[1][1]])
    append(1, prompt1[hit:], k1, v1)
    table = lb.block_table(1)
    assert table[:187] == shared and table == ob.block_table(1)
    q32 = rng.standard_normal((40, H_Q, D)).astype(np.float32)
    q = to_device(q32, "bf16", "cuda")
    out = torch.full_like(q, float("nan"))
    say("prefix cache: prefill chunk of 40 after 2,992 cached tokens")
    ws = prefill_workspace(gp, 40, H_Q, hit)
    assert ws is not None  # 8 position tiles would leave most CUs idle: the keys are split
    pa_prefill_chunk(gp, 0, out, q, torch.tensor(table, dtype=torch.int32).cuda(), hit, scale, ws)
    torch.cuda.synchronize()
    kc = widen(np.concatenate([pk[:3000], tk[1][0]]), "bf16").transpose(1, 0, 2)
    vc = widen(np.concatenate([pv[:3000], tk[1][1]]), "bf16").transpose(1, 0, 2)
    ref = attention.causal_rows(widen(q32, "bf16"), kc, vc, hit, scale, list(range(40)))
    err = max_abs_err(f64(out), ref)
    say("  max abs err", err)
    assert err <= TOL["bf16"]
    # the shared blocks were read, never written
    assert np.array_equal(bits(gp.k[0, :, shared]), before[0]) and np.array_equal(bits(gp.v[0, :, shared]), before[1])
    assert np.array_equal(bits(gp.k).reshape(-1), op.k.reshape(-1))

    # its next decode step: one new token, attention over all 3,033 tokens
    nk, nv = _kv(rng, 1)
    append(1, [7], nk, nv)
    qd32 = rng.standard_normal((1, H_Q, D)).astype(np.float32)
    qd = to_device(qd32, "bf16", "cuda")
    outd = torch.full_like(qd, float("nan"))
    table = lb.block_table(1)
    say("prefix cache: decode at 3,033 tokens")
    pa_decode(gp, 0, outd, qd, torch.tensor([table], dtype=torch.int32).cuda(),
              torch.tensor([3033], dtype=torch.int32).cuda(), 3033, scale, decode_workspace(gp, 1, H_Q, 3033))
    torch.cuda.synchronize()
    kd = np.concatenate([kc, widen(nk, "bf16").transpose(1, 0, 2)], axis=1)
    vd = np.concatenate([vc, widen(nv, "bf16").transpose(1, 0, 2)], axis=1)
    refd = attention.attend(widen(qd32, "bf16")[0], kd, vd, scale)
    errd = max_abs_err(f64(outd)[0], refd)
    say("  max abs err", errd)
    assert errd <= TOL["bf16"]
