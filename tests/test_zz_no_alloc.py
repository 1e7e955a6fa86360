"""pa_decode_noalloc (no workspace argument; the split partials live in the
library's static per-GPU scratch) against pa_decode with a workspace: bit
for bit on two calls in a row, the second smaller, and against the oracle."""

import numpy as np
import pytest
import torch

from gpu_util import TOL, bits, f64, max_abs_err, say
from oracle import attention, encoding
from oracle.block_manager import BlockManager as OracleBM
from oracle.pool import Pool
from oracle.run import widen

pytestmark = pytest.mark.gpu


def _world(rng, lengths, H_q, H_kv, d, bs):
    from paged_kv_cache_140_amd import KVPool

    N = sum(-(-n // bs) for n in lengths) + 7
    bm = OracleBM(N, bs, rng.permutation(N))
    op = Pool(1, H_kv, N, bs, d, "bf16")
    for i, n in enumerate(lengths):
        bm.add_seq(i)
        slots, _ = bm.append_slots(i, n)
        k = rng.standard_normal((n, H_kv, d)).astype(np.float32)
        v = rng.standard_normal((n, H_kv, d)).astype(np.float32)
        op.append(0, encoding.encode(k, "bf16"), encoding.encode(v, "bf16"), slots)
    tables = [bm.block_table(i) for i in range(len(lengths))]
    gp = KVPool(1, H_kv, N, bs, d, "bf16")
    gp.k.view(torch.int16).copy_(torch.from_numpy(op.k.view(np.int16)))
    gp.v.view(torch.int16).copy_(torch.from_numpy(op.v.view(np.int16)))
    tab = np.zeros((len(lengths), max(len(t) for t in tables)), dtype=np.int32)
    for i, t in enumerate(tables):
        tab[i, :len(t)] = t
    return op, gp, tables, torch.from_numpy(tab).cuda()


@pytest.mark.parametrize("H_q,H_kv", [(16, 8), (64, 8)])
def test_noalloc_decode_matches_workspace_decode(H_q, H_kv):
    import paged_kv_cache_140_amd as pa
    from paged_kv_cache_140_amd.runner import to_device

    d, bs, scale = 128, 16, float(np.float32(1 / np.sqrt(128)))
    rng = np.random.default_rng(11 + H_q)
    # a first call and a smaller second one; both split into partitions
    for lengths in ([5000, 3000, 700], [1500, 90]):
        B = len(lengths)
        op, gp, tables, tab = _world(rng, lengths, H_q, H_kv, d, bs)
        lens = torch.tensor(lengths, dtype=torch.int32).cuda()
        max_ctx = max(lengths)
        assert pa.pa_decode_workspace_size(gp, B, H_q, max_ctx) > 0, "the case must split"
        q32 = rng.standard_normal((B, H_q, d)).astype(np.float32)
        q = to_device(q32, "bf16", "cuda")
        say("noalloc decode", H_q, H_kv, lengths)
        ref_out = torch.full_like(q, float("nan"))
        ws = pa.decode_workspace(gp, B, H_q, max_ctx)
        pa.pa_decode(gp, 0, ref_out, q, tab, lens, max_ctx, scale, ws)
        out = torch.full_like(q, float("nan"))
        pa.pa_decode_noalloc(gp, 0, out, q, tab, lens, max_ctx, scale)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), bits(ref_out))
        ref = attention.decode(op, 0, widen(q32, "bf16"), tables, lengths, scale)
        err = max_abs_err(f64(out), ref)
        say("  max abs err", err)
        assert err <= TOL["bf16"]


def test_noalloc_decode_rejects_a_split_larger_than_its_scratch(tune):
    import paged_kv_cache_140_amd as pa
    from paged_kv_cache_140_amd import _lib

    tune(decode_part_blocks=1)  # 1,024 partitions of one block each
    B, H_q, H_kv, d, bs, max_ctx = 64, 64, 8, 128, 16, 16384
    gp = pa.KVPool(1, H_kv, 64, bs, d, "bf16")
    assert pa.pa_decode_workspace_size(gp, B, H_q, max_ctx) > _lib.PA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, H_q, d, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros_like(q)
    tab = torch.zeros(B, max_ctx // bs, dtype=torch.int32, device="cuda")
    lens = torch.full((B,), max_ctx, dtype=torch.int32, device="cuda")
    say("noalloc decode: oversized split rejected on the host")
    with pytest.raises(pa.PAError) as e:
        pa.pa_decode_noalloc(gp, 0, out, q, tab, lens, max_ctx, 0.1)
    assert e.value.status == _lib.PA_ESPACE
    torch.cuda.synchronize()
    assert int(out.abs().sum().item()) == 0  # nothing launched
