"""pa_prefill_chunk against the oracle: causal chunk attention over paged K/V."""

import numpy as np
import pytest
import torch

from gpu_util import TOL, f64, max_abs_err, say
from oracle import attention, encoding
from oracle.block_manager import BlockManager as OracleBM
from oracle.pool import Pool
from oracle.run import widen
from pa_inputs import build_scenario

pytestmark = pytest.mark.gpu


def _chunk_world(rng, total, H_kv, d, bs, dtype, extra_blocks=9):
    from paged_kv_cache_140_amd import KVPool

    N = -(-total // bs) + extra_blocks
    bm = OracleBM(N, bs, rng.permutation(N))
    op = Pool(1, H_kv, N, bs, d, dtype)
    bm.add_seq(0)
    slots, _ = bm.append_slots(0, total)
    k = rng.standard_normal((total, H_kv, d)).astype(np.float32)
    v = rng.standard_normal((total, H_kv, d)).astype(np.float32)
    op.append(0, encoding.encode(k, dtype), encoding.encode(v, dtype), slots)
    gp = KVPool(1, H_kv, N, bs, d, dtype)
    gp.k.view(torch.int16).copy_(torch.from_numpy(op.k.view(np.int16)))
    gp.v.view(torch.int16).copy_(torch.from_numpy(op.v.view(np.int16)))
    return op, gp, bm.block_table(0)


def _run(gp, q32, table, ctx_before, scale, dtype, pad_table=0, split=False):
    """split: pass the workspace, so that a chunk with few position tiles is
    cut over its keys and merged."""
    from paged_kv_cache_140_amd import pa_prefill_chunk, prefill_workspace
    from paged_kv_cache_140_amd.runner import to_device

    q = to_device(q32, dtype, "cuda")
    out = torch.full_like(q, float("nan"))
    tab = np.asarray(list(table) + [0] * pad_table, dtype=np.int32)
    ws = prefill_workspace(gp, q.shape[0], q.shape[1], ctx_before) if split else None
    if ws is not None:
        ws.fill_(255)  # NaN patterns: a merge that read an unwritten split would show
    pa_prefill_chunk(gp, 0, out, q, torch.from_numpy(tab).cuda(), ctx_before, scale, ws)
    torch.cuda.synchronize()
    return out


CASES = [
    # H_q, H_kv, d, bs, dtype, ctx_before, T
    (64, 8, 128, 16, "bf16", 100, 70),
    (64, 8, 128, 16, "bf16", 0, 33),
    (16, 8, 128, 16, "bf16", 513, 130),
    (8, 8, 128, 8, "bf16", 37, 129),
    (32, 8, 64, 32, "bf16", 64, 64),
    (16, 4, 64, 16, "f16", 250, 77),
    (4, 1, 128, 32, "f16", 1, 1),
    (8, 2, 128, 16, "bf16", 1000, 17),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[4]}-hq{c[0]}-hkv{c[1]}-d{c[2]}-bs{c[3]}-c{c[5]}-t{c[6]}"
                                             for c in CASES])
@pytest.mark.parametrize("split", [False, True], ids=["one-pass", "key-split"])
def test_prefill_chunk_small(case, split):
    H_q, H_kv, d, bs, dtype, ctx_before, T = case
    rng = np.random.default_rng(ctx_before * 31 + T)
    say("prefill", case, "split" if split else "")
    op, gp, table = _chunk_world(rng, ctx_before + T, H_kv, d, bs, dtype)
    q32 = rng.standard_normal((T, H_q, d)).astype(np.float32)
    scale = float(np.float32(1 / np.sqrt(d)))
    out = _run(gp, q32, table, ctx_before, scale, dtype, pad_table=3, split=split)
    ref = attention.prefill_chunk(op, 0, widen(q32, dtype), table, ctx_before, scale)
    err = max_abs_err(f64(out), ref)
    say("  max abs err", err)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("ctx_before", [3500, 2476])
def test_prefill_chunk_full_size_sampled_rows(ctx_before):
    """The mixed batch's chunk: 1,024 rows, 64 query / 8 KV heads, after
    3,500 cached tokens (and the reading where the chunk is the last 1,024 of
    3,500).  Sampled rows against the oracle."""
    rng = np.random.default_rng(ctx_before)
    H_q, H_kv, d, bs, T = 64, 8, 128, 16, 1024
    say("prefill full", ctx_before)
    op, gp, table = _chunk_world(rng, ctx_before + T, H_kv, d, bs, "bf16")
    q32 = rng.standard_normal((T, H_q, d)).astype(np.float32)
    scale = float(np.float32(1 / np.sqrt(d)))
    out = f64(_run(gp, q32, table, ctx_before, scale, "bf16"))
    rows = [0, 1, 15, 16, 17, 500, 1007, 1022, 1023]
    ref = attention.prefill_chunk(op, 0, widen(q32, "bf16"), table, ctx_before, scale, rows=rows)
    assert np.all(np.isfinite(out))
    err = max_abs_err(out, ref, rows)
    say("  max abs err", err)
    assert err <= TOL["bf16"]


def tile_rows(T, G):
    """The first and last position of every 256-row position tile of a chunk
    (256 / G positions per tile)."""
    tp = 256 // G
    return sorted({r for t0 in range(0, T, tp) for r in (t0, min(t0 + tp, T) - 1)})


@pytest.mark.parametrize("ctx_before,seed,signal", [(3500, 0, False), (3500, 0, True), (2476, 0, True),
                                                    (3500, 1, True), (3500, 2, True)])
def test_prefill_chunk_of_the_mixed_workload(ctx_before, seed, signal):
    """Config 5's own chunk -- 1,024 rows, 64 query / 8 KV heads, after 3,500
    cached tokens, and the reading where it is the last 1,024 of 3,500 --
    through the step runner (the chunk's rows appended with the decode
    tokens, then decode and prefill), with a shorter decode batch.  The
    first and last position of each of its 32 position tiles against the
    oracle on contiguous K/V."""
    from paged_kv_cache_140_amd.runner import DeviceRun

    scn = build_scenario(5, seed, B=4, ctx=("uniform", 1024, 4096), num_blocks=2048, ctx_before=ctx_before,
                         signal=signal)
    st = scn.steps[0]
    say("prefill workload 5 (4 decode sequences)", ctx_before, seed, "signal" if signal else "")
    gpu = DeviceRun(scn)
    gpu.run_setup()
    si = gpu.run_step(st)
    torch.cuda.synchronize()
    pf = st.prefill
    got = f64(si.prefill[3])
    assert np.all(np.isfinite(got))
    k, v = scn.history(pf.seq, pf.ctx_before)
    kc = np.concatenate([widen(k, "bf16"), widen(st.k_new[-pf.T:], "bf16")]).transpose(1, 0, 2)
    vc = np.concatenate([widen(v, "bf16"), widen(st.v_new[-pf.T:], "bf16")]).transpose(1, 0, 2)
    rows = tile_rows(pf.T, scn.cfg["G"])
    assert len(rows) == 64
    ref = attention.causal_rows(widen(pf.q, "bf16"), kc, vc, pf.ctx_before, scn.cfg["scale"], rows)
    err = max_abs_err(got, ref, rows)
    say("  max abs err", err)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("H_q,T,ctx_before", [(32, 40, 2992), (64, 1, 4000), (8, 200, 6000), (16, 129, 1000)])
def test_prefill_short_chunk_after_long_context_split(H_q, T, ctx_before):
    """The rest of a prompt after a prefix-cache hit (40 rows after 2,992
    cached tokens) and other short chunks over long contexts: run split over
    the keys, every row against the oracle."""
    from paged_kv_cache_140_amd import pa_prefill_workspace_size

    rng = np.random.default_rng(T + ctx_before)
    H_kv, d, bs = 8, 128, 16
    say("prefill split", H_q, T, ctx_before)
    op, gp, table = _chunk_world(rng, ctx_before + T, H_kv, d, bs, "bf16")
    assert pa_prefill_workspace_size(gp, T, H_q, ctx_before) > 0
    q32 = rng.standard_normal((T, H_q, d)).astype(np.float32)
    scale = float(np.float32(1 / np.sqrt(d)))
    out = f64(_run(gp, q32, table, ctx_before, scale, "bf16", split=True))
    ref = attention.prefill_chunk(op, 0, widen(q32, "bf16"), table, ctx_before, scale)
    err = max_abs_err(out, ref)
    say("  max abs err", err)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("H_q,H_kv,T", [(32, 8, 8192), (8, 8, 4096)])
def test_prefill_long_prompt_more_tiles_than_cus(H_q, H_kv, T):
    """A whole long prompt in one chunk (no cached context): 1,024 and 128
    workgroup tiles of 256 rows, several rounds over the 256 CUs.  Sampled
    rows, including the first and last of tiles and of the chunk."""
    rng = np.random.default_rng(T + H_q)
    d, bs = 128, 16
    say("prefill long prompt", H_q, H_kv, T)
    op, gp, table = _chunk_world(rng, T, H_kv, d, bs, "bf16")
    q32 = rng.standard_normal((T, H_q, d)).astype(np.float32)
    scale = float(np.float32(1 / np.sqrt(d)))
    out = f64(_run(gp, q32, table, 0, scale, "bf16"))
    tp = 256 // (H_q // H_kv)  # positions per workgroup tile
    rows = sorted({0, 1, tp - 1, tp, 2 * tp + 5, T // 2, T - tp - 1, T - tp, T - 2, T - 1})
    ref = attention.prefill_chunk(op, 0, widen(q32, "bf16"), table, 0, scale, rows=rows)
    assert np.all(np.isfinite(out))
    err = max_abs_err(out, ref, rows)
    say("  max abs err", err)
    assert err <= TOL["bf16"]


def test_prefill_merge_of_more_than_128_splits(tune):
    """A short chunk after 9,600 cached tokens cut into one split per 64-key
    step: 151 splits, so the merge's wave 0 walks its (m, l) pairs past the
    first 128 splits and every thread sums past its first 16 preloaded ones.
    Every row against the oracle."""
    from paged_kv_cache_140_amd import pa_prefill_workspace_size

    tune(prefill_splits=200)  # n > 1 asks for min(n, 64-key steps) splits
    H_q, H_kv, d, bs, T, ctx_before = 8, 8, 128, 16, 20, 9600
    rng = np.random.default_rng(151)
    say("prefill merge of 151 splits")
    op, gp, table = _chunk_world(rng, ctx_before + T, H_kv, d, bs, "bf16")
    steps = -(-(ctx_before + T) // 64)
    assert steps == 151
    assert pa_prefill_workspace_size(gp, T, H_q, ctx_before) == steps * T * H_q * (d + 2) * 4
    q32 = rng.standard_normal((T, H_q, d)).astype(np.float32)
    scale = float(np.float32(1 / np.sqrt(d)))
    out = f64(_run(gp, q32, table, ctx_before, scale, "bf16", split=True))
    ref = attention.prefill_chunk(op, 0, widen(q32, "bf16"), table, ctx_before, scale)
    err = max_abs_err(out, ref)
    say("  max abs err", err)
    assert err <= TOL["bf16"]
