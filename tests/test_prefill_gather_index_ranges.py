"""Index ranges of the prefill chunk's K/V gathers, simulated on the CPU.

The prefill tile (``prefill_tile`` in csrc/pa_prefill_dev.h, run by
pa_prefill_chunk and by pa_mixed_batch's persistent prefill workgroups)
reads block ids from the sequence's table with scalar loads and gathers 64
keys per step into LDS.  An earlier draft staged the table in LDS for the
keys its rows can see and gathered keys past them: other workgroups then
used uninitialised LDS entries as block ids and loaded far out of range (a
GPU memory fault).  This test restates the tile's index arithmetic -- the
work item of a workgroup, the item's last visible key ``kmax``, the split's
step range, the row each lane loads, the clamp to ``kmax - 1``, the table
reads of ``fetch`` (two per row group at block size 8), and the order of the
load rounds -- and checks, for the shapes the library runs:

  * every table entry read lies in [0, ceil(kmax / block_size)), inside the
    table the caller must pass (ceil((ctx_before + T) / block_size));
  * every gathered row uses the block id of its own key (the table entry of
    key // block_size), so no load ever takes another key's block;
  * the K and V gathers of an item cover each of its keys [0, kmax) in
    exactly one step of exactly one split, and touch no key >= kmax;
  * the launch's workgroups (XCD-contiguous order, or the mixed kernel's
    snake over persistent workgroups) take every (item, split) exactly once.

If the kernel's indexing changes, this model has to change with it.
"""

import math

import numpy as np
import pytest

KT = 64  # keys per step
ROWS_PER_WG = 256  # 8 waves x 32 query rows


def xcd_contiguous(L, total, xcds=8):
    per = (total + xcds - 1) // xcds
    full = total - (per - 1) * xcds
    xcd, local = L % xcds, L // xcds
    return xcd * per + local if xcd < full else full * per + (xcd - full) * (per - 1) + local


def plan_prefill(T, G, H_kv, ctx_before, cus=256, env_n=0):
    """The split plan of pa_prefill_chunk given a workspace (see plan_prefill
    in csrc/pa_prefill.hip): (num_splits, steps_per_split)."""
    TP = ROWS_PER_WG // G
    items = math.ceil(T / TP) * H_kv
    steps = math.ceil((ctx_before + T) / KT)
    if env_n == 1 or steps < 4 or (env_n == 0 and items * 2 > cus):
        return 1, 1 << 30
    n = min(env_n, steps) if env_n > 1 else min(math.ceil(cus / items), steps // 4)
    sps = math.ceil(steps / n)
    return math.ceil(steps / sps), sps


def item_gathers(T, ctx_before, G, BS, w, step_lo, step_hi):
    """Table indices read and, for every K and V row gathered by work item w
    over steps [step_lo, step_hi): whether the row is a key of its step (not
    clamped), the key gathered, and the table index of the block id used."""
    TP = ROWS_PER_WG // G
    ntiles = math.ceil(T / TP)
    t0 = (ntiles - 1 - w % ntiles) * TP
    t_last = min(t0 + TP, T) - 1
    kmax = ctx_before + t_last + 1
    s0 = step_lo
    nsteps = min(math.ceil(kmax / KT), step_hi) - s0
    if nsteps <= 0:
        return kmax, None
    rg = np.arange(KT // 16)                       # row groups of 16 rows (one per wave % 4)
    r = np.arange(16)
    reads = []

    def fetch(step):
        lo = np.minimum((s0 + step) * KT + rg * 16, kmax - 1) // BS
        hi = np.minimum((s0 + step) * KT + rg * 16 + 8, kmax - 1) // BS if BS < 16 else lo
        reads.append(lo)
        if BS < 16:
            reads.append(hi)
        return lo, hi

    gathers = {"K": [], "V": []}

    def issue(which, step, blocks):
        lo, hi = blocks
        raw = (s0 + step) * KT + rg[:, None] * 16 + r[None, :]
        key = np.minimum(raw, kmax - 1)
        idx = np.where((BS >= 16) | (r[None, :] < 8), lo[:, None], hi[:, None])
        gathers[which].append((raw < kmax, key, idx))  # unclamped rows, gathered key, its block's table index

    blk_v, blk_k = fetch(0), fetch(1)
    issue("K", 0, blk_v)
    for mr in range(nsteps + 1):
        if mr + 1 < nsteps:
            issue("K", mr + 1, blk_k)
        if mr < nsteps:
            issue("V", mr, blk_v)
        blk_v, blk_k = blk_k, fetch(mr + 2)
    out = {k: tuple(np.concatenate([g[i].ravel() for g in v]) for i in range(3)) for k, v in gathers.items()}
    return kmax, (np.concatenate(reads), out)


def check_chunk(T, ctx_before, G, H_kv, BS, splits, sps):
    """All (item, split) of one chunk: the four properties above."""
    TP = ROWS_PER_WG // G
    ntiles = math.ceil(T / TP)
    table_len = math.ceil((ctx_before + T) / BS)
    for w in range(ntiles):  # the KV head does not enter the index arithmetic
        covered = {"K": [], "V": []}
        kmax = None
        for sp in range(splits):
            kmax, res = item_gathers(T, ctx_before, G, BS, w, sp * sps, (sp + 1) * sps)
            if res is None:
                continue
            reads, gathers = res
            assert reads.min() >= 0 and reads.max() < math.ceil(kmax / BS) <= table_len
            for which, (live, key, idx) in gathers.items():
                assert key.min() >= 0 and key.max() < kmax
                assert np.array_equal(idx, key // BS), "a row gathered with another key's block id"
                covered[which].append(key[live])
        for which in ("K", "V"):
            keys = np.sort(np.concatenate(covered[which]))
            assert np.array_equal(keys, np.arange(kmax)), f"{which} keys of item {w} not covered exactly once"


CHUNKS = [
    # T, ctx_before, G, H_kv, BS
    (1024, 3500, 8, 8, 16),   # the mixed workload's chunk
    (1024, 2476, 8, 8, 16),   # the reading where it is the last 1,024 of 3,500
    (40, 2992, 4, 8, 16),     # the rest of a prompt after a prefix-cache hit (split)
    (20, 9600, 1, 8, 16),     # 151 splits of one step each (with the split override)
    (130, 513, 2, 8, 16),
    (129, 37, 1, 8, 8),
    (64, 64, 4, 8, 32),
    (77, 250, 4, 4, 16),
    (8192, 0, 4, 8, 16),      # a whole prompt, more tiles than CUs
    (1, 4000, 8, 8, 16),
]


@pytest.mark.parametrize("T,ctx_before,G,H_kv,BS", CHUNKS, ids=[f"T{c[0]}-ctx{c[1]}-G{c[2]}-bs{c[4]}" for c in CHUNKS])
def test_prefill_chunk_gathers_stay_in_range(T, ctx_before, G, H_kv, BS):
    for env_n in (1, 0, 200):
        splits, sps = plan_prefill(T, G, H_kv, ctx_before, env_n=env_n)
        check_chunk(T, ctx_before, G, H_kv, BS, splits, sps)
    TP = ROWS_PER_WG // G
    items = math.ceil(T / TP) * H_kv
    splits, _ = plan_prefill(T, G, H_kv, ctx_before)
    grid = items * splits
    taken = sorted(xcd_contiguous(L, grid) for L in range(grid))
    assert taken == list(range(grid)), "workgroups must take every (item, split) once"


@pytest.mark.parametrize("chunks,G,H_kv,n_pre", [
    ([(1024, 3500)], 8, 8, 64),
    ([(256, 200), (256, 1000), (256, 3500), (256, 8000)], 8, 8, 64),
    ([(400, 100), (0, 7), (33, 0), (5, 2000)], 2, 8, 24),
])
def test_mixed_batch_prefill_items_stay_in_range(chunks, G, H_kv, n_pre):
    """pa_mixed_batch: the persistent prefill workgroups walk the chunks'
    items in snake order (workgroup p takes items p, 2n-1-p, 2n+p, ...);
    every item is taken exactly once, by one workgroup, and each item's
    gathers satisfy the same range properties as a standalone chunk's."""
    TP = ROWS_PER_WG // G
    live = [c for c in chunks if c[0] > 0]
    order = sorted(live, key=lambda c: -(c[1] + c[0]))  # longest chunk first (stable)
    items_before = np.cumsum([0] + [math.ceil(T / TP) * H_kv for T, _ in order])
    n_items = int(items_before[-1])
    n = min(n_pre, n_items)
    taken = []
    for p in range(n):
        r = 0
        while True:
            k = r * n + (n - 1 - p if r & 1 else p)
            if k >= n_items:
                break
            taken.append(k)
            r += 1
    assert sorted(taken) == list(range(n_items))
    for k in range(n_items):
        c = int(np.searchsorted(items_before, k, side="right") - 1)
        T, cb = order[c]
        kl = k - int(items_before[c])
        ntiles = math.ceil(T / TP)
        w = (kl % H_kv) * ntiles + kl // H_kv
        assert 0 <= w < ntiles * H_kv
    for T, cb in live:
        check_chunk(T, cb, G, H_kv, 16, 1, 1 << 30)


def test_the_draft_that_faulted_would_fail_here():
    """The fault's cause, restated: a draft gathered keys up to the chunk's
    end while only the keys below its own kmax had table entries staged.
    Modelled here as gathers clamped to the chunk's last key instead of the
    item's kmax: at the mixed workload's shape, workgroups other than the
    last tile's read keys (and so table entries) past their kmax."""
    T, ctx_before, G, BS = 1024, 3500, 8, 16
    TP = ROWS_PER_WG // G
    ntiles = math.ceil(T / TP)
    bad = 0
    for w in range(ntiles):
        t0 = (ntiles - 1 - w % ntiles) * TP
        kmax = ctx_before + min(t0 + TP, T)
        steps = math.ceil((ctx_before + T) / KT)  # the draft's step count: the chunk's, not the item's
        keys = np.arange(steps * KT)
        bad += int(np.sum(keys >= kmax))
    assert bad > 0
