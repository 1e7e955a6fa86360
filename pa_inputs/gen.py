"""Random draws.  One independent PCG64 stream per (seed, config, purpose, index).

Streams are keyed by tuples so that any one sequence's K/V history can be
regenerated alone (the full-size parity tests sample a few sequences).

Purpose ids:
  0 lengths   1 free-block order   2 churn   3 history K/V (per sequence)
  4 new-token K/V (per step)   5 queries (per step)   6 prefill-chunk K/V
  7 prefill-chunk queries   8 beam survivors (per step and prompt)
"""

import numpy as np

LENGTHS, FREE_ORDER, CHURN, HISTORY, NEW_KV, QUERY, CHUNK_KV, CHUNK_Q, BEAM = range(9)


def rng(seed, cid, purpose, *index):
    return np.random.default_rng([int(seed), int(cid), int(purpose), *map(int, index)])


def lengths(cfg, seed, n=None):
    """Context lengths before the step's append, int64 [n]."""
    spec = cfg["ctx"]
    n = cfg["B"] if n is None else n
    if spec[0] == "fixed":
        return np.asarray(spec[1], dtype=np.int64)
    r = rng(seed, cfg["id"], LENGTHS)
    if spec[0] == "uniform":
        lo, hi = spec[1], spec[2]
        return r.integers(lo, hi, size=n, endpoint=True).astype(np.int64)
    if spec[0] == "lognormal":
        median, sigma, lo, hi = spec[1:]
        x = r.lognormal(np.log(median), sigma, size=n)
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    raise ValueError(spec)


def lognormal_lengths(r, n, median=400.0, sigma=0.8, lo=16, hi=2048):
    x = r.lognormal(np.log(median), sigma, size=n)
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def free_order(cfg, seed):
    """A seeded permutation of the physical block ids: the initial free list."""
    return rng(seed, cfg["id"], FREE_ORDER).permutation(cfg["num_blocks"]).astype(np.int32)


def normal(r, shape):
    """N(0,1) drawn directly in float32 (NumPy's float32 ziggurat)."""
    return r.standard_normal(size=shape, dtype=np.float32)


def history_kv(cfg, seed, seq, length):
    """K and V of a sequence's first ``length`` tokens, float32 [length][H_kv][d]."""
    r = rng(seed, cfg["id"], HISTORY, seq)
    shape = (int(length), cfg["H_kv"], cfg["d"])
    return normal(r, shape), normal(r, shape)


def new_kv(cfg, seed, step, T):
    r = rng(seed, cfg["id"], NEW_KV, step)
    shape = (int(T), cfg["H_kv"], cfg["d"])
    return normal(r, shape), normal(r, shape)


def queries(cfg, seed, step, n):
    return normal(rng(seed, cfg["id"], QUERY, step), (int(n), cfg["H_q"], cfg["d"]))


def chunk_kv(cfg, seed, T):
    r = rng(seed, cfg["id"], CHUNK_KV)
    shape = (int(T), cfg["H_kv"], cfg["d"])
    return normal(r, shape), normal(r, shape)


def chunk_queries(cfg, seed, T):
    return normal(rng(seed, cfg["id"], CHUNK_Q), (int(T), cfg["H_q"], cfg["d"]))


def beam_parents(cfg, seed, step, group):
    """Which current beam each of the next step's beams continues: ``beam``
    indices drawn with replacement (a beam drawn twice forks, one not drawn
    ends)."""
    k = cfg["beam"]
    return rng(seed, cfg["id"], BEAM, step, group).integers(0, k, size=k)


def churn(cfg, seed, add, try_append, free):
    """Fragment a pool by alloc/free churn before the real sequences arrive.

    ``add(seq)``, ``try_append(seq, n) -> bool`` and ``free(seq)`` act on
    whichever allocator the caller passes (the oracle's or the library's); an
    append that does not fit must leave the allocator unchanged and return
    False.  Ghost sequences use ids from 1_000_000 up so that they never clash
    with real ones.  Each round: open a ghost of lognormal length, or if it
    does not fit free a random live ghost instead; then with probability 1/2
    free another random live ghost.  Afterwards every ghost is freed in random
    order.  Returns the number of ghost sequences opened.
    """
    r = rng(seed, cfg["id"], CHURN)
    live = []
    next_id = 1_000_000
    for _ in range(cfg["churn_rounds"]):
        n = int(lognormal_lengths(r, 1)[0])
        sid = next_id
        next_id += 1
        add(sid)
        if try_append(sid, n):
            live.append(sid)
        else:
            free(sid)
            if live:
                free(live.pop(int(r.integers(len(live)))))
        if live and r.random() < 0.5:
            free(live.pop(int(r.integers(len(live)))))
    for i in r.permutation(len(live)):
        free(live[int(i)])
    return next_id - 1_000_000


# ---------------------------------------------------------------- signal inputs
# N(0,1) queries and keys at scale 1/sqrt(d) spread a long context's softmax
# almost evenly, so one 16-token group of 16k keys weighs ~1/1000 and moves
# the output by ~1e-3: far below a bf16 tolerance of 2e-2.  In signal mode
# every V row also carries a marker of its 16-token group: +-c at dim
# (t // 16 + 37 g) mod d for KV head g, the sign flipping each time the
# groups wrap round the d dims (so that a dim's markers cancel instead of
# piling up over a long context), with c proportional to the sequence's
# length.  Every group then moves one output dim by ~16 c / n =
# 16 / SIGNAL_TOKENS_PER_UNIT: leaving a group out, counting it twice or
# taking another head's rows shows as a change of several times the
# tolerance at any context length.  A new token (a decode step's own row, or
# a prefill chunk's row, which its row sees last) carries a second marker
# weighing a whole group (16 c), so losing it, or a causal mask one key off,
# shows too.  Queries are scaled by
# SIGNAL_Q_SCALE, which keeps the weight of the lightest group within a
# small factor of the mean.  The values stay N(0,1) plus the marker.
SIGNAL_Q_SCALE = 0.5
SIGNAL_TOKENS_PER_UNIT = 50.0
SIGNAL_GROUP = 16


def signal_c(final_len):
    """Marker size of a sequence that reaches ``final_len`` visible tokens."""
    return max(1.0, float(final_len) / SIGNAL_TOKENS_PER_UNIT)


def position_signal(cfg, positions, c, new_token=False):
    """Markers of V rows at ``positions`` (float32 [n][H_kv][d]): +-c at dim
    (t // 16 + 37 g) mod d of head g, sign (-1)^((t // 16) // d).  A new
    token (a decode step's appended row, or a prefill chunk's own row, the
    last key its row sees) also carries a marker of a whole group's weight,
    +-16 c at dim (t + 53 g) mod d, sign (-1)^(t // d)."""
    pos = np.asarray(positions, dtype=np.int64).reshape(-1)
    H, d = cfg["H_kv"], cfg["d"]
    out = np.zeros((pos.size, H, d), dtype=np.float32)
    grp = pos // SIGNAL_GROUP
    gval = (np.float32(c) * np.where((grp // d) % 2 == 0, 1, -1)).astype(np.float32)
    tval = (np.float32(c * SIGNAL_GROUP) * np.where((pos // d) % 2 == 0, 1, -1)).astype(np.float32)
    rows = np.arange(pos.size)
    for g in range(H):
        out[rows, g, (grp + 37 * g) % d] += gval
        if new_token:
            out[rows, g, (pos + 53 * g) % d] += tval
    return out
