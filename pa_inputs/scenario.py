"""Each workload as an op list: the allocator and pool calls to make, in order.

An op list is data.  Each side (the oracle's tests, the library's callers)
runs it with its own allocator, its own pool writes and its own attention, so
the two share the sequence of requests and the random values but no code that
computes anything.

Ops in ``setup``:
  ("add", seq)                        open an empty sequence
  ("append", seq, n)                  reserve n slots for seq and write the
                                      sequence's history K/V (``history``)
  ("fork", parent, child)             child shares all of parent's blocks
  ("churn",)                          run ``gen.churn`` against the allocator

Each ``Step`` then: its ``ops`` (("fork", parent, child) and ("free", seq),
in order), one batched append (``appends`` in order, K/V rows
``k_new``/``v_new`` in the same order, copy-on-write pairs first), then decode
attention for ``decode_seqs`` with queries ``q`` and, when present, one causal
prefill chunk.
"""

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

from . import gen
from .configs import config as make_config


@dataclass
class Prefill:
    seq: int
    ctx_before: int
    T: int
    q: np.ndarray  # float32 [T][H_q][d]


@dataclass
class Step:
    appends: List[Tuple[int, int]]
    k_new: np.ndarray  # float32 [T][H_kv][d]
    v_new: np.ndarray
    decode_seqs: List[int]
    q: np.ndarray  # float32 [len(decode_seqs)][H_q][d]
    prefill: Optional[Prefill] = None
    ops: list = field(default_factory=list)  # forks and frees before the appends


@dataclass
class Scenario:
    cfg: dict
    seed: int
    setup: list = field(default_factory=list)
    steps: List[Step] = field(default_factory=list)
    ctx: Optional[np.ndarray] = None  # per decode sequence, before the first step
    # signal mode: marker size per sequence whose history is drawn
    signal_c: dict = field(default_factory=dict)

    def history(self, seq, n):
        """History K/V of ``seq``'s first n tokens (float32 [n][H_kv][d] each)."""
        k, v = gen.history_kv(self.cfg, self.seed, seq, n)
        if self.cfg.get("signal"):
            v += gen.position_signal(self.cfg, np.arange(int(n)), self.signal_c[seq])
        return k, v


def _signal_new_rows(cfg, v, positions, cs, new_token):
    """Signal mode: add the markers of appended rows (positions and marker
    sizes per row) to their V."""
    if cfg.get("signal"):
        for i, (p, c) in enumerate(zip(positions, cs)):
            v[i:i + 1] += gen.position_signal(cfg, [p], c, new_token=new_token)


def _queries(cfg, seed, step_index, n):
    q = gen.queries(cfg, seed, step_index, n)
    if cfg.get("signal"):
        q *= np.float32(gen.SIGNAL_Q_SCALE)
    return q


def _decode_batch(cfg, seed, seqs, step_index, positions=None, cs=None):
    """One new token per sequence at ``positions`` (its length before the
    append), then decode; ``cs``: signal-mode marker sizes."""
    T = len(seqs)
    k, v = gen.new_kv(cfg, seed, step_index, T)
    if cfg.get("signal"):
        _signal_new_rows(cfg, v, positions, cs, new_token=True)
    q = _queries(cfg, seed, step_index, T)
    return Step(appends=[(s, 1) for s in seqs], k_new=k, v_new=v, decode_seqs=list(seqs), q=q)


def build_scenario(cid, seed=0, **overrides):
    cfg = make_config(cid, **overrides)
    scn = Scenario(cfg=cfg, seed=seed)
    kind = cfg["kind"]
    if kind == "decode":
        ctx = gen.lengths(cfg, seed)
        scn.ctx = ctx
        cs = [gen.signal_c(int(n) + 1) for n in ctx]
        if cfg.get("churn_rounds"):
            scn.setup.append(("churn",))
        for s, n in enumerate(ctx):
            scn.setup.append(("add", s))
            scn.setup.append(("append", s, int(n)))
            scn.signal_c[s] = cs[s]
        scn.steps.append(_decode_batch(cfg, seed, list(range(cfg["B"])), 0, [int(n) for n in ctx], cs))
    elif kind == "fork":
        P, S = cfg["prompts"], cfg["samples"]
        c = gen.signal_c(cfg["prefix"] + cfg["tail"] + cfg["steps"])
        for p in range(P):
            root = p * S
            scn.setup.append(("add", root))
            scn.setup.append(("append", root, cfg["prefix"]))
            scn.signal_c[root] = c
            for s in range(1, S):
                scn.setup.append(("fork", root, root + s))
        seqs = list(range(P * S))
        scn.ctx = np.full(P * S, cfg["prefix"], dtype=np.int64)
        # tail: every sample writes its own 32 tokens after the shared prefix
        T = len(seqs) * cfg["tail"]
        k, v = gen.new_kv(cfg, seed, 0, T)
        tail_pos = [cfg["prefix"] + j for _ in seqs for j in range(cfg["tail"])]
        _signal_new_rows(cfg, v, tail_pos, [c] * T, new_token=False)
        scn.steps.append(Step(appends=[(s, cfg["tail"]) for s in seqs], k_new=k, v_new=v,
                              decode_seqs=[], q=np.zeros((0, cfg["H_q"], cfg["d"]), np.float32)))
        for i in range(cfg["steps"]):
            pos = [cfg["prefix"] + cfg["tail"] + i] * len(seqs)
            scn.steps.append(_decode_batch(cfg, seed, seqs, 1 + i, pos, [c] * len(seqs)))
    elif kind == "mixed":
        ctx = gen.lengths(cfg, seed)
        scn.ctx = ctx
        B = cfg["B"]
        cs = [gen.signal_c(int(n) + 1) for n in ctx]
        for s, n in enumerate(ctx):
            scn.setup.append(("add", s))
            scn.setup.append(("append", s, int(n)))
            scn.signal_c[s] = cs[s]
        pseq = B
        c_chunk = gen.signal_c(cfg["ctx_before"] + cfg["chunk"])
        scn.setup.append(("add", pseq))
        scn.setup.append(("append", pseq, cfg["ctx_before"]))
        scn.signal_c[pseq] = c_chunk
        st = _decode_batch(cfg, seed, list(range(B)), 0, [int(n) for n in ctx], cs)
        kc, vc = gen.chunk_kv(cfg, seed, cfg["chunk"])
        _signal_new_rows(cfg, vc, [cfg["ctx_before"] + t for t in range(cfg["chunk"])], [c_chunk] * cfg["chunk"],
                         new_token=True)
        st.appends.append((pseq, cfg["chunk"]))
        st.k_new = np.concatenate([st.k_new, kc])
        st.v_new = np.concatenate([st.v_new, vc])
        qc = gen.chunk_queries(cfg, seed, cfg["chunk"])
        if cfg.get("signal"):
            qc *= np.float32(gen.SIGNAL_Q_SCALE)
        st.prefill = Prefill(seq=pseq, ctx_before=cfg["ctx_before"], T=cfg["chunk"], q=qc)
        scn.steps.append(st)
    elif kind == "beam":
        # Every prompt starts ``beam`` beams sharing its blocks (its last one
        # partly filled).  Each step the next beams are drawn from the current
        # ones with replacement: a beam drawn first keeps its sequence, each
        # further draw forks it, and a beam not drawn is freed; then every
        # beam appends one token and is decoded.
        P, k = cfg["prompts"], cfg["beam"]
        beams, next_id = [], []
        c = gen.signal_c(cfg["prompt_len"] + cfg["steps"])
        for p in range(P):
            root = p * 1000
            scn.setup.append(("add", root))
            scn.setup.append(("append", root, cfg["prompt_len"]))
            scn.signal_c[root] = c
            for j in range(1, k):
                scn.setup.append(("fork", root, root + j))
            beams.append([root + j for j in range(k)])
            next_id.append(root + k)
        for t in range(cfg["steps"]):
            ops = []
            for p in range(P):
                kept, new = set(), []
                for i in gen.beam_parents(cfg, seed, t, p):
                    parent = beams[p][int(i)]
                    if parent not in kept:
                        kept.add(parent)
                        new.append(parent)
                    else:
                        ops.append(("fork", parent, next_id[p]))
                        new.append(next_id[p])
                        next_id[p] += 1
                ops += [("free", b) for b in beams[p] if b not in kept]
                beams[p] = sorted(new)
            seqs = sorted(b for bs_ in beams for b in bs_)
            st = _decode_batch(cfg, seed, seqs, t, [cfg["prompt_len"] + t] * len(seqs), [c] * len(seqs))
            st.ops = ops
            scn.steps.append(st)
        scn.ctx = np.full(P * k, cfg["prompt_len"], dtype=np.int64)
    else:
        raise ValueError(kind)
    return scn
