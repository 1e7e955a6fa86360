"""Drive a ``pa_inputs`` scenario through the oracle.

Two views of the same K/V are kept:
  * the paged view: the oracle allocator hands out slots and copy-on-write
    pairs, the oracle pool receives the writes, attention gathers through the
    block tables;
  * the logical view: each sequence's K/V as the plain list of rows it was
    given (a fork starts from a copy of its parent's list).
The paged view is what the library is compared with.  The logical view needs
no pool, so it serves workloads whose pool is too large for a CPU copy, and
paged == logical is itself one of the oracle's pins (paging changes no result:
[icarus] "不改变模型精度"; [ttlab] "블록과 블록 표").
"""

from dataclasses import dataclass, field

import numpy as np

from . import attention, encoding
from .block_manager import BlockManager, OutOfBlocks
from .pool import Pool


def widen(x, dtype):
    """float32 input -> the exact value the pool / query holds, as float64."""
    return encoding.decode(encoding.encode(x, dtype), dtype)


@dataclass
class StepResult:
    slots: list
    pairs: list
    decode_lengths: list = field(default_factory=list)
    decode_out: np.ndarray = None  # float64 [n][H_q][d] (rows not computed are NaN)
    prefill_out: np.ndarray = None  # float64 [T][H_q][d] (rows not computed are NaN)


class OracleRun:
    def __init__(self, scn, with_pool=True, num_layers=1, layer=0, fill_bits=None, with_data=True):
        """``with_data=False`` runs the allocator alone (no pool, no K/V values)."""
        self.scn = scn
        self.with_data = with_data
        with_pool = with_pool and with_data
        cfg = self.cfg = scn.cfg
        from pa_inputs import gen

        self.free_order = gen.free_order(cfg, scn.seed)
        self.bm = BlockManager(cfg["num_blocks"], cfg["bs"], self.free_order)
        self.layer = layer
        self.pool = (Pool(num_layers, cfg["H_kv"], cfg["num_blocks"], cfg["bs"], cfg["d"], cfg["dtype"], fill_bits)
                     if with_pool else None)
        self.logical = {}  # seq -> list of (k rows, v rows) float64 chunks
        self.results = []

    # -- allocator callbacks used by the churn driver --------------------------
    def _add(self, seq):
        self.bm.add_seq(seq)

    def _try_append(self, seq, n):
        try:
            self.bm.append_slots(seq, n)
        except OutOfBlocks:
            return False
        return True

    def _free(self, seq):
        self.bm.free_seq(seq)

    # -- writes ------------------------------------------------------------------
    def _write(self, seqs_rows, slots, k32, v32):
        if not self.with_data:
            return
        dt = self.cfg["dtype"]
        if self.pool is not None:
            self.pool.append(self.layer, encoding.encode(k32, dt), encoding.encode(v32, dt), slots)
        row = 0
        for seq, n in seqs_rows:
            self.logical[seq].append((widen(k32[row:row + n], dt), widen(v32[row:row + n], dt)))
            row += n

    def logical_kv(self, seq):
        chunks = self.logical[seq]
        d, H = self.cfg["d"], self.cfg["H_kv"]
        if not chunks:
            return np.zeros((H, 0, d)), np.zeros((H, 0, d))
        k = np.concatenate([c[0] for c in chunks]).transpose(1, 0, 2)
        v = np.concatenate([c[1] for c in chunks]).transpose(1, 0, 2)
        return k, v

    def run_setup(self):
        from pa_inputs import gen

        for op in self.scn.setup:
            if op[0] == "add":
                self.bm.add_seq(op[1])
                self.logical[op[1]] = []
            elif op[0] == "append":
                seq, n = op[1], op[2]
                if self.bm.seq_len(seq) != 0:
                    raise ValueError("setup appends start from an empty sequence")
                slots, pairs = self.bm.append_slots(seq, n)
                assert not pairs
                if self.with_data:
                    k, v = self.scn.history(seq, n)
                    self._write([(seq, n)], slots, k, v)
            elif op[0] == "fork":
                self.bm.fork(op[1], op[2])
                self.logical[op[2]] = list(self.logical[op[1]])
            elif op[0] == "churn":
                gen.churn(self.cfg, self.scn.seed, self._add, self._try_append, self._free)
            else:
                raise ValueError(op)

    def run_ops(self, step):
        """The step's forks and frees, before its appends."""
        for op in step.ops:
            if op[0] == "fork":
                self.bm.fork(op[1], op[2])
                self.logical[op[2]] = list(self.logical[op[1]])
            elif op[0] == "free":
                self.bm.free_seq(op[1])
                del self.logical[op[1]]
            else:
                raise ValueError(op)

    def bookkeeping(self, step):
        """Slots and copy-on-write pairs of a step's appends, in append order
        (after the step's forks and frees)."""
        self.run_ops(step)
        slots, pairs = [], []
        for seq, n in step.appends:
            s, p = self.bm.append_slots(seq, n)
            slots += s
            pairs += p
        return slots, pairs

    def run_step(self, step, paged=True, decode_rows=None, prefill_rows=None):
        """Apply one step.  ``decode_rows`` / ``prefill_rows`` limit which output
        rows are computed (None = all); the rest stay NaN."""
        cfg = self.cfg
        dt = cfg["dtype"]
        slots, pairs = self.bookkeeping(step)
        if self.pool is not None:
            self.pool.copy_blocks(pairs)
        self._write(step.appends, slots, step.k_new, step.v_new)
        res = StepResult(slots=slots, pairs=pairs)
        n = len(step.decode_seqs)
        res.decode_lengths = [self.bm.seq_len(s) for s in step.decode_seqs]
        if not self.with_data:
            self.results.append(res)
            return res
        if n:
            q = widen(step.q, dt)
            out = np.full(q.shape, np.nan)
            rows = range(n) if decode_rows is None else decode_rows
            for i in rows:
                seq = step.decode_seqs[i]
                if paged:
                    k, v = attention.gather(self.pool, self.layer, self.bm.block_table(seq), self.bm.seq_len(seq))
                else:
                    k, v = self.logical_kv(seq)
                out[i] = attention.attend(q[i], k, v, cfg["scale"])
            res.decode_out = out
        if step.prefill is not None:
            pf = step.prefill
            q = widen(pf.q, dt)
            if paged:
                out = attention.prefill_chunk(self.pool, self.layer, q, self.bm.block_table(pf.seq),
                                              pf.ctx_before, cfg["scale"], prefill_rows)
            else:
                k, v = self.logical_kv(pf.seq)
                out = attention.causal_rows(q, k, v, pf.ctx_before, cfg["scale"], prefill_rows)
            res.prefill_out = out
        self.results.append(res)
        return res
