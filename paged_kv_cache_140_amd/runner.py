"""Runs a ``pa_inputs`` scenario through the library on one GPU.

Bookkeeping (slots, copy-on-write pairs, block tables) comes from the host
block manager ``pa_bm``; every pool write and every attention runs in the
HIP kernels.  torch supplies device memory, host<->device copies and the
stream.
"""

from dataclasses import dataclass

import numpy as np
import torch

from pa_inputs import gen

from .api import (BlockManager, KVPool, OutOfBlocks, TORCH_DTYPE, decode_shared_workspace, decode_workspace,
                  pa_cache_append, pa_copy_blocks, pa_decode, pa_decode_append, pa_decode_shared, pa_mixed_batch,
                  pa_prefill_chunk, pa_share_groups, prefill_workspace)


def to_device(x, dtype, device):
    """float32 NumPy -> device tensor of the pool dtype (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(TORCH_DTYPE[dtype]).to(device)


@dataclass
class StepInputs:
    """Everything one step needs, resident on the device."""
    slots: torch.Tensor
    pairs: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    q: torch.Tensor
    tables: torch.Tensor
    lens: torch.Tensor
    max_ctx: int
    out: torch.Tensor
    workspace: object
    prefill: object = None  # (q, table, ctx_before, out, workspace)
    n_pairs: int = 0
    # True when the step appends exactly one token to each decoded sequence,
    # in decode order: then append + decode can run as one pa_decode_append.
    fusable: bool = False
    # launch row i of the decode holds the step's decode row order[i]
    order: object = None
    # shared-prefix decode: groups of launch rows sharing leading blocks
    # (first_row, n_rows, shared_blocks) and their workspace
    groups: object = None
    shared_ws: object = None


class DeviceRun:
    """``fill``: "nan" poisons every pool slot before setup (parity runs),
    "randn" fills it with N(0,1) on the device and skips writing the history
    values (timing runs only need the bookkeeping), None leaves it as is."""

    def __init__(self, scn, device="cuda", num_layers=1, layer=0, fill="nan", seed_fill=0, pad_pool=False):
        """``pad_pool``: allocate the workload's ``alloc_bytes_per_head`` per
        KV head (if it names one) instead of exactly num_blocks blocks; the
        block manager hands out num_blocks either way."""
        self.scn, self.cfg = scn, scn.cfg
        cfg = self.cfg
        self.device = device
        self.layer = layer
        self.bm = BlockManager(cfg["num_blocks"], cfg["bs"], gen.free_order(cfg, scn.seed))
        n_alloc = cfg["num_blocks"]
        if pad_pool and cfg.get("alloc_bytes_per_head"):
            per_block = cfg["bs"] * cfg["d"] * TORCH_DTYPE[cfg["dtype"]].itemsize
            n_alloc = max(n_alloc, cfg["alloc_bytes_per_head"] // per_block)
        self.pool = KVPool(num_layers, cfg["H_kv"], n_alloc, cfg["bs"], cfg["d"], cfg["dtype"], device)
        self.write_history = fill != "randn"
        if fill == "nan":
            self.pool.k.fill_(float("nan"))
            self.pool.v.fill_(float("nan"))
        elif fill == "randn":
            g = torch.Generator(device=device)
            g.manual_seed(seed_fill)
            for t in (self.pool.k, self.pool.v):
                flat = t.view(-1)
                step = 1 << 28
                for i in range(0, flat.numel(), step):
                    flat[i:i + step].normal_(generator=g)

    # -- setup ---------------------------------------------------------------
    def _try_append(self, seq, n):
        try:
            self.bm.append_slots(seq, n)
        except OutOfBlocks:
            return False
        return True

    def run_setup(self, chunk_tokens=1 << 16):
        cfg = self.cfg
        for op in self.scn.setup:
            if op[0] == "add":
                self.bm.add_seq(op[1])
            elif op[0] == "append":
                seq, n = op[1], op[2]
                slots, pairs = self.bm.append_slots(seq, n)
                assert not pairs
                if self.write_history:
                    k, v = self.scn.history(seq, n)
                    for a in range(0, n, chunk_tokens):
                        b = min(n, a + chunk_tokens)
                        pa_cache_append(self.pool, self.layer, to_device(k[a:b], cfg["dtype"], self.device),
                                        to_device(v[a:b], cfg["dtype"], self.device),
                                        torch.from_numpy(slots[a:b]).to(self.device))
            elif op[0] == "fork":
                self.bm.fork(op[1], op[2])
            elif op[0] == "churn":
                gen.churn(cfg, self.scn.seed, self.bm.add_seq, self._try_append, self.bm.free_seq)
            else:
                raise ValueError(op)

    # -- one step ------------------------------------------------------------
    def prepare(self, step, longest_first=False, shared=False):
        """Host bookkeeping for ``step`` (its forks and frees, then its
        appends) and H2D staging of all its inputs.

        ``longest_first``: submit the decode batch longest context first, as
        a scheduler can (the decode starts its workgroups in batch order;
        when they outnumber the CUs, the long ones then do not trail).  The
        bookkeeping stays in the step's order; only the decode's launch rows
        (tables, lengths, queries and, for a fused step, the new tokens and
        their slots) are permuted, and ``si.order[i]`` is the step row that
        launch row i holds.

        ``shared``: also group the launch rows that share leading blocks
        (pa_share_groups on the host tables) for pa_decode_shared."""
        cfg, dev = self.cfg, self.device
        for op in step.ops:
            if op[0] == "fork":
                self.bm.fork(op[1], op[2])
            elif op[0] == "free":
                self.bm.free_seq(op[1])
            else:
                raise ValueError(op)
        seqs = [s for s, _ in step.appends]
        ns = [n for _, n in step.appends]
        slots, pairs = self.bm.append_slots_batch(seqs, ns)
        si = StepInputs(
            slots=torch.from_numpy(slots).to(dev),
            pairs=torch.from_numpy(np.ascontiguousarray(pairs.reshape(-1, 2))).to(dev),
            k_new=to_device(step.k_new, cfg["dtype"], dev),
            v_new=to_device(step.v_new, cfg["dtype"], dev),
            q=None, tables=None, lens=None, max_ctx=0, out=None, workspace=None, n_pairs=len(pairs))
        si.host_slots, si.host_pairs = slots, pairs
        if step.decode_seqs:
            lens = np.array([self.bm.seq_len(s) for s in step.decode_seqs], dtype=np.int32)
            max_ctx = int(lens.max())
            max_blocks = -(-max_ctx // cfg["bs"])
            tables = self.bm.block_tables(step.decode_seqs, max_blocks)
            si.q = to_device(step.q, cfg["dtype"], dev)
            si.tables = torch.from_numpy(tables).to(dev)
            si.lens = torch.from_numpy(lens).to(dev)
            si.max_ctx = max_ctx
            si.out = torch.empty_like(si.q)
            si.workspace = decode_workspace(self.pool, len(step.decode_seqs), cfg["H_q"], max_ctx, dev)
            si.fusable = list(step.appends) == [(s_, 1) for s_ in step.decode_seqs]
            si.order = np.arange(len(lens))
            if longest_first:
                perm = np.argsort(-lens, kind="stable")
                pt = torch.from_numpy(perm).to(dev)
                si.order = perm
                si.tables, si.lens, si.q = si.tables[pt].contiguous(), si.lens[pt].contiguous(), si.q[pt].contiguous()
                if si.fusable:
                    si.k_new, si.v_new = si.k_new[pt].contiguous(), si.v_new[pt].contiguous()
                    si.slots = si.slots[pt].contiguous()
                tables, lens = tables[perm], lens[perm]
            if shared:
                si.groups = pa_share_groups(tables, lens, cfg["bs"])
                si.shared_ws = decode_shared_workspace(self.pool, len(lens), cfg["H_q"], max_ctx, si.groups, dev)
        if step.prefill is not None:
            pf = step.prefill
            table = np.array(self.bm.block_table(pf.seq), dtype=np.int32)
            q = to_device(pf.q, cfg["dtype"], dev)
            ws = prefill_workspace(self.pool, pf.T, cfg["H_q"], pf.ctx_before, dev)
            si.prefill = (q, torch.from_numpy(table).to(dev), pf.ctx_before, torch.empty_like(q), ws)
        return si

    def launch(self, si, stream=None, do_copy=True, do_append=True, do_decode=True, do_prefill=True, fused=False,
               mixed=False, prefill_workgroups=0, shared=False):
        """Enqueue the step's kernels in the contract order: copies, appends,
        attention.  ``fused``: a step that appends one token per decoded
        sequence runs its append and decode as one pa_decode_append.
        ``mixed``: a step with both a decode batch and a prefill chunk runs
        the two attentions as one pa_mixed_batch.  ``shared``: the decode
        runs as pa_decode_shared over the groups ``prepare(shared=True)``
        found."""
        cfg = self.cfg
        if mixed and do_decode and do_prefill and si.q is not None and si.prefill is not None:
            if do_copy and si.n_pairs:
                pa_copy_blocks(self.pool, si.pairs, stream)
            if do_append and si.slots.numel():
                pa_cache_append(self.pool, self.layer, si.k_new, si.v_new, si.slots, stream)
            q, table, ctx_before, out, _ = si.prefill
            pa_mixed_batch(self.pool, self.layer, si.out, si.q, si.tables, si.lens, si.max_ctx, out, q,
                           [(q.shape[0], ctx_before)], table.view(1, -1), cfg["scale"], prefill_workgroups,
                           si.workspace, stream)
            return
        if do_copy and si.n_pairs:
            pa_copy_blocks(self.pool, si.pairs, stream)
        if fused and si.fusable and do_append and do_decode:
            pa_decode_append(self.pool, self.layer, si.out, si.q, si.k_new, si.v_new, si.slots, si.tables, si.lens,
                             si.max_ctx, cfg["scale"], si.workspace, stream)
            do_append = do_decode = False
        if do_append and si.slots.numel():
            pa_cache_append(self.pool, self.layer, si.k_new, si.v_new, si.slots, stream)
        if do_decode and si.q is not None and shared:
            pa_decode_shared(self.pool, self.layer, si.out, si.q, si.tables, si.lens, si.max_ctx, cfg["scale"],
                             si.groups, si.shared_ws, stream)
        elif do_decode and si.q is not None:
            pa_decode(self.pool, self.layer, si.out, si.q, si.tables, si.lens, si.max_ctx, cfg["scale"],
                      si.workspace, stream)
        if do_prefill and si.prefill is not None:
            q, table, ctx_before, out, ws = si.prefill
            pa_prefill_chunk(self.pool, self.layer, out, q, table, ctx_before, cfg["scale"], ws, stream)

    def run_step(self, step, fused=False, longest_first=False, shared=False):
        si = self.prepare(step, longest_first=longest_first, shared=shared)
        self.launch(si, fused=fused, shared=shared)
        return si
