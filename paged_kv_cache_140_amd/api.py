"""Python binding of the C ABI: argument marshalling only.

Each function has the name of the C entry point it calls and takes torch
tensors for device buffers.  Every step of the hot path runs in the HIP
kernels of ``libpa.so``; nothing here computes on the data.
"""

import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import KVPoolStruct, PAError, check, lib

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
PA_DTYPE = {"f32": _lib.PA_F32, "bf16": _lib.PA_BF16, "f16": _lib.PA_F16}


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


class KVPool:
    """The physical block pool: K and V, each [layers][kv_heads][blocks][block_size][head_dim].

    Device memory comes from torch; the library only reads and writes it.
    """

    def __init__(self, num_layers, num_kv_heads, num_blocks, block_size, head_dim, dtype, device="cuda",
                 k=None, v=None):
        self.num_layers, self.num_kv_heads, self.num_blocks = num_layers, num_kv_heads, num_blocks
        self.block_size, self.head_dim, self.dtype = block_size, head_dim, dtype
        shape = (num_layers, num_kv_heads, num_blocks, block_size, head_dim)
        self.k = k if k is not None else torch.empty(shape, dtype=TORCH_DTYPE[dtype], device=device)
        self.v = v if v is not None else torch.empty(shape, dtype=TORCH_DTYPE[dtype], device=device)
        _need(self.k, "pool.k", TORCH_DTYPE[dtype], shape)
        _need(self.v, "pool.v", TORCH_DTYPE[dtype], shape)

    @property
    def torch_dtype(self):
        return TORCH_DTYPE[self.dtype]

    def struct(self):
        return KVPoolStruct(self.k.data_ptr(), self.v.data_ptr(), self.num_layers, self.num_kv_heads,
                            self.num_blocks, self.block_size, self.head_dim, PA_DTYPE[self.dtype])

    def nbytes(self):
        return 2 * self.k.numel() * self.k.element_size()


def pa_cache_append(pool, layer, k_new, v_new, slot_mapping, stream=None):
    T = int(k_new.shape[0])
    row = (T, pool.num_kv_heads, pool.head_dim)
    _need(k_new, "k_new", pool.torch_dtype, row)
    _need(v_new, "v_new", pool.torch_dtype, row)
    _need(slot_mapping, "slot_mapping", torch.int32, (T,))
    s = pool.struct()
    check(lib().pa_cache_append(ctypes.byref(s), layer, _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), T,
                                _stream(stream)), "pa_cache_append")


def pa_copy_blocks(pool, pairs, stream=None):
    n = int(pairs.shape[0])
    _need(pairs, "pairs", torch.int32, (n, 2))
    s = pool.struct()
    check(lib().pa_copy_blocks(ctypes.byref(s), _ptr(pairs), n, _stream(stream)), "pa_copy_blocks")


def pa_decode_workspace_size(pool, B, H_q, max_ctx):
    s = pool.struct()
    return int(lib().pa_decode_workspace_size(ctypes.byref(s), B, H_q, max_ctx))


def pa_decode(pool, layer, out, q, block_tables, context_lens, max_ctx, scale, workspace=None, stream=None):
    B, H_q, d = (int(x) for x in q.shape)
    _need(q, "q", pool.torch_dtype, (B, H_q, pool.head_dim))
    _need(out, "out", pool.torch_dtype, (B, H_q, pool.head_dim))
    _need(block_tables, "block_tables", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B][max_blocks]")
    _need(context_lens, "context_lens", torch.int32, (B,))
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    s = pool.struct()
    check(lib().pa_decode(ctypes.byref(s), layer, _ptr(out), _ptr(q), B, H_q, _ptr(block_tables),
                          int(block_tables.shape[1]), _ptr(context_lens), int(max_ctx), float(scale),
                          _ptr(workspace), ws_bytes, _stream(stream)), "pa_decode")


def pa_decode_noalloc(pool, layer, out, q, block_tables, context_lens, max_ctx, scale, stream=None):
    """pa_decode with no workspace: a split keeps its partials in the
    library's static per-GPU scratch (calls on one GPU must not overlap)."""
    B, H_q, d = (int(x) for x in q.shape)
    _need(q, "q", pool.torch_dtype, (B, H_q, pool.head_dim))
    _need(out, "out", pool.torch_dtype, (B, H_q, pool.head_dim))
    _need(block_tables, "block_tables", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B][max_blocks]")
    _need(context_lens, "context_lens", torch.int32, (B,))
    s = pool.struct()
    check(lib().pa_decode_noalloc(ctypes.byref(s), layer, _ptr(out), _ptr(q), B, H_q, _ptr(block_tables),
                                  int(block_tables.shape[1]), _ptr(context_lens), int(max_ctx), float(scale),
                                  _stream(stream)), "pa_decode_noalloc")


def _groups_arg(groups):
    groups = [(int(a), int(b), int(c)) for a, b, c in groups]
    arr = (_lib.ShareGroupStruct * max(len(groups), 1))(*[_lib.ShareGroupStruct(*g) for g in groups])
    return arr, len(groups)


def pa_decode_shared_workspace_size(pool, B, H_q, max_ctx, groups):
    arr, n = _groups_arg(groups)
    s = pool.struct()
    return int(lib().pa_decode_shared_workspace_size(ctypes.byref(s), int(B), int(H_q), int(max_ctx), arr, n))


def decode_shared_workspace(pool, B, H_q, max_ctx, groups, device="cuda"):
    """The workspace tensor pa_decode_shared needs for this batch and groups."""
    n = pa_decode_shared_workspace_size(pool, B, H_q, max_ctx, groups)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def pa_decode_shared(pool, layer, out, q, block_tables, context_lens, max_ctx, scale, groups, workspace,
                     stream=None):
    """pa_decode for a batch whose rows share leading blocks: ``groups`` is a
    list of (first_row, n_rows, shared_blocks)."""
    B, H_q, d = (int(x) for x in q.shape)
    _need(q, "q", pool.torch_dtype, (B, H_q, pool.head_dim))
    _need(out, "out", pool.torch_dtype, (B, H_q, pool.head_dim))
    _need(block_tables, "block_tables", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B][max_blocks]")
    _need(context_lens, "context_lens", torch.int32, (B,))
    _need(workspace, "workspace")
    arr, n = _groups_arg(groups)
    s = pool.struct()
    check(lib().pa_decode_shared(ctypes.byref(s), layer, _ptr(out), _ptr(q), B, H_q, _ptr(block_tables),
                                 int(block_tables.shape[1]), _ptr(context_lens), int(max_ctx), arr, n, float(scale),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
          "pa_decode_shared")


def pa_share_groups(block_tables, context_lens, block_size, min_rows=2, min_blocks=1):
    """Groups of consecutive rows sharing leading full blocks, from host
    tables (int32 [B][max_blocks]) and context lengths ([B]) -> list of
    (first_row, n_rows, shared_blocks)."""
    tab, tp = _arr(block_tables)
    if tab.ndim != 2:
        raise ValueError("block_tables must be [B][max_blocks]")
    lens, lp = _arr(context_lens)
    B, maxb = tab.shape
    cap = max(B // 2, 1)
    out = (_lib.ShareGroupStruct * cap)()
    n = ctypes.c_int32(0)
    check(lib().pa_share_groups(tp, B, maxb, lp, int(block_size), int(min_rows), int(min_blocks), out, cap,
                                ctypes.byref(n)), "pa_share_groups")
    return [(out[i].first_row, out[i].n_rows, out[i].shared_blocks) for i in range(n.value)]


def pa_gather_checksum_size(pool, B, H_q, max_ctx):
    s = pool.struct()
    return int(lib().pa_gather_checksum_size(ctypes.byref(s), int(B), int(H_q), int(max_ctx)))


def pa_gather_checksum(pool, layer, H_q, block_tables, context_lens, max_ctx, checksums=None, stream=None):
    """pa_decode's walk and loads without the arithmetic (a measuring aid):
    returns the uint32 checksum tensor ([B][P][H_kv][W] per-wave XORs)."""
    B = int(context_lens.shape[0])
    _need(block_tables, "block_tables", torch.int32)
    _need(context_lens, "context_lens", torch.int32, (B,))
    s = pool.struct()
    n = int(lib().pa_gather_checksum_size(ctypes.byref(s), B, int(H_q), int(max_ctx)))
    if checksums is None:
        checksums = torch.empty(max(n // 4, 1), dtype=torch.int32, device=block_tables.device)
    check(lib().pa_gather_checksum(ctypes.byref(s), layer, B, int(H_q), _ptr(block_tables),
                                   int(block_tables.shape[1]), _ptr(context_lens), int(max_ctx), _ptr(checksums),
                                   checksums.numel() * checksums.element_size(), _stream(stream)),
          "pa_gather_checksum")
    return checksums


def pa_plan_step(budget, n_decode, prompts, max_chunks=32):
    """One step's prefill chunks under a token budget (pa_plan_step):
    prompts = [(prompt_len, computed)] in arrival order -> [(prompt index,
    ctx_before, T)]."""
    arr = (_lib.PromptStateStruct * max(len(prompts), 1))(
        *[_lib.PromptStateStruct(int(n), int(c)) for n, c in prompts])
    out = (_lib.ChunkPlanStruct * max(int(max_chunks), 1))()
    n = ctypes.c_int32(0)
    check(lib().pa_plan_step(int(budget), int(n_decode), arr, len(prompts), int(max_chunks), out, ctypes.byref(n)),
          "pa_plan_step")
    return [(out[i].prompt, out[i].ctx_before, out[i].T) for i in range(n.value)]


def pa_decode_append(pool, layer, out, q, k_new, v_new, slot_mapping, block_tables, context_lens, max_ctx, scale,
                     workspace=None, stream=None):
    """One decode step in one launch: append each sequence's new token
    (k_new/v_new [B][H_kv][d] at slot_mapping [B]), then decode."""
    B, H_q, d = (int(x) for x in q.shape)
    _need(q, "q", pool.torch_dtype, (B, H_q, pool.head_dim))
    _need(out, "out", pool.torch_dtype, (B, H_q, pool.head_dim))
    _need(k_new, "k_new", pool.torch_dtype, (B, pool.num_kv_heads, pool.head_dim))
    _need(v_new, "v_new", pool.torch_dtype, (B, pool.num_kv_heads, pool.head_dim))
    _need(slot_mapping, "slot_mapping", torch.int32, (B,))
    _need(block_tables, "block_tables", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B][max_blocks]")
    _need(context_lens, "context_lens", torch.int32, (B,))
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    s = pool.struct()
    check(lib().pa_decode_append(ctypes.byref(s), layer, _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new),
                                 _ptr(slot_mapping), B, H_q, _ptr(block_tables), int(block_tables.shape[1]),
                                 _ptr(context_lens), int(max_ctx), float(scale), _ptr(workspace), ws_bytes,
                                 _stream(stream)), "pa_decode_append")


def pa_prefill_workspace_size(pool, T, H_q, ctx_before):
    s = pool.struct()
    return int(lib().pa_prefill_workspace_size(ctypes.byref(s), int(T), int(H_q), int(ctx_before)))


def prefill_workspace(pool, T, H_q, ctx_before, device="cuda"):
    """A workspace tensor that lets pa_prefill_chunk split a short chunk over
    its keys (None when it would not split)."""
    n = pa_prefill_workspace_size(pool, T, H_q, ctx_before)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def pa_prefill_chunk(pool, layer, out, q, block_table, ctx_before, scale, workspace=None, stream=None):
    T, H_q, d = (int(x) for x in q.shape)
    _need(q, "q", pool.torch_dtype, (T, H_q, pool.head_dim))
    _need(out, "out", pool.torch_dtype, (T, H_q, pool.head_dim))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 1:
        raise ValueError("block_table must be 1-D")
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    s = pool.struct()
    check(lib().pa_prefill_chunk(ctypes.byref(s), layer, _ptr(out), _ptr(q), T, H_q, _ptr(block_table),
                                 int(block_table.shape[0]), int(ctx_before), float(scale), _ptr(workspace), ws_bytes,
                                 _stream(stream)), "pa_prefill_chunk")


def pa_mixed_batch(pool, layer, dec_out, dec_q, block_tables, context_lens, max_ctx, pf_out, pf_q, chunks,
                   pf_tables, scale, prefill_workgroups=0, workspace=None, stream=None):
    """A decode batch (as pa_decode) and prefill chunks (as pa_prefill_chunk
    each) in one launch.  dec_q may have B = 0 rows.  chunks: list of
    (T, ctx_before); their rows are packed in order in pf_q / pf_out
    ([sum T][H_q][d]); pf_tables: int32 [len(chunks)][max_blocks], row c the
    block table of chunk c."""
    B, H_q, _ = (int(x) for x in dec_q.shape)
    chunks = [(int(t), int(c)) for t, c in chunks]
    rows = sum(t for t, _ in chunks)
    _need(dec_q, "dec_q", pool.torch_dtype, (B, H_q, pool.head_dim))
    _need(dec_out, "dec_out", pool.torch_dtype, (B, H_q, pool.head_dim))
    _need(block_tables, "block_tables", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B][max_blocks]")
    _need(context_lens, "context_lens", torch.int32, (B,))
    _need(pf_q, "pf_q", pool.torch_dtype, (rows, H_q, pool.head_dim))
    _need(pf_out, "pf_out", pool.torch_dtype, (rows, H_q, pool.head_dim))
    _need(pf_tables, "pf_tables", torch.int32)
    if pf_tables.dim() != 2 or pf_tables.shape[0] != len(chunks):
        raise ValueError("pf_tables must be [n_chunks][max_blocks]")
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    arr = (_lib.ChunkStruct * max(len(chunks), 1))(*[_lib.ChunkStruct(t, c) for t, c in chunks])
    s = pool.struct()
    check(lib().pa_mixed_batch(ctypes.byref(s), layer, _ptr(dec_out), _ptr(dec_q), B, H_q, _ptr(block_tables),
                               int(block_tables.shape[1]), _ptr(context_lens), int(max_ctx), _ptr(pf_out),
                               _ptr(pf_q), arr, len(chunks), _ptr(pf_tables), int(pf_tables.shape[1]), float(scale),
                               int(prefill_workgroups), _ptr(workspace), ws_bytes, _stream(stream)),
          "pa_mixed_batch")


def pa_set_validate(on):
    """Validate mode on or off (returns the previous setting)."""
    return bool(lib().pa_set_validate(1 if on else 0))


TUNING_KEYS = {"decode_waves": _lib.PA_TUNE_DECODE_WAVES, "decode_part_blocks": _lib.PA_TUNE_DECODE_PART_BLOCKS,
               "prefill_splits": _lib.PA_TUNE_PREFILL_SPLITS}


def pa_set_tuning(key, value):
    """Set a grid-plan override ("decode_waves", "decode_part_blocks",
    "prefill_splits"; 0 = the library's choice); returns the previous value."""
    st = lib().pa_set_tuning(TUNING_KEYS[key], int(value))
    if st < 0:
        check(st, "pa_set_tuning")
    return st


class tuning:
    """Context manager: grid-plan overrides for the duration of a block,
    e.g. ``with tuning(decode_waves=4, decode_part_blocks=3): ...``."""

    def __init__(self, **values):
        self.values = values
        self.saved = {}

    def __enter__(self):
        for k, v in self.values.items():
            self.saved[k] = pa_set_tuning(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self.saved.items():
            pa_set_tuning(k, v)
        return False


def pa_sha256(data):
    """SHA-256 digest (32 bytes) of ``data``, computed by the library."""
    data = bytes(data)
    out = ctypes.create_string_buffer(32)
    check(lib().pa_sha256(data, len(data), out), "pa_sha256")
    return out.raw


def decode_workspace(pool, B, H_q, max_ctx, device="cuda"):
    """A workspace tensor of the size pa_decode needs (None if it needs none)."""
    n = pa_decode_workspace_size(pool, B, H_q, max_ctx)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


# ----------------------------------------------------------------- allocator

class OutOfBlocks(PAError):
    pass


def _arr(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class BlockManager:
    """Host block manager (``pa_bm_*``): free queue, tables, refcounts, CoW."""

    def __init__(self, num_blocks, block_size, free_order):
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        order, p = _arr(free_order)
        if order.shape != (self.num_blocks,):
            raise ValueError("free_order must have num_blocks entries")
        h = ctypes.c_void_p()
        check(lib().pa_bm_create(self.num_blocks, self.block_size, p, ctypes.byref(h)), "pa_bm_create")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib._lib is not None:
            _lib._lib.pa_bm_destroy(h)
            self._h = None

    def _check(self, st, where):
        if st == _lib.PA_ENOMEM:
            raise OutOfBlocks(st, where)
        return check(st, where)

    def add_seq(self, seq):
        self._check(lib().pa_bm_add_seq(self._h, int(seq)), "pa_bm_add_seq")

    def fork(self, parent, child):
        self._check(lib().pa_bm_fork(self._h, int(parent), int(child)), "pa_bm_fork")

    def free_seq(self, seq):
        self._check(lib().pa_bm_free_seq(self._h, int(seq)), "pa_bm_free_seq")

    def append_slots(self, seq, n):
        """-> (slots int32 [n], list of (src, dst) pairs)."""
        slots, ps = _arr(np.zeros(max(int(n), 1)))
        pair, pp = _arr(np.zeros(2))
        npair = ctypes.c_int32(0)
        self._check(lib().pa_bm_append_slots(self._h, int(seq), int(n), ps, pp, ctypes.byref(npair)),
                    "pa_bm_append_slots")
        return slots[:int(n)].copy(), ([(int(pair[0]), int(pair[1]))] if npair.value else [])

    # -- prefix cache --------------------------------------------------------
    def add_seq_prefix(self, seq, tokens, extra=0):
        """New sequence for a prompt; returns the prompt tokens its cached
        prefix blocks already hold."""
        toks, tp = _arr(np.asarray(tokens) if len(tokens) else np.zeros(1))
        hit = ctypes.c_int32(0)
        self._check(lib().pa_bm_add_seq_prefix(self._h, int(seq), tp, len(tokens), int(extra) & (2**64 - 1),
                                               ctypes.byref(hit)), "pa_bm_add_seq_prefix")
        return hit.value

    def append_tokens(self, seq, tokens):
        """append_slots for these token ids (full blocks get cached) ->
        (slots int32 [n], list of (src, dst) pairs)."""
        n = len(tokens)
        toks, tp = _arr(np.asarray(tokens) if n else np.zeros(1))
        slots, ps = _arr(np.zeros(max(n, 1)))
        pair, pp = _arr(np.zeros(2))
        npair = ctypes.c_int32(0)
        self._check(lib().pa_bm_append_tokens(self._h, int(seq), tp, n, ps, pp, ctypes.byref(npair)),
                    "pa_bm_append_tokens")
        return slots[:n].copy(), ([(int(pair[0]), int(pair[1]))] if npair.value else [])

    def prefix_lookup(self, tokens, extra=0):
        toks, tp = _arr(np.asarray(tokens) if len(tokens) else np.zeros(1))
        st = lib().pa_bm_prefix_lookup(self._h, tp, len(tokens), int(extra) & (2**64 - 1))
        if st < 0:
            self._check(st, "pa_bm_prefix_lookup")
        return st

    def num_cached(self):
        return lib().pa_bm_num_cached(self._h)

    def blocks_needed(self, seq, n):
        """Free blocks append_slots(seq, n) would take."""
        st = lib().pa_bm_blocks_needed(self._h, int(seq), int(n))
        if st < 0:
            self._check(st, "pa_bm_blocks_needed")
        return st

    def admit_cost(self, tokens, extra=0):
        """Free-queue blocks admitting this prompt would take."""
        toks, tp = _arr(np.asarray(tokens) if len(tokens) else np.zeros(1))
        st = lib().pa_bm_admit_cost(self._h, tp, len(tokens), int(extra) & (2**64 - 1))
        if st < 0:
            self._check(st, "pa_bm_admit_cost")
        return st

    def block_key_of(self, block):
        """The block's 32-byte cache key, or None if it is not cached."""
        buf = ctypes.create_string_buffer(32)
        st = lib().pa_bm_block_key(self._h, int(block), buf)
        if st < 0:
            self._check(st, "pa_bm_block_key")
        return buf.raw if st == 1 else None

    def append_slots_batch(self, seqs, ns):
        """All-or-nothing batch -> (slots int32 [sum ns], pairs int32 [k][2])."""
        seqs_a, sp = _arr(seqs)
        ns_a, np_ = _arr(ns)
        total = int(ns_a.sum())
        slots, slp = _arr(np.zeros(max(total, 1)))
        pairs, pp = _arr(np.zeros(2 * max(len(seqs_a), 1)))
        npair = ctypes.c_int32(0)
        self._check(lib().pa_bm_append_slots_batch(self._h, sp, np_, len(seqs_a), slp, pp, ctypes.byref(npair)),
                    "pa_bm_append_slots_batch")
        return slots[:total].copy(), pairs[:2 * npair.value].reshape(-1, 2).copy()

    def block_table(self, seq):
        n = ctypes.c_int32(0)
        self._check(lib().pa_bm_block_table(self._h, int(seq), None, 0, ctypes.byref(n)), "pa_bm_block_table")
        out, p = _arr(np.zeros(max(n.value, 1)))
        self._check(lib().pa_bm_block_table(self._h, int(seq), p, n.value, ctypes.byref(n)), "pa_bm_block_table")
        return [int(x) for x in out[:n.value]]

    def block_tables(self, seqs, max_blocks, pad=0):
        seqs_a, sp = _arr(seqs)
        out, p = _arr(np.zeros((len(seqs_a), max_blocks)))
        self._check(lib().pa_bm_block_tables(self._h, sp, len(seqs_a), p, int(max_blocks), int(pad)),
                    "pa_bm_block_tables")
        return out

    def seq_len(self, seq):
        st = lib().pa_bm_seq_len(self._h, int(seq))
        if st < 0:
            self._check(st, "pa_bm_seq_len")
        return st

    def refcount(self, block):
        st = lib().pa_bm_refcount(self._h, int(block))
        if st < 0:
            self._check(st, "pa_bm_refcount")
        return st

    def num_free(self):
        return lib().pa_bm_num_free(self._h)

    def free_list(self):
        n = lib().pa_bm_free_list(self._h, None, 0)
        out, p = _arr(np.zeros(max(n, 1)))
        lib().pa_bm_free_list(self._h, p, n)
        return [int(x) for x in out[:n]]
