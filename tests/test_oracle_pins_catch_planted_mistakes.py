"""The oracle's pins must fail when the oracle is wrong.

Each case plants one plausible mistake in the oracle's source (a dropped term,
an off-by-one, a wrong index or order, a transposed operand, a wrong rounding),
loads the planted copy in place of the oracle module for the duration of the
case, and runs the pin tests that cover that function: at least one of them
has to fail.  Everything runs on the CPU; the oracle's files are never
modified.
"""

import importlib
import inspect
import json
import os
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

import test_oracle_attention as T_ATT  # noqa: E402
import test_oracle_block_manager as T_BM  # noqa: E402
import test_oracle_capacity as T_CAP  # noqa: E402
import test_oracle_encoding as T_ENC  # noqa: E402
import test_oracle_pool as T_POOL  # noqa: E402
import test_oracle_prefix_cache as T_PC  # noqa: E402
import test_oracle_run as T_RUN  # noqa: E402
import test_oracle_scheduler as T_SCHED  # noqa: E402


def plant(monkeypatch, module_name, old, new):
    """Load ``module_name`` from its source with ``old`` replaced by ``new``
    and route every reference to the original's functions and classes (in
    the oracle package and the pin modules) to the planted copy."""
    orig = importlib.import_module(module_name)
    src = inspect.getsource(orig)
    assert src.count(old) == 1, f"{module_name}: the planted text must occur exactly once: {old!r}"
    mut = types.ModuleType(module_name)
    mut.__package__ = orig.__package__
    mut.__file__ = orig.__file__
    exec(compile(src.replace(old, new), orig.__file__, "exec"), mut.__dict__)
    swap = {}
    for name, obj in list(vars(orig).items()):
        if name.startswith("__") or name not in mut.__dict__:
            continue
        if getattr(obj, "__module__", None) == module_name:
            swap[id(obj)] = mut.__dict__[name]
            monkeypatch.setattr(orig, name, mut.__dict__[name])
    for mname, m in list(sys.modules.items()):
        if m is None or not (mname.startswith("oracle") or mname.startswith("test_oracle")):
            continue
        for name, obj in list(vars(m).items()):
            if id(obj) in swap:
                monkeypatch.setattr(m, name, swap[id(obj)])


def cases_of(fn):
    """Keyword-argument sets of a pin test, from its parametrize marks."""
    cases = [{}]
    for mark in getattr(fn, "pytestmark", []):
        if mark.name != "parametrize":
            continue
        names = mark.args[0]
        names = [n.strip() for n in names.split(",")] if isinstance(names, str) else list(names)
        grown = []
        for c in cases:
            for v in mark.args[1]:
                v = v.values if hasattr(v, "values") else v
                v = tuple(v) if len(names) > 1 else (v,)
                grown.append({**c, **dict(zip(names, v))})
        cases = grown
    return cases


def first_failure(pins):
    """Run the pins in order; return a description of the first that fails."""
    with open(os.path.join(ROOT, "tests", "golden", "page_examples.json")) as f:
        golden = json.load(f)
    for fn in pins:
        for kw in cases_of(fn):
            if "golden" in inspect.signature(fn).parameters:
                kw = {**kw, "golden": golden}
            try:
                fn(**kw)
            except Exception as e:  # noqa: BLE001 - any failure of a pin counts
                return f"{fn.__name__}({kw}): {type(e).__name__}"
    return None


ATT = [T_ATT.test_closed_forms, T_ATT.test_gqa_group_mapping_is_contiguous,
       T_ATT.test_softmax_rows_sum_to_one_and_large_logits_are_safe, T_ATT.test_unused_slots_are_never_read,
       T_ATT.test_paged_decode_equals_sdpa_on_contiguous, T_ATT.test_prefill_chunk_equals_last_rows_of_causal_sdpa,
       T_ATT.test_permuting_physical_blocks_changes_nothing]
ENC = [T_ENC.test_bf16_round_nearest_even_matches_torch, T_ENC.test_fp16_and_fp32_round_trip_match_torch,
       T_ENC.test_bf16_decode_is_upper_half]
BM = [T_BM.test_600_tokens_take_38_blocks, T_BM.test_printed_block_tables, T_BM.test_self_check_two_requests,
      T_BM.test_waste_illustration, T_BM.test_cow_copies_only_the_written_shared_block,
      T_BM.test_free_returns_blocks_tail_first_at_the_back, T_BM.test_random_ops_keep_history_and_invariants,
      T_BM.test_brute_force_small_pools]
PC = [T_PC.test_key_is_sha256_of_previous_key_tokens_and_extra,
      T_PC.test_equal_tokens_after_different_prefixes_get_different_keys,
      T_PC.test_only_full_blocks_page_prefix_workload, T_PC.test_freed_blocks_wait_tail_first_and_lru_is_evicted_first,
      T_PC.test_hits_on_live_blocks_share_them, T_PC.test_append_without_token_ids_stops_keying,
      T_PC.test_failed_append_changes_nothing, T_PC.test_identity_pool_fuzz]
ADM = [T_PC.test_admission_queries_closed_forms, T_PC.test_admission_queries_equal_their_effect]
SCHED = [T_SCHED.test_page_caps_on_a_3500_token_input, T_SCHED.test_decodes_count_against_the_budget,
         T_SCHED.test_budget_below_the_decodes_leaves_no_prefill, T_SCHED.test_prompts_in_arrival_order_and_chunk_limit,
         T_SCHED.test_brute_force_small_cases]
CAP = [T_CAP.test_page_illustration, T_CAP.test_lognormal_lengths_waste_below_one_block,
       T_CAP.test_active_requests_in_the_page_pool, T_CAP.test_shared_blocks_count_once]
RUN = [T_RUN.test_config1_paged_equals_logical_and_uses_12_blocks, T_RUN.test_config4_copy_on_write_pairs_small,
       T_RUN.test_beam_search_paged_equals_logical_every_step]
POOL = [T_POOL.test_copy_duplicates_every_layer_head_and_both_tensors, T_POOL.test_copies_apply_in_order,
        T_POOL.test_append_writes_slot_block_and_offset]

# (id, module, text, planted text, pins that must catch it)
PLANTED = [
    # attention
    ("scale-dropped", "oracle.attention", "s = scale * (k[h // G] @ q[h])", "s = k[h // G] @ q[h]", ATT),
    ("gqa-head-modulo", "oracle.attention", "s = scale * (k[h // G] @ q[h])", "s = scale * (k[h % H_kv] @ q[h])", ATT),
    ("gqa-v-head-modulo", "oracle.attention", "out[h] = p[h] @ v[h // G]", "out[h] = p[h] @ v[h % H_kv]", ATT),
    ("k-for-v", "oracle.attention", "out[h] = p[h] @ v[h // G]", "out[h] = p[h] @ k[h // G]", ATT),
    ("softmax-unnormalised", "oracle.attention", "p[h] = e / e.sum()", "p[h] = e", ATT),
    ("softmax-no-max-shift", "oracle.attention", "e = np.exp(s - s.max())", "e = np.exp(s)", ATT),
    ("causal-excludes-self", "oracle.attention", "n = ctx_before + t + 1", "n = ctx_before + t", ATT),
    ("causal-ignores-context", "oracle.attention", "n = ctx_before + t + 1", "n = t + 1", ATT),
    ("gather-last-token-dropped", "oracle.attention", "n = min(bs, int(length) - j * bs)",
     "n = min(bs, int(length) - j * bs - 1)", ATT),
    ("gather-block-order", "oracle.attention", "phys = int(table[j])", "phys = int(table[need - 1 - j])", ATT),
    ("gather-k-as-v", "oracle.attention", "vs.append(pool.v[layer, :, phys, :n, :])",
     "vs.append(pool.k[layer, :, phys, :n, :])", ATT),
    # encoding
    ("bf16-truncates", "oracle.encoding", "r = hi + up.astype(np.uint64)", "r = hi", ENC),
    ("bf16-ties-away", "oracle.encoding", "up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))",
     "up = lo >= 0x8000", ENC),
    ("bf16-nan-to-inf", "oracle.encoding", "r = np.where(is_nan, np.uint64(BF16_QNAN), r)", "pass", ENC),
    ("bf16-lower-half", "oracle.encoding", "u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16",
     "u = np.asarray(b, dtype=np.uint16).astype(np.uint32)", ENC),
    # block manager
    ("cow-always", "oracle.block_manager", "elif self.ref[tab[j]] > 1:", "elif self.ref[tab[j]] >= 1:", BM),
    ("cow-never", "oracle.block_manager", "elif self.ref[tab[j]] > 1:", "elif False:", BM),
    ("cow-keeps-old-count", "oracle.block_manager", "                    self.ref[old] -= 1\n", "", BM),
    ("free-lifo", "oracle.block_manager", "b = self.free.popleft()", "b = self.free.pop()", BM),
    ("free-head-first", "oracle.block_manager", "for b in reversed(blocks):", "for b in blocks:", BM),
    ("slot-offset-wrong", "oracle.block_manager", "slots.append(tab[j] * self.block_size + p % self.block_size)",
     "slots.append(tab[j] * self.block_size + p % self.block_size - (p % self.block_size > 0))", BM),
    ("fork-no-refcount", "oracle.block_manager", "        for b in self.table[child]:\n            self.ref[b] += 1\n",
     "", BM),
    # prefix cache
    ("key-not-chained", "oracle.block_manager",
     "data = prev_key + struct.pack(", "data = struct.pack(", PC),
    ("key-ignores-extra", "oracle.block_manager", "+ struct.pack(\"<Q\", int(extra))", "", PC),
    ("key-big-endian-tokens", "oracle.block_manager", "struct.pack(f\"<{len(tokens)}i\"", "struct.pack(f\">{len(tokens)}i\"",
     PC),
    ("cache-partial-blocks", "oracle.block_manager", "if len(part) == self.block_size:  # block j is full: key it",
     "if len(part) == self.block_size or p == self.length[seq] + n - 1:", PC),
    ("no-eviction", "oracle.block_manager", "            del self.cache[self.key_of.pop(b)]\n", "            pass\n", PC),
    ("hit-not-pulled-from-queue", "oracle.block_manager", "                self.free.remove(b)\n", "                pass\n", PC),
    # admission queries
    ("blocks-needed-ignores-cow", "oracle.block_manager",
     "cow = 1 if ln % bs and self.ref[tab[-1]] > 1 else 0", "cow = 0", ADM),
    ("blocks-needed-cow-on-full-block", "oracle.block_manager",
     "cow = 1 if ln % bs and self.ref[tab[-1]] > 1 else 0", "cow = 1 if tab and self.ref[tab[-1]] > 1 else 0", ADM),
    ("blocks-needed-rounds-down", "oracle.block_manager",
     "fresh = -(-(ln + n) // bs) - len(tab)", "fresh = (ln + n) // bs - len(tab)", ADM),
    ("admit-cost-ignores-waiting-hits", "oracle.block_manager", "            waiting += self.ref[b] == 0\n", "", ADM),
    ("admit-cost-ignores-hits", "oracle.block_manager",
     "return waiting + -(-len(tokens) // bs) - hits", "return waiting + -(-len(tokens) // bs)", ADM),
    # chunked-prefill planner
    ("decodes-not-counted", "oracle.scheduler", "left = budget - n_decode", "left = budget", SCHED),
    ("chunk-ignores-budget", "oracle.scheduler", "t = min(rest, left)", "t = rest", SCHED),
    ("chunk-restarts-at-zero", "oracle.scheduler", "out.append((i, done, t))", "out.append((i, 0, t))", SCHED),
    ("no-chunk-limit", "oracle.scheduler", "if left <= 0 or len(out) == max_chunks:", "if left <= 0:", SCHED),
    ("prompts-last-first", "oracle.scheduler", "for i, (length, done) in enumerate(prompts):",
     "for i, (length, done) in reversed(list(enumerate(prompts))):", SCHED),
    # capacity
    ("shared-blocks-counted-twice", "oracle.capacity", "blocks = set()", "blocks = []", CAP),
    ("waste-off-by-one", "oracle.capacity", "return [len(bm.block_table(s)) * bm.block_size - bm.seq_len(s) for s in seqs]",
     "return [len(bm.block_table(s)) * bm.block_size - bm.seq_len(s) + 1 for s in seqs]", CAP),
    ("n-active-rounds-up", "oracle.capacity", "return capacity_tokens // footprint_tokens",
     "return -(-capacity_tokens // footprint_tokens)", CAP),
    # pool
    ("copy-k-only", "oracle.pool", "            self.v[:, :, int(dst)] = self.v[:, :, int(src)]\n", "", POOL),
    ("copy-first-layer-only", "oracle.pool", "self.k[:, :, int(dst)] = self.k[:, :, int(src)]",
     "self.k[0, :, int(dst)] = self.k[0, :, int(src)]", POOL),
    ("copy-reversed-order", "oracle.pool", "for src, dst in pairs:", "for src, dst in reversed(pairs):", POOL),
    ("append-offset-swapped", "oracle.pool", "block, offset = divmod(slot, self.bs)",
     "offset, block = divmod(slot, self.bs)", POOL),
    ("append-negative-slot-written", "oracle.pool", "            if slot < 0:\n                continue\n", "", POOL),
    # workload driver
    ("copy-after-write", "oracle.run", """        if self.pool is not None:
            self.pool.copy_blocks(pairs)
        self._write(step.appends, slots, step.k_new, step.v_new)
""", """        self._write(step.appends, slots, step.k_new, step.v_new)
        if self.pool is not None:
            self.pool.copy_blocks(pairs)
""", RUN),
    ("decode-misses-new-token", "oracle.run",
     "k, v = attention.gather(self.pool, self.layer, self.bm.block_table(seq), self.bm.seq_len(seq))",
     "k, v = attention.gather(self.pool, self.layer, self.bm.block_table(seq), self.bm.seq_len(seq) - 1)", RUN),
    # the same pool mistakes, caught end to end by the workload pins too
    ("copy-k-only-run", "oracle.pool", "            self.v[:, :, int(dst)] = self.v[:, :, int(src)]\n", "", RUN),
    ("append-offset-swapped-run", "oracle.pool", "block, offset = divmod(slot, self.bs)",
     "offset, block = divmod(slot, self.bs)", RUN + ATT),
]


@pytest.mark.parametrize("case", PLANTED, ids=[c[0] for c in PLANTED])
@pytest.mark.filterwarnings("ignore::RuntimeWarning")  # a planted mistake may overflow on purpose
def test_planted_mistake_fails_a_pin(case, monkeypatch):
    _, module, old, new, pins = case
    plant(monkeypatch, module, old, new)
    caught = first_failure(pins)
    assert caught is not None, f"no pin fails when the oracle has {case[0]!r}"


def test_pins_pass_on_the_oracle_as_it_is():
    assert first_failure(ATT + ENC + PC[:4] + ADM + SCHED + CAP + RUN[:1] + POOL) is None
