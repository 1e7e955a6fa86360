/*
 * pa.h -- C ABI of a paged KV cache and PagedAttention hot path for AMD
 * Instinct MI355X (gfx950).
 *
 * Pages cited (title, site, section heading):
 *   [youngju] "vLLM 내부 구조 (2) — PagedAttention은 KV 캐시를 왜 페이지로 쪼갰는가",
 *             youngju.dev
 *   [icarus]  "PagedAttention", icarus.shaojiemike.top
 *   [ttlab]   "llm-kv-cache-02-serving-engine-kv", ttlab.hopto.org
 *
 * Conventions for every call below
 *   - Device pointers point at memory the caller allocated (hipMalloc or a
 *     torch tensor).  The library never allocates, frees or synchronises;
 *     each call only enqueues kernels on ``stream`` and returns.  The caller
 *     orders calls on one stream: copy-on-write copies, then appends, then
 *     attention.
 *   - ``pa_kv_pool`` is a host struct, read during the call only.
 *   - Return value: PA_OK (0) or a negative PA_E* code.  On an error nothing
 *     has been enqueued.  ``pa_status_string`` gives a message; for PA_EHIP
 *     it also carries the HIP error text of the failed launch.
 *   - Device-side contents (block ids, slots, copy pairs, context lengths)
 *     are trusted: the kernels do not range-check them.  Host-side sizes
 *     are checked.  In validate mode (pa_set_validate) every call first
 *     copies its device indices to the host and checks them.
 *   - Element types: PA_F32, PA_BF16, PA_F16.  Queries, new K/V and outputs
 *     use the pool's element type.  Arithmetic is fp32; outputs are rounded
 *     to nearest-even.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_F16 = 2 } pa_dtype;

enum {
  PA_OK = 0,
  PA_EINVAL = -1,  /* null pointer, bad size, head counts that do not divide, layer out of range */
  PA_ENOTSUP = -2, /* a (dtype, head_dim, block_size, query-group) combination that is not compiled */
  PA_ENOMEM = -3,  /* the block manager has too few free blocks (state unchanged) */
  PA_EHIP = -4,    /* a kernel launch failed */
  PA_ENOENT = -5,  /* the block manager has no such sequence (or it already exists) */
  PA_ESPACE = -6   /* an output buffer or workspace is too small */
};

/*
 * The physical block pool.  KV is cut into fixed-size blocks of
 * ``block_size`` token slots held in one shared pool ([youngju] "블록 테이블:
 * 논리적으로 연속, 물리적으로 흩어짐"; [ttlab] "블록과 블록 표"); the kernel
 * reads K/V by layer, KV head, token and head dimension ([icarus] "类比的边界").
 *
 * k, v: device, each [num_layers][num_kv_heads][num_blocks][block_size][head_dim]
 * row-major, element type ``dtype``, 16-byte aligned (every call returns
 * PA_EINVAL otherwise).  One block of one head is a contiguous
 * block_size * head_dim run (4 KiB for 16 x 128 bf16).  Slot s of a layer and
 * head is token s % block_size of block s / block_size.
 */
typedef struct pa_kv_pool {
  void* k;
  void* v;
  int32_t num_layers;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t block_size; /* 8, 16 or 32 */
  int32_t head_dim;   /* 64 or 128 */
  int32_t dtype;      /* pa_dtype */
} pa_kv_pool;

/*
 * Append: write each new token's K/V into its slot of the current block
 * ([icarus] "Block Table 如何工作"; [ttlab] "블록과 블록 표").
 *   k_new, v_new: device [T][num_kv_heads][head_dim], pool dtype, 16-byte
 *                 aligned.
 *   slot_mapping: device int32 [T]; a negative slot skips that row.  Slots
 *                 must be distinct and < num_blocks * block_size.
 *   T >= 0 (T == 0 enqueues nothing).
 * A bit copy: pool bytes equal the input bytes.
 */
int pa_cache_append(const pa_kv_pool* pool, int32_t layer, const void* k_new, const void* v_new,
                    const int32_t* slot_mapping, int32_t T, hipStream_t stream);

/*
 * Copy-on-write block copies: a block shared by several sequences is copied
 * only when one of them must write into it ([icarus] "支持块级共享"; [ttlab]
 * "블록을 함께 쓰기").
 *   pairs: device int32 [n][2] = (src, dst) physical block ids.  For each
 *          pair, the whole block -- every layer, every KV head, K and V -- is
 *          copied bit for bit.  No dst may appear as another pair's src or dst.
 *   n >= 0.
 */
int pa_copy_blocks(const pa_kv_pool* pool, const int32_t* pairs, int32_t n, hipStream_t stream);

/*
 * Workspace bytes ``pa_decode`` needs for a batch (0 when it will not split a
 * sequence over several workgroups).  Depends on host-side sizes, the
 * current device's CU count and the tuning overrides only.  A split planned
 * from max_ctx may still run unsplit: the kernels read context_lens and,
 * when the longest sequence holds no more blocks than one CU's share of the
 * batch, decode each (sequence, KV head) whole and leave the workspace
 * untouched (not with a PA_TUNE_DECODE_PART_BLOCKS override).
 */
size_t pa_decode_workspace_size(const pa_kv_pool* pool, int32_t B, int32_t H_q, int32_t max_ctx);

/*
 * Decode attention: each sequence's newest query reads all of its visible
 * K/V, found through its block table, and computes softmax(scale * q K^T) V
 * ([icarus] "Block Table 如何工作", "KV Cache 为什么难管理" and
 * "不会降低单请求的理论读取量"; [ttlab] "블록과 블록 표").
 *   out: device [B][H_q][head_dim], pool dtype (written for every sequence;
 *        a sequence with context_lens == 0 gets zeros).
 *   q:   device [B][H_q][head_dim], pool dtype.
 *   H_q: a multiple of num_kv_heads; query head h reads KV head
 *        h / (H_q / num_kv_heads).
 *   block_tables: device int32 [B][max_blocks]; entry j of row i is the
 *        physical block holding tokens j*block_size .. of sequence i.
 *   context_lens: device int32 [B], visible tokens per sequence (the token
 *        just appended included); each <= max_ctx and
 *        <= max_blocks * block_size.
 *   max_ctx: host upper bound of context_lens, used to size the grid.
 *   scale: multiplies q.k before the softmax.
 *   workspace: device, at least pa_decode_workspace_size(...) bytes
 *        (may be NULL when that is 0).  Contents need no initialisation.
 * Workgroups start in batch order.  When a batch has more (sequence, KV
 * head) pairs than the GPU has CUs, submitting it longest context first
 * keeps the long sequences from trailing (measured on MI355X: 8% on 64
 * lognormal lengths with 40 KV heads, 3.5% on 63 contexts of 1k-32k).
 */
int pa_decode(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t B, int32_t H_q,
              const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t max_ctx,
              float scale, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One decode step in one launch: each sequence's new token is appended and
 * then attended to with the rest of its context ([icarus] "Block Table 如何
 * 工作": the new token's K/V go into the current block, and the query reads
 * every visible block).  Same result, pool contents included, as
 * pa_cache_append(pool, layer, k_new, v_new, slot_mapping, B) followed by
 * pa_decode(pool, layer, out, q, B, ...).
 *   k_new, v_new: device [B][num_kv_heads][head_dim], pool dtype, 16-byte
 *        aligned: sequence b's new token.
 *   slot_mapping: device int32 [B]; slot_mapping[b] is the slot of position
 *        context_lens[b] - 1 in row b of block_tables (what the block manager
 *        returns for a one-token append), or negative to skip that write
 *        (then the pool's own row at that position is read, as pa_decode
 *        would).  The slot's block must not be shared with another sequence
 *        (copy-on-write copies come first).
 *   context_lens: include the new token (>= 1).
 *   Everything else as pa_decode, workspace size included.
 */
int pa_decode_append(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, const void* k_new,
                     const void* v_new, const int32_t* slot_mapping, int32_t B, int32_t H_q,
                     const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t max_ctx,
                     float scale, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  A split decode keeps its partials in
 * a static device array of PA_NOALLOC_SCRATCH_BYTES that the library holds
 * on every GPU it runs on until the process ends; the call itself allocates
 * nothing.  Same arguments and same results, bit for bit, as pa_decode with
 * a workspace.
 *   Returns PA_ESPACE, with nothing launched, when the batch's split needs
 *   more than PA_NOALLOC_SCRATCH_BYTES (pa_decode_workspace_size tells).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (concurrent streams, or host threads) race and must be serialised
 *   by the caller.  Nothing in the array needs to start at zero.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int pa_decode_noalloc(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t B, int32_t H_q,
                      const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t max_ctx,
                      float scale, hipStream_t stream);

/*
 * A measuring aid, not part of the hot path: pa_decode's grid, block-table
 * reads, unit walk and K/V loads, without the arithmetic.  Every loaded
 * 16-byte chunk of K and V is XORed into one uint32 per wave.  What
 * pa_decode's access pattern alone can stream; a benchmark states the
 * decode's rate as a fraction of this one.  bf16 pools, head_dim 64 or 128.
 *   checksums: device uint32, at least pa_gather_checksum_size(...) bytes;
 *        entry ((b * P + p) * H_kv + g) * W + w is wave w of partition p
 *        of (sequence b, KV head g) (P partitions, W waves: pa_decode's
 *        plan; when pa_decode would run the plan unsplit, so does this walk,
 *        and the entries of partitions 1 .. P-1 are 0).  The XOR of a
 *        (b, g)'s entries is the XOR of the K and V dwords of every token
 *        of the units its waves read (every visible token; at a partly
 *        filled last unit, its whole unit).
 *   Everything else as pa_decode (no q, no out, no workspace).
 */
size_t pa_gather_checksum_size(const pa_kv_pool* pool, int32_t B, int32_t H_q, int32_t max_ctx);
int pa_gather_checksum(const pa_kv_pool* pool, int32_t layer, int32_t B, int32_t H_q, const int32_t* block_tables,
                       int32_t max_blocks, const int32_t* context_lens, int32_t max_ctx, uint32_t* checksums,
                       size_t checksum_bytes, hipStream_t stream);

/*
 * Workspace bytes pa_prefill_chunk can use to split a chunk over its keys
 * (0 when it would not split).  Depends on host-side sizes and the current
 * device's CU count only.
 */
size_t pa_prefill_workspace_size(const pa_kv_pool* pool, int32_t T, int32_t H_q, int32_t ctx_before);

/*
 * Causal prefill chunk over paged K/V: a long prompt is processed in chunks
 * ([ttlab] "새 문제: 긴 프리필이 디코드를 멈춘다"); chunk row t sits at position
 * ctx_before + t and attends to positions 0 .. ctx_before + t of its own
 * sequence ([icarus] "KV Cache 为什么难管理").  The chunk's own K/V must
 * already be appended.  bf16 and f16 pools only (matrix cores).
 *   out, q: device [T][H_q][head_dim], pool dtype.
 *   block_table: device int32 [nb], nb >= ceil((ctx_before + T) / block_size).
 *   workspace: optional device buffer.  A short chunk after a long context
 *        (the rest of a prompt after a prefix-cache hit) has too few position
 *        tiles to fill the GPU; given pa_prefill_workspace_size(...) bytes,
 *        the call splits the keys over more workgroups and merges the splits
 *        (a second, small launch).  NULL: no split, same result up to
 *        rounding.  A non-NULL workspace smaller than needed is PA_ESPACE.
 *        Contents need no initialisation; 16-byte aligned.
 */
int pa_prefill_chunk(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t T, int32_t H_q,
                     const int32_t* block_table, int32_t nb, int32_t ctx_before, float scale, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * A mixed batch in one launch: the decode step of B sequences and the causal
 * prefill chunks of others.  Chunked prefill lets the running requests'
 * decode steps share a step with pieces of long prompts, so that the prompts
 * do not stall them ([ttlab] "새 문제: 긴 프리필이 디코드를 멈춘다").  Same
 * results as pa_decode(pool, layer, dec_out, dec_q, B, H_q, block_tables,
 * max_blocks, context_lens, max_ctx, scale, workspace, ...) followed by, for
 * each chunk c, pa_prefill_chunk(pool, layer, its rows of pf_out, its rows
 * of pf_q, chunks[c].T, H_q, row c of pf_tables, pf_max_blocks,
 * chunks[c].ctx_before, scale, NULL, 0, ...): bit for bit, since both halves
 * run the same per-workgroup code.  The decode half streams K/V from HBM
 * while the chunks' tiles run on the matrix cores of prefill_workgroups CUs.
 *   Decode arguments: as pa_decode (B may be 0).
 *   pf_q, pf_out: device [sum of T][H_q][head_dim], the chunks' rows packed
 *        in chunk order.
 *   chunks: host [n_chunks], 0 <= n_chunks <= 32; a chunk may have T = 0.
 *        The chunks' sequences must not be decoded in the same call, and
 *        their own K/V must already be appended.
 *   pf_tables: device int32 [n_chunks][pf_max_blocks]; row c is chunk c's
 *        block table, pf_max_blocks >= ceil((ctx_before + T) / block_size).
 *   prefill_workgroups: persistent workgroups that share the chunks'
 *        (position tile, KV head) items, longest first; 0 lets the library
 *        pick (a number that should let the chunks end before the decode).
 *        More than the number of items is clamped to it.
 *   workspace: as pa_decode, for the decode half (pa_decode_workspace_size).
 *   bf16 and f16 pools only.  The decode half runs 8 waves per workgroup
 *   whatever PA_TUNE_DECODE_WAVES says.  A split decode adds a second, small
 *   launch (the partition merge), as in pa_decode.
 */
typedef struct pa_chunk {
  int32_t T;          /* rows of the chunk */
  int32_t ctx_before; /* tokens of its sequence before the chunk */
} pa_chunk;

int pa_mixed_batch(const pa_kv_pool* pool, int32_t layer, void* dec_out, const void* dec_q, int32_t B, int32_t H_q,
                   const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t max_ctx,
                   void* pf_out, const void* pf_q, const pa_chunk* chunks, int32_t n_chunks,
                   const int32_t* pf_tables, int32_t pf_max_blocks, float scale, int32_t prefill_workgroups,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Decode attention of a batch whose sequences share leading blocks, reading
 * each shared block once for all of its sharers.  Parallel sampling, beam
 * search and common prompt prefixes leave several sequences whose block
 * tables start with the same physical blocks, shared by reference count
 * ([icarus] "支持块级共享"; [ttlab] "블록을 함께 쓰기"); pa_decode reads such
 * a block once per sharer.  Same results as pa_decode (up to rounding
 * order), for bf16 and f16 pools.
 *   groups: host [n_groups], 0 <= n_groups <= 64, non-overlapping: rows
 *        first_row .. first_row + n_rows - 1 of the batch all hold the same
 *        physical blocks in their first shared_blocks table entries, and
 *        each row's context covers them (shared_blocks * block_size <=
 *        context_lens).  Rows in no group are decoded as pa_decode would.
 *        The shared keys of a group run on the matrix cores for all its
 *        rows and query heads at once; the rest of each row, and the
 *        combination of the two, on the decode path.
 *   workspace: device, 16-byte aligned, at least
 *        pa_decode_shared_workspace_size(...) bytes (never 0 for B > 0).
 *   Everything else as pa_decode.  Two launches (the decode, then a merge).
 */
typedef struct pa_share_group {
  int32_t first_row;     /* first batch row of the group */
  int32_t n_rows;        /* >= 1 consecutive rows */
  int32_t shared_blocks; /* leading table entries all its rows share (>= 0) */
} pa_share_group;

size_t pa_decode_shared_workspace_size(const pa_kv_pool* pool, int32_t B, int32_t H_q, int32_t max_ctx,
                                       const pa_share_group* groups, int32_t n_groups);
int pa_decode_shared(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t B, int32_t H_q,
                     const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t max_ctx,
                     const pa_share_group* groups, int32_t n_groups, float scale, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * Host helper for pa_decode_shared: scans a batch's host-side block tables
 * ([B][max_blocks]) and context lengths ([B]) and returns the groups of
 * consecutive rows (at least min_rows >= 2 of them) whose tables start
 * with the same at least min_blocks >= 1 physical blocks, each fully inside
 * every row's context.  Greedy, in row order: a run grows while its rows
 * keep min_blocks common blocks, and shares as many as all of them hold.
 *   out: host [cap]; *n_out = groups found.  PA_ESPACE if more than cap.
 */
int pa_share_groups(const int32_t* block_tables, int32_t B, int32_t max_blocks, const int32_t* context_lens,
                    int32_t block_size, int32_t min_rows, int32_t min_blocks, pa_share_group* out, int32_t cap,
                    int32_t* n_out);

/*
 * Chunked prefill planning for pa_mixed_batch: a long prompt prefilled in
 * one step stalls every running request's next token, so it is cut into
 * chunks that share each step with the decodes, under a cap on the tokens a
 * step processes ([ttlab] "3. 연속 배칭: 빈 자리를 걸음마다 채우기", part "새
 * 문제: 긴 프리필이 디코드를 멈춘다").  The cap counts every token of the
 * step: each of the n_decode running decodes takes one and is never
 * postponed; the waiting prompts then take, in the given (arrival) order,
 * chunks of their remaining prompt tokens until the cap is spent, at most
 * max_chunks of them.  A prompt's chunk starts where its last one ended.
 *   prompts: host [n_prompts], prompt_len >= computed >= 0 (prompt tokens
 *            already prefilled).
 *   out: host [max_chunks]; *n_out = chunks planned (0 when the decodes
 *        fill the budget).  out[k] = (index into prompts, ctx_before = that
 *        prompt's computed, T = tokens of this chunk), in prompt order: the
 *        (T, ctx_before) pairs are pa_mixed_batch's chunk list.
 * Host only; no state.  The caller advances each prompt's computed by T.
 */
typedef struct pa_prompt_state {
  int32_t prompt_len;
  int32_t computed;
} pa_prompt_state;
typedef struct pa_chunk_plan {
  int32_t prompt;
  int32_t ctx_before;
  int32_t T;
} pa_chunk_plan;
int pa_plan_step(int32_t budget, int32_t n_decode, const pa_prompt_state* prompts, int32_t n_prompts,
                 int32_t max_chunks, pa_chunk_plan* out, int32_t* n_out);

/*
 * Validate mode (for debugging): when on, every call above copies the device
 * indices it would trust to the host on its stream (synchronising it) and
 * returns PA_EINVAL, with nothing launched, if any is wrong -- a block id
 * outside [0, num_blocks) among a sequence's visible blocks, a context
 * length outside [0, max_ctx] or past its table, a slot out of range or
 * repeated, a fused append's slot that is not position context_lens - 1 of
 * its row, a copy pair out of range or whose destination is reused, a share group
 * whose rows differ in their shared blocks or do not see all of them.  Off by
 * default; PA_VALIDATE=1 in the environment turns it on at load.  Not for
 * use under graph capture.  Returns the previous setting.
 */
int pa_set_validate(int on);

/*
 * Tuning overrides of the grid plans, for sweeps and tests (0 = the
 * library's own choice, the default).  Initial values come from the
 * environment variables of the same names (PA_DECODE_WAVES,
 * PA_DECODE_PART_BLOCKS, PA_PREFILL_SPLITS), read once at first use.
 *   PA_TUNE_DECODE_WAVES:       waves per decode workgroup (capped at 16, or
 *                               8 with more than 2 query heads per KV head).
 *   PA_TUNE_DECODE_PART_BLOCKS: blocks per decode partition (a sequence
 *                               longer than that is split and merged,
 *                               however the lengths fall).
 *   PA_TUNE_PREFILL_SPLITS:     1 never splits a prefill chunk over its keys;
 *                               n > 1 asks for n splits whenever the caller
 *                               gives a workspace.
 * Process-wide; workspace sizes follow the current values.  Returns the
 * previous value, or PA_EINVAL for an unknown key or a negative value.
 */
enum { PA_TUNE_DECODE_WAVES = 0, PA_TUNE_DECODE_PART_BLOCKS = 1, PA_TUNE_PREFILL_SPLITS = 2 };
int pa_set_tuning(int key, int value);

/* Message for a status code (thread-local copy of the last error detail). */
const char* pa_status_string(int status);

/*
 * Host block manager: the bookkeeping that produces block tables, slots and
 * copy-on-write pairs ([icarus] "Block Table 如何工作" and "支持块级共享";
 * [ttlab] "블록과 블록 표" and "블록을 함께 쓰기").
 *
 *   - Free pool: a FIFO queue initialised with ``free_order`` (a permutation
 *     of 0 .. num_blocks-1); allocation takes the front.
 *   - append_slots(seq, n): for each new position p, block j = p / block_size;
 *     if j is one past the table's end, take a free block; else if that
 *     block's refcount is above 1, copy-on-write: take a free block, emit
 *     (old, new), drop old's count by one.  slot = table[j]*block_size +
 *     p % block_size.  At most one copy-on-write pair per call.
 *   - fork(parent, child): child's table = parent's; every block's count +1.
 *   - free_seq(seq): walking the table from its last block to its first,
 *     drop each count; blocks reaching 0 go to the back of the free queue.
 *   - Out of blocks: PA_ENOMEM, nothing changed.
 * The handle is not thread-safe.  Sequence ids are any int32 values.
 */
typedef struct pa_bm pa_bm;

int pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order, pa_bm** out);
void pa_bm_destroy(pa_bm* bm);
int pa_bm_add_seq(pa_bm* bm, int32_t seq);
int pa_bm_fork(pa_bm* bm, int32_t parent, int32_t child);
/* slots_out: host int32 [n]; cow_pairs_out: host int32 [2] (may be NULL only if no pair results). */
int pa_bm_append_slots(pa_bm* bm, int32_t seq, int32_t n, int32_t* slots_out, int32_t* cow_pairs_out,
                       int32_t* n_cow_out);
/* Batched form: for i in order, append ns[i] slots to seqs[i].  slots_out: host [sum ns];
 * cow_pairs_out: host int32 [2*count].  All-or-nothing: on PA_ENOMEM no sequence changes. */
int pa_bm_append_slots_batch(pa_bm* bm, const int32_t* seqs, const int32_t* ns, int32_t count, int32_t* slots_out,
                             int32_t* cow_pairs_out, int32_t* n_cow_out);
int pa_bm_free_seq(pa_bm* bm, int32_t seq);
/* Copies up to cap entries of seq's table to out; *n_out = full table length. */
int pa_bm_block_table(pa_bm* bm, int32_t seq, int32_t* out, int32_t cap, int32_t* n_out);
/* Writes a [count][max_blocks] table (rows padded with pad) for seqs[0..count). */
int pa_bm_block_tables(pa_bm* bm, const int32_t* seqs, int32_t count, int32_t* out, int32_t max_blocks,
                       int32_t pad);
int pa_bm_seq_len(pa_bm* bm, int32_t seq);  /* >= 0, or PA_ENOENT */
int pa_bm_refcount(pa_bm* bm, int32_t block); /* >= 0, or PA_EINVAL */
int pa_bm_num_free(pa_bm* bm);
int pa_bm_free_list(pa_bm* bm, int32_t* out, int32_t cap); /* returns the count; copies up to cap */

/*
 * Capacity queries for admission and preemption: the block is the unit of
 * capacity, so a scheduler admits, waits or preempts by comparing these
 * with pa_bm_num_free ([icarus] "改善调度与回收"; [ttlab] "5. KV 자리가
 * 모자라면": a request that does not fit waits, and when even running
 * requests run short one of them gives its KV back and is computed again
 * later).  No state change.
 */
/* Free blocks pa_bm_append_slots(seq, n) would take: one per new logical
 * block, plus one when the partly filled last block is shared (>= 0). */
int pa_bm_blocks_needed(pa_bm* bm, int32_t seq, int32_t n);
/* Free-queue blocks that admitting this prompt would take
 * (pa_bm_add_seq_prefix, then pa_bm_append_tokens of the rest): cached
 * blocks of its prefix that wait in the free queue, plus a block for each
 * of the rest (>= 0). */
int pa_bm_admit_cost(pa_bm* bm, const int32_t* tokens, int32_t n, uint64_t extra);

/*
 * Automatic prefix caching ([ttlab] "4. 프리픽스 캐시"; [icarus] "支持块级共享"):
 * a later request whose prompt starts like an earlier one reuses the blocks
 * that already hold that prefix's K/V instead of computing them again.
 *   - Every full block of a sequence whose token ids the manager knows gets
 *     a key: sha256 over the previous block's key (32 zero bytes for the
 *     first block), the block's token ids as little-endian int32 and the
 *     sequence's ``extra`` (LoRA adapter, multimodal inputs, cache salt --
 *     hashed by the caller into 64 bits) as a little-endian uint64.  Through
 *     the previous key, a key stands for the whole prefix up to its block.
 *   - Only full blocks are cached.  A key already cached under another block
 *     leaves the new block uncached.
 *   - A freed block keeps its key and contents while it waits in the free
 *     queue (free_seq queues a sequence's blocks tail first); taking a block
 *     from the front of the queue evicts its key, so the least recently
 *     freed goes first.
 *   - Sequences made by pa_bm_add_seq and appended with pa_bm_append_tokens
 *     are keyed too (extra = 0).  pa_bm_append_slots or
 *     pa_bm_append_slots_batch (no token ids) stops a sequence's keying;
 *     the manager then behaves exactly as without caching.
 */
/* New sequence for a prompt: its table starts with the cached blocks of the
 * prompt's longest cached run of full blocks (taken out of the free queue
 * if they wait there; refcounts +1).  *n_hit_out = tokens those blocks hold
 * (a multiple of block_size).  The caller appends the rest of the prompt
 * with pa_bm_append_tokens.  Takes no free block, so it cannot fail with
 * PA_ENOMEM. */
int pa_bm_add_seq_prefix(pa_bm* bm, int32_t seq, const int32_t* tokens, int32_t n, uint64_t extra,
                         int32_t* n_hit_out);
/* pa_bm_append_slots for the given token ids (host int32 [n]); every block
 * the append fills is keyed and cached. */
int pa_bm_append_tokens(pa_bm* bm, int32_t seq, const int32_t* tokens, int32_t n, int32_t* slots_out,
                        int32_t* cow_pairs_out, int32_t* n_cow_out);
/* Prompt tokens a new request would find cached (>= 0); no state change. */
int pa_bm_prefix_lookup(pa_bm* bm, const int32_t* tokens, int32_t n, uint64_t extra);
int pa_bm_num_cached(pa_bm* bm); /* blocks with a cached key */
/* 1 and the 32-byte key in key_out if the block is cached, 0 if not. */
int pa_bm_block_key(pa_bm* bm, int32_t block, uint8_t* key_out);
/* SHA-256 (FIPS 180-4) of n bytes, the hash behind the block keys. */
int pa_sha256(const void* data, size_t n, uint8_t* digest_out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
