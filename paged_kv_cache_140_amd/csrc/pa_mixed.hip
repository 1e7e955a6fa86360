// One launch for a mixed batch: the decode step of many sequences plus the
// causal prefill chunks of others.
//
// What it computes: exactly what pa_decode and pa_prefill_chunk (once per
// chunk) compute for the same arguments.  Chunked prefill feeds a long prompt a chunk at a time
// and lets the decode steps of the running requests share the same step, so
// that a long prefill does not stall them ([ttlab]
// "llm-kv-cache-02-serving-engine-kv", ttlab.hopto.org, section "새 문제: 긴
// 프리필이 디코드를 멈춘다").
//
// Why one launch: the two halves bound on different units.  Decode streams
// every visible K/V byte once (HBM-bound, a few flops per byte); the chunk
// reuses each staged K/V tile for 256 query rows (matrix-core bound).  Run
// one after the other, the matrix cores idle through the decode and HBM
// idles through the chunks.  Here the chunks' tiles go to a bounded number
// of persistent workgroups at the front of the grid, and the decode's
// workgroups stream on every other CU at the same time.
//  * grid = [prefill workgroups | decode workgroups (kv head, partition,
//    sequence), kv head fastest, as in the decode kernel].  Both halves run
//    8 waves; one CU holds one workgroup of either kind (their register
//    needs are alike), so a prefill workgroup keeps its CU to itself.
//  * prefill workgroup p of n takes items p, 2n-1-p, 2n+p, 4n-1-p, ... of
//    the chunks' (position tile, KV head) items, chunk by chunk with the
//    longest chunk first and, inside a chunk, the tiles longest first (a
//    later tile sees more keys): a snake order that evens out the work per
//    workgroup.  With n a multiple of 8, all prefill workgroups of one XCD
//    work on the same KV head in the same round, so its K/V stays in that
//    XCD's L2.  The chunk list travels in the kernel arguments.
//  * the decode half is split into partitions exactly as pa_decode splits
//    it; a split decode is finished by the same merge kernel (a second,
//    small launch).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "pa_decode_dev.h"
#include "pa_prefill_dev.h"

namespace pa {

constexpr int kMaxChunks = 32;

// The prefill chunks of a launch, in item order (longest chunk first).
struct ChunkList {
  int32_t n;
  int32_t T[kMaxChunks];           // rows
  int32_t ctx_before[kMaxChunks];  // cached tokens before the chunk
  int32_t row0[kMaxChunks];        // first row in the packed q / out
  int32_t table_row[kMaxChunks];   // its row of the chunk tables
  int32_t items_before[kMaxChunks + 1];
};

template <typename E, int D, int G, int BS>
__global__ void __launch_bounds__(kPrefillThreads)
    mixed_kernel(char* __restrict__ pool_k, char* __restrict__ pool_v, int64_t layer_off, int64_t head_stride,
                 int32_t H_kv, int32_t H_q, float scale_log2,
                 // decode half
                 const char* __restrict__ dq, void* __restrict__ dout, const int32_t* __restrict__ block_tables,
                 int32_t max_blocks, const int32_t* __restrict__ context_lens, int32_t blocks_per_part,
                 int32_t num_parts, int32_t unsplit_cus, float* __restrict__ ws_ml, float* __restrict__ ws_acc,
                 // prefill half
                 const uint16_t* __restrict__ pq, uint16_t* __restrict__ pout, const int32_t* __restrict__ ptables,
                 int32_t pt_stride, int32_t n_pre, ChunkList ch) {
  static_assert(kPrefillThreads == 512, "both halves run 8 waves");
  static_assert(8 * G * (D + 2) * sizeof(float) <= sizeof(PrefillLds<D>), "decode merge fits the prefill LDS");
  __shared__ __attribute__((aligned(1024))) PrefillLds<D> lds;
  const int id = blockIdx.x;
  if (id < n_pre) {
    constexpr int TP = kRowsPerWave * kPrefillWaves / G;
    const int n_items = ch.items_before[ch.n];
    for (int r = 0;; ++r) {
      const int k = r * n_pre + ((r & 1) ? n_pre - 1 - id : id);  // k-th item in longest-first order
      if (k >= n_items) break;
      int c = 0;
      while (k >= ch.items_before[c + 1]) ++c;
      // inside chunk c: the (kl / H_kv)-th tile from the end, KV head kl % H_kv
      const int kl = k - ch.items_before[c];
      const int ntiles = (ch.T[c] + TP - 1) / TP;
      const int w = (kl % H_kv) * ntiles + kl / H_kv;
      const int64_t rows = static_cast<int64_t>(ch.row0[c]) * H_q * D;
      if (r > 0) __syncthreads();  // the previous item's output staging is read
      prefill_tile<E, D, G, BS>(w, lds, pool_k, pool_v, layer_off, head_stride, pq + rows, pout + rows,
                                ptables + static_cast<int64_t>(ch.table_row[c]) * pt_stride, ch.T[c], H_q,
                                ch.ctx_before[c], scale_log2, 0, INT32_MAX, nullptr, nullptr, INT32_MAX);
    }
    return;
  }
  // decode workgroups in the decode kernel's order: kv head fastest, then
  // the partition slot (rotated as there by the sequence index's low bits),
  // then the sequence
  const int j = id - n_pre;
  const int g = j % H_kv;
  const int rest = j / H_kv;
  // the decode kernel's unsplit decision and order, over the decode half's
  // B rows
  const int B = static_cast<int>((gridDim.x - n_pre) / (H_kv * num_parts));
  if (decode_unsplit(context_lens, B, BS, H_kv, unsplit_cus)) {
    if (rest >= B) return;
    decode_body<E, D, G, BS, false>(kPrefillWaves, g, 0, H_kv, rest, reinterpret_cast<float*>(&lds[0][0]), pool_k,
                                    pool_v, layer_off, head_stride, dq, dout, block_tables, max_blocks, context_lens,
                                    scale_log2, H_q, max_blocks, 1, ws_ml, ws_acc, nullptr, nullptr, nullptr);
    return;
  }
  const int b = rest / num_parts;
  int part = rest % num_parts;
  if (num_parts >= 4) {
    part += b & 3;
    if (part >= num_parts) part -= num_parts;
  }
  decode_body<E, D, G, BS, false>(kPrefillWaves, g, part, H_kv, b, reinterpret_cast<float*>(&lds[0][0]),
                                  pool_k, pool_v, layer_off, head_stride, dq, dout, block_tables, max_blocks,
                                  context_lens, scale_log2, H_q, blocks_per_part, num_parts, ws_ml, ws_acc, nullptr,
                                  nullptr, nullptr);
}

struct MixedLaunch {
  int64_t layer_off, head_stride;
  float scale_log2;
  const void* dq;
  void* dout;
  const int32_t* bt;
  int32_t max_blocks;
  const int32_t* ctx;
  int32_t B, H_q;
  DecodePlan pl;
  Workspace ws;
  const void* pq;
  void* pout;
  const int32_t* ptables;
  int32_t pt_stride, n_pre;
  ChunkList ch;
};

using MixedFn = void (*)(const pa_kv_pool*, const MixedLaunch&, hipStream_t);

template <typename E, int D, int G, int BS>
static void launch_mixed(const pa_kv_pool* pool, const MixedLaunch& m, hipStream_t stream) {
  const int64_t n_dec = static_cast<int64_t>(pool->num_kv_heads) * m.pl.num_parts * m.B;
  const dim3 grid(static_cast<uint32_t>(m.n_pre + n_dec));
  hipLaunchKernelGGL((mixed_kernel<E, D, G, BS>), grid, dim3(kPrefillThreads), 0, stream, static_cast<char*>(pool->k),
                     static_cast<char*>(pool->v), m.layer_off, m.head_stride, pool->num_kv_heads, m.H_q, m.scale_log2,
                     static_cast<const char*>(m.dq), m.dout, m.bt, m.max_blocks, m.ctx, m.pl.blocks_per_part,
                     m.pl.num_parts, m.pl.unsplit_cus, m.ws.ml, m.ws.acc, static_cast<const uint16_t*>(m.pq),
                     static_cast<uint16_t*>(m.pout), m.ptables, m.pt_stride, m.n_pre, m.ch);
}

template <typename E, int D, int G>
static MixedFn mixed_bs(int bs) {
  switch (bs) {
    case 8: return &launch_mixed<E, D, G, 8>;
    case 16: return &launch_mixed<E, D, G, 16>;
    case 32: return &launch_mixed<E, D, G, 32>;
  }
  return nullptr;
}
template <typename E, int D>
static MixedFn mixed_g(int G, int bs) {
  switch (G) {
    case 1: return mixed_bs<E, D, 1>(bs);
    case 2: return mixed_bs<E, D, 2>(bs);
    case 4: return mixed_bs<E, D, 4>(bs);
    case 8: return mixed_bs<E, D, 8>(bs);
  }
  return nullptr;
}
template <typename E>
static MixedFn mixed_d(int D, int G, int bs) {
  switch (D) {
    case 64: return mixed_g<E, 64>(G, bs);
    case 128: return mixed_g<E, 128>(G, bs);
  }
  return nullptr;
}

// 64-key steps of all the chunks' items.
static double chunk_steps(const pa_kv_pool* pool, const ChunkList& ch, int G) {
  const int TP = kRowsPerWave * kPrefillWaves / G;
  double steps = 0.0;
  for (int c = 0; c < ch.n; ++c) {
    const int ntiles = static_cast<int>(ceil_div(ch.T[c], TP));
    for (int i = 0; i < ntiles; ++i) {
      const int64_t kmax = static_cast<int64_t>(ch.ctx_before[c]) +
                           std::min<int64_t>(static_cast<int64_t>(i + 1) * TP, ch.T[c]);
      steps += static_cast<double>(ceil_div(kmax, kKeysPerStep));
    }
  }
  return steps * pool->num_kv_heads;
}

// Prefill workgroups when the caller leaves the choice to the library: enough
// that the chunks end a little before the decode half would on its own (the
// margin, 1.25x, is where sweeps of the 63-sequence decode with one 1,024-row
// chunk and with four 256-row chunks bottom out: one box, two alternations,
// 782-785 us at n = 56 for the one chunk, 766-776 us at n = 40-48 for the
// four, against 809-822 and 787-789 us at n = 64; the margin gives 56 and
// 48).  Since the decode runs such batches unsplit, its workgroups
// are long (a 32k context is one workgroup per KV head), and leaving it more
// CUs pays more than the chunks finishing early.
// Estimates: a 64-key step of one 256-row item takes ~2 us at head_dim 128
// (less at 64); the decode streams half of B * max_ctx tokens per KV head at
// ~5 TB/s.  Rounded up to a multiple of 8 (whole rounds per XCD), at most
// one item per workgroup and one workgroup per CU.
static int default_prefill_wgs(const pa_kv_pool* pool, int B, int max_ctx, const ChunkList& ch, int G) {
  const int n_items = ch.items_before[ch.n];
  const double prefill_cu_us = chunk_steps(pool, ch, G) * 2.0 * pool->head_dim / 128.0;
  const int elem = pool->dtype == PA_F32 ? 4 : 2;
  const double decode_us = static_cast<double>(B) * pool->num_kv_heads * 0.5 * max_ctx * 2.0 * pool->head_dim * elem /
                           5.0e6;
  const int cap = std::min(n_items, device_cus());
  if (decode_us <= 0.0) return cap;
  int n = static_cast<int>(std::ceil(1.25 * prefill_cu_us / decode_us));
  n = static_cast<int>(ceil_div(std::max(n, 8), 8) * 8);
  return std::min(n, cap);
}

}  // namespace pa

extern "C" int pa_mixed_batch(const pa_kv_pool* pool, int32_t layer, void* dec_out, const void* dec_q, int32_t B,
                              int32_t H_q, const int32_t* block_tables, int32_t max_blocks,
                              const int32_t* context_lens, int32_t max_ctx, void* pf_out, const void* pf_q,
                              const pa_chunk* chunks, int32_t n_chunks, const int32_t* pf_tables,
                              int32_t pf_max_blocks, float scale, int32_t prefill_workgroups, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  using namespace pa;
  const std::string w("pa_mixed_batch");
  if (int e = validate_decode(w, pool, layer, dec_out, dec_q, B, H_q, block_tables, max_blocks, context_lens,
                              max_ctx))
    return e;
  if (n_chunks < 0 || n_chunks > kMaxChunks)
    return fail(PA_EINVAL, w + ": n_chunks must be in [0, " + std::to_string(kMaxChunks) + "]");
  if (n_chunks > 0 && !chunks) return fail(PA_EINVAL, w + ": NULL chunks");
  if (pf_max_blocks < 0) return fail(PA_EINVAL, w + ": negative pf_max_blocks");
  if (prefill_workgroups < 0) return fail(PA_EINVAL, w + ": negative prefill_workgroups");
  // Chunks packed in order in pf_q / pf_out; chunk c's table is row c of
  // pf_tables.  Each is checked as a pa_prefill_chunk call would be.
  int64_t rows = 0;
  int order[kMaxChunks];
  int live = 0;
  for (int c = 0; c < n_chunks; ++c) {
    const pa_chunk& k = chunks[c];
    const int64_t off = rows * (H_q > 0 ? H_q : 0) * pool->head_dim * 2;
    if (int e = validate_prefill(w + " chunk " + std::to_string(c), pool, layer,
                                 pf_out ? static_cast<char*>(pf_out) + off : nullptr,
                                 pf_q ? static_cast<const char*>(pf_q) + off : nullptr, k.T, H_q,
                                 pf_tables ? pf_tables + static_cast<int64_t>(c) * pf_max_blocks : nullptr,
                                 pf_max_blocks, k.ctx_before))
      return e;
    if (k.T > 0) order[live++] = c;
    rows += k.T;
  }
  if (rows > INT32_MAX) return fail(PA_EINVAL, w + ": too many chunk rows");
  if (B == 0 && live == 0) return PA_OK;
  const int G = H_q / pool->num_kv_heads;
  MixedFn fn = nullptr;
  if (pool->dtype == PA_BF16) fn = mixed_d<BF16>(pool->head_dim, G, pool->block_size);
  if (pool->dtype == PA_F16) fn = mixed_d<F16>(pool->head_dim, G, pool->block_size);
  if (!fn) return fail(PA_ENOTSUP, w + ": needs a bf16/f16 pool, head_dim 64/128, block 8/16/32, H_q/H_kv in {1,2,4,8}");

  MixedLaunch m{};
  m.head_stride = static_cast<int64_t>(pool->num_blocks) * pool->block_size * pool->head_dim * 2;
  m.layer_off = static_cast<int64_t>(layer) * pool->num_kv_heads * m.head_stride;
  m.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  m.dq = dec_q, m.dout = dec_out, m.bt = block_tables, m.max_blocks = max_blocks, m.ctx = context_lens;
  m.B = B, m.H_q = H_q;
  m.pl = DecodePlan{8, 1, 0};
  if (B > 0) {
    m.pl = plan_decode(B, pool->num_kv_heads, G, pool->block_size, max_ctx);
    m.pl.waves = 8;  // the mixed kernel's workgroups are 8 waves
    if (int e = decode_workspace_check(w, m.pl, pool, B, H_q, workspace, workspace_bytes, &m.ws)) return e;
  }
  // Item order: the chunk whose last row sees the most keys first.
  std::stable_sort(order, order + live, [&](int a, int b) {
    return static_cast<int64_t>(chunks[a].ctx_before) + chunks[a].T >
           static_cast<int64_t>(chunks[b].ctx_before) + chunks[b].T;
  });
  const int TP = kRowsPerWave * kPrefillWaves / G;
  int64_t row0[kMaxChunks];
  for (int c = 0, r = 0; c < n_chunks; r += chunks[c].T, ++c) row0[c] = r;
  m.ch.n = live;
  m.ch.items_before[0] = 0;
  for (int i = 0; i < live; ++i) {
    const int c = order[i];
    m.ch.T[i] = chunks[c].T;
    m.ch.ctx_before[i] = chunks[c].ctx_before;
    m.ch.row0[i] = static_cast<int32_t>(row0[c]);
    m.ch.table_row[i] = c;
    m.ch.items_before[i + 1] =
        m.ch.items_before[i] + static_cast<int32_t>(ceil_div(chunks[c].T, TP) * pool->num_kv_heads);
  }
  m.pq = pf_q, m.pout = pf_out, m.ptables = pf_tables, m.pt_stride = pf_max_blocks;
  m.n_pre = 0;
  if (live > 0) {
    const int64_t n_items = m.ch.items_before[live];
    const int64_t n = prefill_workgroups > 0 ? prefill_workgroups : default_prefill_wgs(pool, B, max_ctx, m.ch, G);
    m.n_pre = static_cast<int32_t>(std::min<int64_t>(n, n_items));
  }
  const int64_t n_dec = static_cast<int64_t>(pool->num_kv_heads) * m.pl.num_parts * B;
  if (m.n_pre + n_dec > INT32_MAX) return fail(PA_EINVAL, w + ": grid too large");
  if (validate_on()) {
    if (B > 0)
      if (int e = check_decode_indices(w, pool, B, block_tables, max_blocks, context_lens, max_ctx, nullptr, stream))
        return e;
    for (int i = 0; i < live; ++i) {
      const int c = order[i];
      if (int e = check_prefill_indices(w, pool, pf_tables + static_cast<int64_t>(c) * pf_max_blocks, pf_max_blocks,
                                        chunks[c].T, chunks[c].ctx_before, stream))
        return e;
    }
  }
  fn(pool, m, stream);
  if (B > 0 && m.pl.num_parts > 1)
    launch_decode_merge(pool->dtype, pool->head_dim, dec_out, m.ws, context_lens, B, H_q, pool->num_kv_heads, m.pl,
                        pool->block_size,
                        stream);
  return check_launch("pa_mixed_batch");
}
