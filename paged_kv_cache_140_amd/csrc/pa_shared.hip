// Decode attention of a batch whose sequences share prefixes, reading every
// shared block once for all of its sharers.
//
// What it computes: exactly what pa_decode computes -- each sequence's
// newest query reads all of its visible K/V through its block table
// ([icarus] "PagedAttention", icarus.shaojiemike.top, sections "Block Table
// 如何工作" and "不会降低单请求的理论读取量").  Parallel sampling, beam search
// and common prompt prefixes leave several sequences whose tables start
// with the same physical blocks, shared by reference count ([icarus] "支持块
// 级共享"; [ttlab] "llm-kv-cache-02-serving-engine-kv", section "블록을 함께
// 쓰기").  A plain decode reads such a block once per sharer; here it is read
// once per step for all of them.
//
// How: the caller names groups of consecutive batch rows and how many
// leading blocks each group's rows share.
//  * prefix pass: for a group of n rows the shared keys [0, shared_blocks *
//    block_size) are the same for all n * G query rows of a KV head, so
//    S = Q K^T and O = P V over them are dense contractions.  They run on
//    the matrix cores through the prefill tile (no causal mask, all rows see
//    every shared key), cut into key splits that write (m, l, o) partials.
//  * suffix pass: every row's remaining blocks through the decode body,
//    which writes (m, l, acc) partials per partition.
//  * both passes are one launch, prefix workgroups first; a merge launch
//    combines each row's prefix and suffix partials into its output.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <string>
#include <vector>

#include "pa_decode_dev.h"
#include "pa_prefill_dev.h"

namespace pa {

constexpr int kMaxGroups = 64;

// The groups of a launch (those with shared blocks), in the kernel arguments.
struct GroupList {
  int32_t n;
  int32_t first_row[kMaxGroups];
  int32_t n_rows[kMaxGroups];
  int32_t shared_blocks[kMaxGroups];
  int32_t splits[kMaxGroups];          // key splits of the group's prefix
  int32_t steps_per_split[kMaxGroups];  // 64-key steps per split
  int32_t pre_before[kMaxGroups + 1];  // prefix workgroups before group c
  int64_t row_off[kMaxGroups];         // first partial row of group c ([split][row][head] rows)
};

template <typename E, int D, int G, int BS>
__global__ void __launch_bounds__(kPrefillThreads)
    shared_decode_kernel(char* __restrict__ pool_k, char* __restrict__ pool_v, int64_t layer_off,
                         int64_t head_stride, int32_t H_kv, int32_t H_q, float scale_log2, const char* __restrict__ q,
                         const int32_t* __restrict__ block_tables, int32_t max_blocks,
                         const int32_t* __restrict__ context_lens, int32_t blocks_per_part, int32_t num_parts,
                         float* __restrict__ ws_ml, float* __restrict__ ws_acc, float* __restrict__ pre_o,
                         float* __restrict__ pre_ml, int32_t n_pre, GroupList gl) {
  static_assert(8 * G * (D + 2) * sizeof(float) <= sizeof(PrefillLds<D>), "decode merge fits the prefill LDS");
  __shared__ __attribute__((aligned(1024))) PrefillLds<D> lds;
  const int id = blockIdx.x;
  if (id < n_pre) {
    // Prefix: group c, (split, item) with the items of one split adjacent.
    int c = 0;
    while (id >= gl.pre_before[c + 1]) ++c;
    constexpr int TP = kRowsPerWave * kPrefillWaves / G;
    const int n = gl.n_rows[c];
    const int items = (n + TP - 1) / TP * H_kv;
    const int local = id - gl.pre_before[c];
    const int split = local / items;
    const int sps = gl.steps_per_split[c];
    const int key_end = gl.shared_blocks[c] * BS;
    const int64_t roff = gl.row_off[c] + static_cast<int64_t>(split) * n * H_q;
    prefill_tile<E, D, G, BS>(local % items, lds, pool_k, pool_v, layer_off, head_stride,
                              reinterpret_cast<const uint16_t*>(q) + static_cast<int64_t>(gl.first_row[c]) * H_q * D,
                              nullptr, block_tables + static_cast<int64_t>(gl.first_row[c]) * max_blocks, n, H_q,
                              key_end, scale_log2, split * sps, (split + 1) * sps, pre_o + roff * D,
                              pre_ml + roff * 2, key_end);
    return;
  }
  // Suffix: the decode kernel's order (kv head fastest, then the rotated
  // partition slot, then the sequence), past the row's shared blocks.
  const int j = id - n_pre;
  const int g = j % H_kv;
  const int rest = j / H_kv;
  const int b = rest / num_parts;
  int part = rest % num_parts;
  if (num_parts >= 4) {
    part += b & 3;
    if (part >= num_parts) part -= num_parts;
  }
  int skip = 0;
  for (int c = 0; c < gl.n; ++c)
    if (b >= gl.first_row[c] && b < gl.first_row[c] + gl.n_rows[c]) skip = gl.shared_blocks[c];
  decode_body<E, D, G, BS, false, true>(kPrefillWaves, g, part, H_kv, b, reinterpret_cast<float*>(&lds[0][0]), pool_k,
                                        pool_v, layer_off, head_stride, q, nullptr, block_tables, max_blocks,
                                        context_lens, scale_log2, H_q, blocks_per_part, num_parts, ws_ml, ws_acc,
                                        nullptr, nullptr, nullptr, skip);
}

// Combines each (sequence, query head)'s partials: the prefix splits of its
// group (if any) and the suffix partitions that hold some of its blocks:
// out = sum_k o_k 2^(m_k - M) / sum_k l_k 2^(m_k - M), M = max_k m_k.  Every
// load is issued before any result is used -- each thread's first kPre
// partial outputs and one partial's (m, l) -- so the merge waits for one
// memory round trip; the weights go through LDS.
template <typename E, int D>
__global__ void __launch_bounds__(D)
    shared_merge_kernel(void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
                        const float* __restrict__ pre_o, const float* __restrict__ pre_ml,
                        const int32_t* __restrict__ context_lens, int32_t H_q, int32_t num_parts,
                        int32_t blocks_per_part, int32_t bs, GroupList gl) {
  extern __shared__ float wt[];  // [max splits + num_parts] weights
  __shared__ float red[2];
  const int64_t bh = blockIdx.x;
  const int b = static_cast<int>(bh / H_q);
  const int hd = static_cast<int>(bh % H_q);
  const int e = threadIdx.x;
  int c = -1;
  for (int k = 0; k < gl.n; ++k)
    if (b >= gl.first_row[k] && b < gl.first_row[k] + gl.n_rows[k]) c = k;
  const int skip = c >= 0 ? gl.shared_blocks[c] : 0;
  const int ns = c >= 0 ? gl.splits[c] : 0;
  const int nblk = (context_lens[b] + bs - 1) / bs;
  const int np = max(0, min(num_parts, (nblk - skip + blocks_per_part - 1) / blocks_per_part));
  const int nk = ns + np;
  // partial k: prefix split k (k < ns) or suffix partition k - ns
  const int64_t prow0 = c >= 0 ? gl.row_off[c] + static_cast<int64_t>(b - gl.first_row[c]) * H_q + hd : 0;
  const int64_t pstride = c >= 0 ? static_cast<int64_t>(gl.n_rows[c]) * H_q : 0;  // rows per split
  auto row_of = [&](int k) { return k < ns ? prow0 + k * pstride : bh * num_parts + (k - ns); };
  auto o_of = [&](int k) { return k < ns ? pre_o[row_of(k) * D + e] : ws_acc[row_of(k) * D + e]; };
  constexpr int kPre = 16;
  float pre[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) pre[i] = i < nk ? o_of(i) : 0.0f;
  float2 ml = make_float2(kNegInf, 0.0f);
  if (e < nk) {
    const float* src = e < ns ? pre_ml : ws_ml;
    ml = *reinterpret_cast<const float2*>(src + 2 * row_of(e));
  }
  float mx = ml.x;
  for (int k = e + D; k < nk; k += D) mx = fmaxf(mx, (k < ns ? pre_ml : ws_ml)[2 * row_of(k)]);
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((e & 63) == 0) red[e >> 6] = mx;
  __syncthreads();
  mx = D > 64 ? fmaxf(red[0], red[1]) : red[0];
  const float ms = (mx == kNegInf) ? 0.0f : mx;
  float lsum = 0.0f;
  if (e < nk) {
    const float w = exp2_fast(ml.x - ms);
    wt[e] = w;
    lsum = ml.y * w;
  }
  for (int k = e + D; k < nk; k += D) {
    const float* src = (k < ns ? pre_ml : ws_ml) + 2 * row_of(k);
    const float w = exp2_fast(src[0] - ms);
    wt[k] = w;
    lsum += src[1] * w;
  }
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);
  __syncthreads();
  if ((e & 63) == 0) red[e >> 6] = lsum;
  __syncthreads();
  const float lt = D > 64 ? red[0] + red[1] : red[0];
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int i = 0; i < kPre; i += 2) {
    if (i < nk) a0 += pre[i] * wt[i];
    if (i + 1 < nk) a1 += pre[i + 1] * wt[i + 1];
  }
  for (int k = kPre; k < nk; ++k) a0 += o_of(k) * wt[k];
  store_elem(E{}, out, bh * D + e, lt > 0.0f ? (a0 + a1) / lt : 0.0f);
}

// ------------------------------------------------------------------ host

struct SharedPlan {
  DecodePlan dec;
  GroupList gl;
  int32_t n_pre;
  int64_t pre_rows;  // prefix partial rows (sum over groups of splits * n_rows * H_q)
  int32_t max_splits;
};

// Host checks of a group list and the launch plan (PA_OK or an error).
static int plan_shared(const std::string& w, const pa_kv_pool* pool, int32_t B, int32_t H_q, int32_t max_ctx,
                       int32_t max_blocks, const pa_share_group* groups, int32_t n_groups, SharedPlan* p) {
  if (n_groups < 0 || n_groups > kMaxGroups)
    return fail(PA_EINVAL, w + ": n_groups must be in [0, " + std::to_string(kMaxGroups) + "]");
  if (n_groups > 0 && !groups) return fail(PA_EINVAL, w + ": NULL groups");
  const int G = H_q / pool->num_kv_heads;
  const int bs = pool->block_size;
  std::vector<std::pair<int, int>> spans;
  for (int c = 0; c < n_groups; ++c) {
    const pa_share_group& gr = groups[c];
    if (gr.first_row < 0 || gr.n_rows < 1 || static_cast<int64_t>(gr.first_row) + gr.n_rows > B)
      return fail(PA_EINVAL, w + ": group " + std::to_string(c) + " rows outside the batch");
    if (gr.shared_blocks < 0 || gr.shared_blocks > max_blocks ||
        static_cast<int64_t>(gr.shared_blocks) * bs > max_ctx)
      return fail(PA_EINVAL, w + ": group " + std::to_string(c) + " shared_blocks out of range");
    spans.emplace_back(gr.first_row, gr.first_row + gr.n_rows);
  }
  std::sort(spans.begin(), spans.end());
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i].first < spans[i - 1].second) return fail(PA_EINVAL, w + ": groups overlap");

  p->dec = plan_decode(B, pool->num_kv_heads, G, bs, max_ctx);
  p->dec.waves = kPrefillWaves;  // the fused kernel's workgroups are 8 waves
  if (p->dec.num_parts > 65535) return fail(PA_EINVAL, w + ": too many partitions for the grid");
  // Key splits: about two workgroups per CU over all groups' prefix items,
  // at least two 64-key steps each.
  const int TP = kRowsPerWave * kPrefillWaves / G;
  int64_t item_steps = 0;
  for (int c = 0; c < n_groups; ++c) {
    const int64_t steps = ceil_div(static_cast<int64_t>(groups[c].shared_blocks) * bs, kKeysPerStep);
    item_steps += ceil_div(groups[c].n_rows, TP) * pool->num_kv_heads * steps;
  }
  const int64_t target = 2 * static_cast<int64_t>(device_cus());
  const int sps = static_cast<int>(std::max<int64_t>(2, ceil_div(item_steps, target)));
  GroupList& gl = p->gl;
  gl = GroupList{};
  gl.pre_before[0] = 0;
  int64_t pre = 0, rows = 0;
  int max_splits = 0;
  for (int c = 0; c < n_groups; ++c) {
    if (groups[c].shared_blocks == 0) continue;
    const int k = gl.n++;
    const int64_t steps = ceil_div(static_cast<int64_t>(groups[c].shared_blocks) * bs, kKeysPerStep);
    gl.first_row[k] = groups[c].first_row;
    gl.n_rows[k] = groups[c].n_rows;
    gl.shared_blocks[k] = groups[c].shared_blocks;
    gl.steps_per_split[k] = sps;
    gl.splits[k] = static_cast<int32_t>(ceil_div(steps, sps));
    gl.row_off[k] = rows;
    rows += static_cast<int64_t>(gl.splits[k]) * groups[c].n_rows * H_q;
    pre += ceil_div(groups[c].n_rows, TP) * pool->num_kv_heads * gl.splits[k];
    gl.pre_before[k + 1] = static_cast<int32_t>(std::min<int64_t>(pre, INT32_MAX));
    max_splits = std::max(max_splits, gl.splits[k]);
  }
  const int64_t n_dec = static_cast<int64_t>(pool->num_kv_heads) * p->dec.num_parts * B;
  if (pre + n_dec > INT32_MAX) return fail(PA_EINVAL, w + ": grid too large");
  p->n_pre = static_cast<int32_t>(pre);
  p->pre_rows = rows;
  p->max_splits = max_splits;
  return PA_OK;
}

static size_t shared_ws_bytes(const SharedPlan& p, int32_t B, int32_t H_q, int D) {
  return (static_cast<size_t>(p.pre_rows) + static_cast<size_t>(B) * H_q * p.dec.num_parts) * (D + 2) *
         sizeof(float);
}

using SharedFn = void (*)(const pa_kv_pool*, int32_t, void*, const void*, int32_t, int32_t, const int32_t*, int32_t,
                          const int32_t*, float, const SharedPlan&, float*, hipStream_t);

template <typename E, int D, int G, int BS>
static void launch_shared(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t B, int32_t H_q,
                          const int32_t* bt, int32_t max_blocks, const int32_t* ctx, float scale_log2,
                          const SharedPlan& p, float* ws, hipStream_t stream) {
  const int64_t head_stride = static_cast<int64_t>(pool->num_blocks) * BS * D * 2;
  const int64_t layer_off = static_cast<int64_t>(layer) * pool->num_kv_heads * head_stride;
  // Workspace: prefix o [rows][D] first (its 16-byte stores need the
  // caller's 16-byte alignment), prefix (m, l) [rows][2], then the suffix's
  // acc [B][H_q][P][D] and (m, l) [B][H_q][P][2].
  const int64_t dec_rows = static_cast<int64_t>(B) * H_q * p.dec.num_parts;
  float* pre_o = ws;
  float* pre_ml = pre_o + p.pre_rows * D;
  float* ws_acc = pre_ml + p.pre_rows * 2;
  float* ws_ml = ws_acc + dec_rows * D;
  const int64_t n_dec = static_cast<int64_t>(pool->num_kv_heads) * p.dec.num_parts * B;
  hipLaunchKernelGGL((shared_decode_kernel<E, D, G, BS>), dim3(static_cast<uint32_t>(p.n_pre + n_dec)),
                     dim3(kPrefillThreads), 0, stream, static_cast<char*>(pool->k), static_cast<char*>(pool->v),
                     layer_off, head_stride, pool->num_kv_heads, H_q, scale_log2, static_cast<const char*>(q), bt,
                     max_blocks, ctx, p.dec.blocks_per_part, p.dec.num_parts, ws_ml, ws_acc, pre_o, pre_ml, p.n_pre,
                     p.gl);
  const size_t lds = (p.max_splits + p.dec.num_parts) * sizeof(float);
  hipLaunchKernelGGL((shared_merge_kernel<E, D>), dim3(static_cast<uint32_t>(B) * H_q), dim3(D), lds, stream, out,
                     ws_ml, ws_acc, pre_o, pre_ml, ctx, H_q, p.dec.num_parts, p.dec.blocks_per_part, BS, p.gl);
}

template <typename E, int D, int G>
static SharedFn shared_bs(int bs) {
  switch (bs) {
    case 8: return &launch_shared<E, D, G, 8>;
    case 16: return &launch_shared<E, D, G, 16>;
    case 32: return &launch_shared<E, D, G, 32>;
  }
  return nullptr;
}
template <typename E, int D>
static SharedFn shared_g(int G, int bs) {
  switch (G) {
    case 1: return shared_bs<E, D, 1>(bs);
    case 2: return shared_bs<E, D, 2>(bs);
    case 4: return shared_bs<E, D, 4>(bs);
    case 8: return shared_bs<E, D, 8>(bs);
  }
  return nullptr;
}
template <typename E>
static SharedFn shared_d(int D, int G, int bs) {
  switch (D) {
    case 64: return shared_g<E, 64>(G, bs);
    case 128: return shared_g<E, 128>(G, bs);
  }
  return nullptr;
}

}  // namespace pa

extern "C" size_t pa_decode_shared_workspace_size(const pa_kv_pool* pool, int32_t B, int32_t H_q, int32_t max_ctx,
                                                  const pa_share_group* groups, int32_t n_groups) {
  using namespace pa;
  if (!pool || B <= 0 || H_q <= 0 || pool->num_kv_heads <= 0 || pool->block_size <= 0 || H_q % pool->num_kv_heads)
    return 0;
  SharedPlan p;
  const int32_t max_blocks = static_cast<int32_t>(ceil_div(std::max(max_ctx, 1), pool->block_size));
  if (plan_shared("pa_decode_shared_workspace_size", pool, B, H_q, max_ctx, max_blocks, groups, n_groups, &p))
    return 0;
  return shared_ws_bytes(p, B, H_q, pool->head_dim);
}

extern "C" int pa_decode_shared(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t B,
                                int32_t H_q, const int32_t* block_tables, int32_t max_blocks,
                                const int32_t* context_lens, int32_t max_ctx, const pa_share_group* groups,
                                int32_t n_groups, float scale, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  using namespace pa;
  const std::string w("pa_decode_shared");
  if (int e = validate_decode(w, pool, layer, out, q, B, H_q, block_tables, max_blocks, context_lens, max_ctx))
    return e;
  if (B == 0) return PA_OK;
  const int G = H_q / pool->num_kv_heads;
  SharedFn fn = nullptr;
  if (pool->dtype == PA_BF16) fn = shared_d<BF16>(pool->head_dim, G, pool->block_size);
  if (pool->dtype == PA_F16) fn = shared_d<F16>(pool->head_dim, G, pool->block_size);
  if (!fn) return fail(PA_ENOTSUP, w + ": needs a bf16/f16 pool, head_dim 64/128, block 8/16/32, H_q/H_kv in {1,2,4,8}");
  SharedPlan p;
  if (int e = plan_shared(w, pool, B, H_q, max_ctx, max_blocks, groups, n_groups, &p)) return e;
  const size_t need = shared_ws_bytes(p, B, H_q, pool->head_dim);
  if (!workspace || workspace_bytes < need)
    return fail(PA_ESPACE, w + ": workspace of " + std::to_string(need) + " bytes needed");
  if (reinterpret_cast<uintptr_t>(workspace) & 15u) return fail(PA_EINVAL, w + ": workspace must be 16-byte aligned");
  if (validate_on()) {
    if (int e = check_decode_indices(w, pool, B, block_tables, max_blocks, context_lens, max_ctx, nullptr, stream))
      return e;
    if (int e = check_share_groups(w, pool, B, block_tables, max_blocks, context_lens, groups, n_groups, stream))
      return e;
  }
  const float scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  fn(pool, layer, out, q, B, H_q, block_tables, max_blocks, context_lens, scale_log2, p, static_cast<float*>(workspace),
     stream);
  return check_launch("pa_decode_shared");
}

extern "C" int pa_share_groups(const int32_t* block_tables, int32_t B, int32_t max_blocks,
                               const int32_t* context_lens, int32_t block_size, int32_t min_rows, int32_t min_blocks,
                               pa_share_group* out, int32_t cap, int32_t* n_out) {
  using namespace pa;
  if (B < 0 || max_blocks < 0 || block_size <= 0 || min_rows < 2 || min_blocks < 1 || cap < 0 || !n_out ||
      (B > 0 && (!block_tables || !context_lens)) || (cap > 0 && !out))
    return fail(PA_EINVAL, "pa_share_groups: bad argument");
  // Full blocks of row r that its context covers (padding never counts).
  auto full = [&](int r) {
    return std::min<int64_t>(max_blocks, std::max(0, context_lens[r]) / block_size);
  };
  int n = 0;
  int i = 0;
  while (i < B) {
    const int32_t* ti = block_tables + static_cast<int64_t>(i) * max_blocks;
    int64_t k = full(i);
    int j = i + 1;
    // Greedy: extend the run while its rows keep >= min_blocks common
    // leading blocks.
    while (j < B) {
      const int32_t* tj = block_tables + static_cast<int64_t>(j) * max_blocks;
      int64_t kk = std::min(k, full(j)), m = 0;
      while (m < kk && tj[m] == ti[m]) ++m;
      if (m < min_blocks) break;
      k = m;
      ++j;
    }
    if (j - i >= min_rows && k >= min_blocks) {
      if (n >= cap) return fail(PA_ESPACE, "pa_share_groups: more groups than cap");
      out[n++] = pa_share_group{i, j - i, static_cast<int32_t>(k)};
      i = j;
    } else {
      ++i;
    }
  }
  *n_out = n;
  return PA_OK;
}
