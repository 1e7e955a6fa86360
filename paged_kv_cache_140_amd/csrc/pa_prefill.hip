// Causal prefill chunk over paged K/V on the gfx950 matrix cores.
//
// What it computes: a long prompt is fed in chunks ([ttlab]
// "llm-kv-cache-02-serving-engine-kv", ttlab.hopto.org, section "새 문제:
// 긴 프리필이 디코드를 멈춘다"); prefill builds K/V for every prompt token and
// each prompt row attends to every earlier position and itself ([icarus]
// "PagedAttention", icarus.shaojiemike.top, section "KV Cache 为什么难管理").
// Chunk row t sits at position ctx_before + t; its keys 0 .. ctx_before + t
// are gathered through the sequence's block table ("Block Table 如何工作").
//
// How: QK^T and PV are dense contractions, so they run on bf16/f16 MFMA
// (v_mfma_f32_32x32x16_{bf16,f16}) with fp32 accumulation.
//  * workgroup = 8 waves x 32 query rows of one KV head: TP = 256/G
//    positions x the G query heads that share the KV head, so every K/V tile
//    staged in LDS serves all G heads.  Row r is (position r / G, head r % G).
//    32 rows per wave make each K/V byte read from LDS feed 32 rows.
//  * ping-pong: waves 0-3 and 4-7 run the same sequence of MFMA units (QK of
//    the next step + PV of this one) and softmax units one phase apart, so
//    on every SIMD one wave keeps the matrix core busy while the other works
//    on the vector ALU.
//  * keys advance 64 at a time.  K and V tiles go from HBM straight into
//    double-buffered LDS (global_load_lds_dwordx4), K one step ahead of V,
//    in a layout that keeps MFMA operand reads and transposing reads free of
//    bank conflicts.  The block id of every load is wave-uniform and read
//    with a scalar load.
//  * S^T = K Q^T is computed (keys on the MFMA row axis), so the fp32 result
//    a lane holds -- 16 keys of one query row per 32x32 tile -- is, after the
//    softmax, exactly its B operand of O^T += V^T P^T: P never leaves
//    registers.  The V^T operand comes from two ds_read_b64_tr_b16 reads.
//  * online softmax in the log2 domain with the scale folded into the
//    exponent; the running output is rescaled only when a row's maximum
//    grows, and the causal mask is applied only in the last steps, whose keys
//    can pass a row's position.
//  * the output is transposed through LDS and written as whole rows.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "pa_prefill_dev.h"

namespace pa {

template <typename E, int D, int G, int BS>
__global__ void __launch_bounds__(kPrefillThreads)
    prefill_chunk_kernel(const char* __restrict__ pool_k, const char* __restrict__ pool_v, int64_t layer_off,
                         int64_t head_stride, const uint16_t* __restrict__ q, uint16_t* __restrict__ out,
                         const int32_t* __restrict__ table, int32_t T, int32_t H_q, int32_t ctx_before,
                         float scale_log2, int32_t num_splits, int32_t steps_per_split, int32_t xcd_order,
                         float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  __shared__ __attribute__((aligned(1024))) PrefillLds<D> lds;
  // One (work item, key split) per workgroup; gridDim.x = ntiles * H_kv *
  // num_splits.  By default consecutive ids take the items of one split, so
  // the tiles of one KV head, which read the same keys, share an XCD's L2.
  // With xcd_order (a split whose partials fit the L2s) the KV head is
  // fastest: head g's tiles and splits run on XCD g mod 8 (with H_kv a
  // multiple of 8), where the merge takes head g's rows and finds their
  // partials in that XCD's L2.
  const int items = gridDim.x / num_splits;
  int w, split;
  if (xcd_order) {
    constexpr int TP = kRowsPerWave * kPrefillWaves / G;
    const int ntiles = (T + TP - 1) / TP;
    const int H_kv = items / ntiles;
    const int L = blockIdx.x;
    const int rest = L / H_kv;
    w = (L % H_kv) * ntiles + rest % ntiles;
    split = rest / ntiles;
  } else {
    const int wl = xcd_contiguous(blockIdx.x, gridDim.x);
    w = wl % items;
    split = wl / items;
  }
  float* wo = nullptr;
  float* wml = nullptr;
  if (num_splits > 1) {
    wo = ws_o + static_cast<int64_t>(split) * T * H_q * D;
    wml = ws_ml + static_cast<int64_t>(split) * T * H_q * 2;
  }
  prefill_tile<E, D, G, BS>(w % items, lds, pool_k, pool_v, layer_off, head_stride, q, out, table, T, H_q,
                            ctx_before, scale_log2, split * steps_per_split, (split + 1) * steps_per_split, wo, wml,
                            INT32_MAX);
}

// Combines the key splits of each chunk row (position, query head):
// out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), M = max_s m_s, over
// the splits that hold some of the keys of the row's position tile.  The
// splits' weights are computed once, in LDS; each thread sums its dimension
// over the splits, the first 16 of them loaded before anything waits.
template <typename E, int D>
__global__ void __launch_bounds__(D)
    prefill_merge_kernel(void* __restrict__ out, const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                         int32_t T, int32_t H_q, int32_t G, int32_t ctx_before, int32_t num_splits,
                         int32_t steps_per_split, int32_t xcd_order) {
  extern __shared__ float wt[];  // [num_splits] weights, then the total weight
  // pos * H_q + head (with xcd_order: KV head g's rows on XCD g mod 8)
  const int64_t row = xcd_order ? merge_row(blockIdx.x, H_q, H_q / G) : blockIdx.x;
  const int pos = static_cast<int>(row / H_q);
  const int e = threadIdx.x;
  const int TP = kRowsPerWave * kPrefillWaves / G;
  const int t_last = min((pos / TP) * TP + TP, T) - 1;
  const int tile_steps = (ctx_before + t_last + 1 + kKeysPerStep - 1) / kKeysPerStep;
  const int ns = min(num_splits, (tile_steps + steps_per_split - 1) / steps_per_split);
  const int64_t stride = static_cast<int64_t>(T) * H_q;
  // Every load is issued before any result is used: the first splits'
  // outputs (one per thread and split) and, in wave 0, the splits' (m, l),
  // so that the merge waits for one memory round trip, not three.
  constexpr int kPre = 16;
  const float* o = ws_o + row * D + e;
  const int64_t so = stride * D;
  float pre[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) pre[i] = i < ns ? o[i * so] : 0.0f;
  if (e < 64) {
    // wave 0: the splits' (m, l), one split per lane (64 at a time), reduced by shuffles
    float2 ml[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int sp = e + 64 * r;
      ml[r] = sp < ns ? *reinterpret_cast<const float2*>(ws_ml + 2 * (sp * stride + row)) : make_float2(-INFINITY, 0.0f);
    }
    float mx = fmaxf(ml[0].x, ml[1].x);
    for (int sp = e + 128; sp < ns; sp += 64) mx = fmaxf(mx, ws_ml[2 * (sp * stride + row)]);
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float ms = mx == -INFINITY ? 0.0f : mx;
    float lt = 0.0f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int sp = e + 64 * r;
      if (sp < ns) {
        const float w = __builtin_amdgcn_exp2f(ml[r].x - ms);
        wt[sp] = w;
        lt += ml[r].y * w;
      }
    }
    for (int sp = e + 128; sp < ns; sp += 64) {
      const float2 m2 = *reinterpret_cast<const float2*>(ws_ml + 2 * (sp * stride + row));
      const float w = __builtin_amdgcn_exp2f(m2.x - ms);
      wt[sp] = w;
      lt += m2.y * w;
    }
    for (int off = 32; off > 0; off >>= 1) lt += __shfl_xor(lt, off);
    if (e == 0) wt[num_splits] = lt;
  }
  __syncthreads();
  float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
  for (int i = 0; i < kPre; i += 4) {
    if (i < ns) a0 += pre[i] * wt[i];
    if (i + 1 < ns) a1 += pre[i + 1] * wt[i + 1];
    if (i + 2 < ns) a2 += pre[i + 2] * wt[i + 2];
    if (i + 3 < ns) a3 += pre[i + 3] * wt[i + 3];
  }
  int sp = kPre;
  for (; sp + 3 < ns; sp += 4) {
    a0 += o[(sp + 0) * so] * wt[sp + 0];
    a1 += o[(sp + 1) * so] * wt[sp + 1];
    a2 += o[(sp + 2) * so] * wt[sp + 2];
    a3 += o[(sp + 3) * so] * wt[sp + 3];
  }
  for (; sp < ns; ++sp) a0 += o[sp * so] * wt[sp];
  const float lt = wt[num_splits];
  store_elem(E{}, out, row * D + e, lt > 0.0f ? ((a0 + a1) + (a2 + a3)) / lt : 0.0f);
}

// Split plan of a chunk.  Few position tiles (a short chunk after a long
// context, as after a prefix-cache hit) leave most CUs idle with each
// workgroup walking every key; then the keys are cut into splits, as many
// as give every CU a workgroup but of at least four 64-key steps each: a
// workgroup's first output costs a chain of about four dependent memory
// round trips whatever its length, and every split adds its partials'
// traffic (measured on 40 rows after 2,992 tokens, 32/8 heads: 76 us
// unsplit, 15.5 us + a 4.8 us merge at 12 splits of 4 steps, 19.7 us +
// merge at 48 splits of 1 step).
struct PrefillPlan {
  int num_splits;
  int steps_per_split;
};

static PrefillPlan plan_prefill(const pa_kv_pool* pool, int32_t T, int32_t H_q, int32_t ctx_before) {
  PrefillPlan p{1, 1 << 30};
  const int G = H_q / pool->num_kv_heads;
  const int TP = kRowsPerWave * kPrefillWaves / G;
  const int64_t items = ceil_div(T, TP) * pool->num_kv_heads;
  const int64_t steps = ceil_div(static_cast<int64_t>(ctx_before) + T, kKeysPerStep);
  const int cus = device_cus();
  // Tuning override (pa_set_tuning): 1 never splits, n > 1 asks for n
  // splits whenever a split is possible.
  const int env_n = tuning(PA_TUNE_PREFILL_SPLITS);
  if (env_n == 1 || steps < 4 || (env_n == 0 && items * 2 > cus)) return p;
  int64_t n = env_n > 1 ? std::min<int64_t>(env_n, steps) : std::min<int64_t>(ceil_div(cus, items), steps / 4);
  const int64_t sps = ceil_div(steps, n);
  p.steps_per_split = static_cast<int>(sps);
  p.num_splits = static_cast<int>(ceil_div(steps, sps));
  return p;
}

static size_t prefill_ws_bytes(const PrefillPlan& p, int32_t T, int32_t H_q, int D) {
  if (p.num_splits <= 1) return 0;
  return static_cast<size_t>(p.num_splits) * T * H_q * (D + 2) * sizeof(float);
}

using PrefillFn = void (*)(const pa_kv_pool*, int32_t, void*, const void*, int32_t, int32_t, const int32_t*,
                           int32_t, float, const PrefillPlan&, float*, float*, hipStream_t);

template <typename E, int D, int G, int BS>
static void launch_prefill(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t T, int32_t H_q,
                           const int32_t* table, int32_t ctx_before, float scale_log2, const PrefillPlan& pl,
                           float* ws_o, float* ws_ml, hipStream_t stream) {
  constexpr int TP = kRowsPerWave * kPrefillWaves / G;
  const int64_t head_stride = static_cast<int64_t>(pool->num_blocks) * BS * D * 2;
  const int64_t layer_off = static_cast<int64_t>(layer) * pool->num_kv_heads * head_stride;
  dim3 grid(static_cast<uint32_t>((T + TP - 1) / TP) * pool->num_kv_heads * pl.num_splits);
  const int xcd = pl.num_splits > 1 && static_cast<int64_t>(prefill_ws_bytes(pl, T, H_q, D)) <= kMergeFromL2Bytes;
  hipLaunchKernelGGL((prefill_chunk_kernel<E, D, G, BS>), grid, dim3(kPrefillThreads), 0, stream,
                     static_cast<const char*>(pool->k), static_cast<const char*>(pool->v), layer_off, head_stride,
                     static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out), table, T, H_q, ctx_before,
                     scale_log2, pl.num_splits, pl.steps_per_split, xcd, ws_o, ws_ml);
  if (pl.num_splits > 1)
    hipLaunchKernelGGL((prefill_merge_kernel<E, D>), dim3(static_cast<uint32_t>(T) * H_q), dim3(D),
                       (pl.num_splits + 1) * sizeof(float), stream, out, ws_o, ws_ml, T, H_q, G, ctx_before,
                       pl.num_splits, pl.steps_per_split, xcd);
}

template <typename E, int D, int G>
static PrefillFn prefill_bs(int bs) {
  switch (bs) {
    case 8: return &launch_prefill<E, D, G, 8>;
    case 16: return &launch_prefill<E, D, G, 16>;
    case 32: return &launch_prefill<E, D, G, 32>;
  }
  return nullptr;
}
template <typename E, int D>
static PrefillFn prefill_g(int G, int bs) {
  switch (G) {
    case 1: return prefill_bs<E, D, 1>(bs);
    case 2: return prefill_bs<E, D, 2>(bs);
    case 4: return prefill_bs<E, D, 4>(bs);
    case 8: return prefill_bs<E, D, 8>(bs);
  }
  return nullptr;
}
template <typename E>
static PrefillFn prefill_d(int D, int G, int bs) {
  switch (D) {
    case 64: return prefill_g<E, 64>(G, bs);
    case 128: return prefill_g<E, 128>(G, bs);
  }
  return nullptr;
}

}  // namespace pa

namespace pa {
int validate_prefill(const std::string& w, const pa_kv_pool* pool, int32_t layer, void* out, const void* q,
                     int32_t T, int32_t H_q, const int32_t* block_table, int32_t nb, int32_t ctx_before) {
  if (int e = check_pool(pool, layer)) return e;
  if (T < 0 || H_q <= 0 || nb < 0 || ctx_before < 0) return fail(PA_EINVAL, w + ": negative size");
  if (T == 0) return PA_OK;
  if (!out || !q || !block_table) return fail(PA_EINVAL, w + ": NULL argument");
  if (H_q % pool->num_kv_heads) return fail(PA_EINVAL, w + ": H_q must be a multiple of num_kv_heads");
  const int64_t total = static_cast<int64_t>(ctx_before) + T;
  if (total > INT32_MAX) return fail(PA_EINVAL, w + ": ctx_before + T overflows");
  if (ceil_div(total, pool->block_size) > nb) return fail(PA_EINVAL, w + ": block table too short");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(pool->k) |
       reinterpret_cast<uintptr_t>(pool->v)) & 15u)
    return fail(PA_EINVAL, w + ": q, out and pool must be 16-byte aligned");
  if (ceil_div(T, 16) * pool->num_kv_heads > INT32_MAX) return fail(PA_EINVAL, w + ": grid too large");
  return PA_OK;
}
}  // namespace pa

extern "C" size_t pa_prefill_workspace_size(const pa_kv_pool* pool, int32_t T, int32_t H_q, int32_t ctx_before) {
  using namespace pa;
  if (!pool || T <= 0 || H_q <= 0 || ctx_before < 0 || pool->num_kv_heads <= 0 || H_q % pool->num_kv_heads) return 0;
  return prefill_ws_bytes(plan_prefill(pool, T, H_q, ctx_before), T, H_q, pool->head_dim);
}

extern "C" int pa_prefill_chunk(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t T,
                                int32_t H_q, const int32_t* block_table, int32_t nb, int32_t ctx_before, float scale,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace pa;
  if (int e = validate_prefill("pa_prefill_chunk", pool, layer, out, q, T, H_q, block_table, nb, ctx_before)) return e;
  if (T == 0) return PA_OK;
  const int G = H_q / pool->num_kv_heads;
  PrefillFn fn = nullptr;
  if (pool->dtype == PA_BF16) fn = prefill_d<BF16>(pool->head_dim, G, pool->block_size);
  if (pool->dtype == PA_F16) fn = prefill_d<F16>(pool->head_dim, G, pool->block_size);
  if (!fn) return fail(PA_ENOTSUP, "pa_prefill_chunk: needs a bf16/f16 pool, head_dim 64/128, block 8/16/32, "
                                   "H_q/H_kv in {1,2,4,8}");
  // A split needs the caller's workspace; without one the chunk runs unsplit.
  PrefillPlan pl{1, 1 << 30};
  float* ws_o = nullptr;
  float* ws_ml = nullptr;
  if (workspace) {
    pl = plan_prefill(pool, T, H_q, ctx_before);
    const size_t need = prefill_ws_bytes(pl, T, H_q, pool->head_dim);
    if (workspace_bytes < need)
      return fail(PA_ESPACE, "pa_prefill_chunk: workspace of " + std::to_string(need) + " bytes needed");
    if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 15u))
      return fail(PA_EINVAL, "pa_prefill_chunk: workspace must be 16-byte aligned");
    if (pl.num_splits > 1) {
      ws_o = static_cast<float*>(workspace);
      ws_ml = ws_o + static_cast<size_t>(pl.num_splits) * T * H_q * pool->head_dim;
    }
  }
  if (validate_on())
    if (int e = check_prefill_indices("pa_prefill_chunk", pool, block_table, nb, T, ctx_before, stream)) return e;
  const float scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  fn(pool, layer, out, q, T, H_q, block_table, ctx_before, scale_log2, pl, ws_o, ws_ml, stream);
  return check_launch("pa_prefill_chunk");
}
