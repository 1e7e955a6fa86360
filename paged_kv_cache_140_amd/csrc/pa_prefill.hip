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

#include <cmath>
#include <type_traits>

#include "pa_prefill_dev.h"

namespace pa {

template <typename E, int D, int G, int BS>
__global__ void __launch_bounds__(kPrefillThreads)
    prefill_chunk_kernel(const char* __restrict__ pool_k, const char* __restrict__ pool_v, int64_t layer_off,
                         int64_t head_stride, const uint16_t* __restrict__ q, uint16_t* __restrict__ out,
                         const int32_t* __restrict__ table, int32_t T, int32_t H_q, int32_t ctx_before,
                         float scale_log2) {
  __shared__ __attribute__((aligned(1024))) PrefillLds<D> lds;
  // One work item per workgroup; gridDim.x = ntiles * H_kv.
  prefill_tile<E, D, G, BS>(xcd_contiguous(blockIdx.x, gridDim.x), lds, pool_k, pool_v, layer_off, head_stride, q,
                            out, table, T, H_q, ctx_before, scale_log2);
}

using PrefillFn = void (*)(const pa_kv_pool*, int32_t, void*, const void*, int32_t, int32_t, const int32_t*,
                           int32_t, float, hipStream_t);

template <typename E, int D, int G, int BS>
static void launch_prefill(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t T, int32_t H_q,
                           const int32_t* table, int32_t ctx_before, float scale_log2, hipStream_t stream) {
  constexpr int TP = kRowsPerWave * kPrefillWaves / G;
  const int64_t head_stride = static_cast<int64_t>(pool->num_blocks) * BS * D * 2;
  const int64_t layer_off = static_cast<int64_t>(layer) * pool->num_kv_heads * head_stride;
  dim3 grid(static_cast<uint32_t>((T + TP - 1) / TP) * pool->num_kv_heads);
  hipLaunchKernelGGL((prefill_chunk_kernel<E, D, G, BS>), grid, dim3(kPrefillThreads), 0, stream,
                     static_cast<const char*>(pool->k), static_cast<const char*>(pool->v), layer_off, head_stride,
                     static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out), table, T, H_q, ctx_before,
                     scale_log2);
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

extern "C" int pa_prefill_chunk(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t T,
                                int32_t H_q, const int32_t* block_table, int32_t nb, int32_t ctx_before, float scale,
                                hipStream_t stream) {
  using namespace pa;
  if (int e = validate_prefill("pa_prefill_chunk", pool, layer, out, q, T, H_q, block_table, nb, ctx_before)) return e;
  if (T == 0) return PA_OK;
  const int G = H_q / pool->num_kv_heads;
  PrefillFn fn = nullptr;
  if (pool->dtype == PA_BF16) fn = prefill_d<BF16>(pool->head_dim, G, pool->block_size);
  if (pool->dtype == PA_F16) fn = prefill_d<F16>(pool->head_dim, G, pool->block_size);
  if (!fn) return fail(PA_ENOTSUP, "pa_prefill_chunk: needs a bf16/f16 pool, head_dim 64/128, block 8/16/32, "
                                   "H_q/H_kv in {1,2,4,8}");
  const float scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  fn(pool, layer, out, q, T, H_q, block_table, ctx_before, scale_log2, stream);
  return check_launch("pa_prefill_chunk");
}
