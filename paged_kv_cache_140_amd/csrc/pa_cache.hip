// Pool writes: appending new tokens' K/V into their slots, and whole-block
// copies for copy-on-write.  Both are bit copies moved in 16-byte chunks so
// that each wave touches whole 128-byte lines.
//
// Pages: [icarus] "PagedAttention" (icarus.shaojiemike.top), sections
// "Block Table 如何工作" (the new token's K/V go into the current block) and
// "支持块级共享" (copy a shared block before a sharer writes into it);
// [ttlab] "llm-kv-cache-02-serving-engine-kv", section "블록을 함께 쓰기".
#include <hip/hip_runtime.h>

#include "pa_common.h"

namespace pa {

// One thread per 16-byte chunk of one (token, kv head) row, K rows first,
// then V rows.  A negative slot leaves that token's rows untouched.
__global__ void __launch_bounds__(256) append_kernel(char* __restrict__ pool_k, char* __restrict__ pool_v,
                                                     const char* __restrict__ k_new,
                                                     const char* __restrict__ v_new,
                                                     const int32_t* __restrict__ slots, int64_t chunks_per_side,
                                                     int32_t chunks_per_row, int32_t H, int32_t bs,
                                                     int64_t layer_head0_stride, int64_t head_stride,
                                                     int64_t row_bytes) {
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= 2 * chunks_per_side) return;
  const bool is_v = i >= chunks_per_side;
  if (is_v) i -= chunks_per_side;
  const int32_t c = static_cast<int32_t>(i % chunks_per_row);
  const int64_t row = i / chunks_per_row;  // = t * H + h
  const int32_t h = static_cast<int32_t>(row % H);
  const int64_t t = row / H;
  const int32_t slot = slots[t];
  if (slot < 0) return;
  const int64_t dst = layer_head0_stride + h * head_stride + static_cast<int64_t>(slot) * row_bytes + c * 16;
  const int64_t src = row * row_bytes + c * 16;
  (void)bs;
  const char* s = is_v ? v_new : k_new;
  char* d = is_v ? pool_v : pool_k;
  *reinterpret_cast<uint4*>(d + dst) = load16(s + src);
}

// One workgroup per (pair, layer, kv head, K|V) tile; a tile is the
// contiguous block_size * head_dim run of one block.
__global__ void __launch_bounds__(256) copy_blocks_kernel(char* __restrict__ pool_k, char* __restrict__ pool_v,
                                                          const int32_t* __restrict__ pairs, int32_t LH,
                                                          int64_t head_stride, int64_t tile_bytes) {
  const int64_t w = blockIdx.x;
  const int32_t side = static_cast<int32_t>(w & 1);
  const int64_t lh = (w >> 1) % LH;  // layer * H + head
  const int64_t p = (w >> 1) / LH;
  const int32_t src = pairs[2 * p];
  const int32_t dst = pairs[2 * p + 1];
  char* base = (side ? pool_v : pool_k) + lh * head_stride;
  const char* s = base + src * tile_bytes;
  char* d = base + dst * tile_bytes;
  for (int64_t off = static_cast<int64_t>(threadIdx.x) * 16; off < tile_bytes; off += 256 * 16)
    *reinterpret_cast<uint4*>(d + off) = load16(s + off);
}

static int elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : 2; }

}  // namespace pa

extern "C" int pa_cache_append(const pa_kv_pool* pool, int32_t layer, const void* k_new, const void* v_new,
                               const int32_t* slot_mapping, int32_t T, hipStream_t stream) {
  using namespace pa;
  if (int e = check_pool(pool, layer)) return e;
  if (T < 0) return fail(PA_EINVAL, "pa_cache_append: T < 0");
  if (T == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping) return fail(PA_EINVAL, "pa_cache_append: NULL input");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(PA_EINVAL, "pa_cache_append: k_new and v_new must be 16-byte aligned");
  const int64_t row_bytes = static_cast<int64_t>(pool->head_dim) * elem_bytes(pool->dtype);
  const int32_t chunks_per_row = static_cast<int32_t>(row_bytes / 16);
  const int64_t chunks_per_side = static_cast<int64_t>(T) * pool->num_kv_heads * chunks_per_row;
  const int64_t head_stride = static_cast<int64_t>(pool->num_blocks) * pool->block_size * row_bytes;
  const int64_t layer0 = static_cast<int64_t>(layer) * pool->num_kv_heads * head_stride;
  const int64_t threads = 2 * chunks_per_side;
  const int64_t blocks = ceil_div(threads, 256);
  if (blocks > INT32_MAX) return fail(PA_EINVAL, "pa_cache_append: T too large for one launch");
  if (validate_on())
    if (int e = check_slots("pa_cache_append", pool, slot_mapping, T, stream)) return e;
  hipLaunchKernelGGL(append_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                     static_cast<char*>(pool->k), static_cast<char*>(pool->v), static_cast<const char*>(k_new),
                     static_cast<const char*>(v_new), slot_mapping, chunks_per_side, chunks_per_row,
                     pool->num_kv_heads, pool->block_size, layer0, head_stride, row_bytes);
  return check_launch("pa_cache_append");
}

extern "C" int pa_copy_blocks(const pa_kv_pool* pool, const int32_t* pairs, int32_t n, hipStream_t stream) {
  using namespace pa;
  if (int e = check_pool(pool, 0)) return e;
  if (n < 0) return fail(PA_EINVAL, "pa_copy_blocks: n < 0");
  if (n == 0) return PA_OK;
  if (!pairs) return fail(PA_EINVAL, "pa_copy_blocks: NULL pairs");
  const int64_t tile_bytes = static_cast<int64_t>(pool->block_size) * pool->head_dim * elem_bytes(pool->dtype);
  const int64_t head_stride = static_cast<int64_t>(pool->num_blocks) * tile_bytes;
  const int32_t LH = pool->num_layers * pool->num_kv_heads;
  const int64_t wgs = static_cast<int64_t>(n) * LH * 2;
  if (wgs > INT32_MAX) return fail(PA_EINVAL, "pa_copy_blocks: too many tiles for one launch");
  if (validate_on())
    if (int e = check_pairs("pa_copy_blocks", pool, pairs, n, stream)) return e;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<uint32_t>(wgs)), dim3(256), 0, stream,
                     static_cast<char*>(pool->k), static_cast<char*>(pool->v), pairs, LH, head_stride, tile_bytes);
  return check_launch("pa_copy_blocks");
}
