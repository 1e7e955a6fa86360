// Paged decode attention for gfx950.
//
// What it computes: every sequence's newest query reads all of its visible
// K/V, found through the block table that maps logical to physical blocks,
// and takes softmax(scale * q K^T) V ([icarus] "PagedAttention",
// icarus.shaojiemike.top, sections "Block Table 如何工作" and
// "不会降低单请求的理论读取量"; [ttlab] "llm-kv-cache-02-serving-engine-kv",
// section "블록과 블록 표").  Paging moves no arithmetic: the result is plain
// attention over the sequence in token order.
//
// How, on CDNA4 (bandwidth-bound: 2*G flops per K/V element read, G = query
// heads per KV head; no matrix cores):
//  * grid (kv head, partition, sequence).  A partition is a run of blocks of
//    one sequence; one K/V read serves all G query heads of the KV head.
//  * inside a workgroup each wave takes every W-th unit of U tokens
//    (U <= block size) and keeps the next unit's K and V in flight in
//    registers while it computes on the current one.  W is 8 (plan_decode).
//  * K and V are loaded non-temporal: each byte is read once per launch,
//    and the stream should not churn the L2 that every launch first reads
//    its block tables and lengths from.
//  * lanes split a token row into 16-byte chunks (LPT lanes per token, one
//    128-byte line per 8 lanes), so each wave load covers whole lines of one
//    block; q.k partial sums are combined across the LPT lanes by DPP.
//  * each group of LPT lanes keeps its own online-softmax state (running
//    max m, sum l, weighted V sum acc) in the log2 domain; the groups of a
//    wave are merged by cross-lane shuffles, the waves of a workgroup through
//    LDS.
//  * a sequence split over several partitions writes (m, l, acc) partials
//    to the workspace and a small merge kernel combines them.  The grid is
//    planned from max_ctx; the workgroups read all lengths and, when no
//    sequence is longer than a CU's share of the batch, run unsplit
//    instead (decode_unsplit) and the merge writes nothing.
//  * fused append (pa_decode_append, FUSED): the step's new token of each
//    sequence, at position ctx - 1, is written into its slot by the
//    workgroup whose partition holds that position; that workgroup's paged
//    pass stops at ctx - 1 and one wave adds the new token from the input,
//    so no read waits on the write.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "pa_decode_dev.h"

namespace pa {

template <typename E, int D, int G, int BS, int MAXT, bool FUSED>
__global__ void __launch_bounds__(MAXT)
    decode_kernel(char* __restrict__ pool_k, char* __restrict__ pool_v, int64_t layer_off, int64_t head_stride,
                  const char* __restrict__ q, void* __restrict__ out, const int32_t* __restrict__ block_tables,
                  int32_t max_blocks, const int32_t* __restrict__ context_lens, float scale_log2, int32_t H_q,
                  int32_t blocks_per_part, int32_t num_parts, int32_t unsplit_cus, int32_t waves,
                  float* __restrict__ ws_ml, float* __restrict__ ws_acc, const char* __restrict__ k_new,
                  const char* __restrict__ v_new, const int32_t* __restrict__ new_slots) {
  extern __shared__ float smem[];
  // Grid (kv head, partition slot, sequence), kv head fastest: workgroup i
  // runs on XCD i % 8, so with H_kv a multiple of 8 every XCD gets the same
  // heads of every partition of every sequence -- the same bytes.  Inside an
  // XCD the workgroups are dealt round its CUs in turn, so one partition per
  // slot would, with a partition count that is a multiple of 4, give some
  // CUs every sequence's first partition (always present) and others only
  // the late ones of long sequences; rotating the partition by the low bits
  // of the sequence index spreads them.  (Measured on 63 contexts of
  // 1k-32k: 4 / 8 / 16 partitions 1,023 / 895 / 863 us unrotated, 788 /
  // 787 / 819 us rotated.)  Fewer than 4 partitions: no rotation, no cost.
  if (decode_unsplit(context_lens, gridDim.z, BS, gridDim.x, unsplit_cus)) {
    // Unsplit: the grid's first B * H_kv workgroups, in the order an unsplit
    // grid would launch them, each decode one (sequence, KV head) whole and
    // write its output; the others exit.
    const int b = blockIdx.y + num_parts * blockIdx.z;
    if (b >= static_cast<int>(gridDim.z)) return;
    decode_body<E, D, G, BS, FUSED>(waves, blockIdx.x, 0, gridDim.x, b, smem, pool_k, pool_v, layer_off, head_stride,
                                    q, out, block_tables, max_blocks, context_lens, scale_log2, H_q, max_blocks, 1,
                                    ws_ml, ws_acc, k_new, v_new, new_slots);
    return;
  }
  int part = blockIdx.y;
  if (num_parts >= 4) {
    part += blockIdx.z & 3;
    if (part >= num_parts) part -= num_parts;
  }
  decode_body<E, D, G, BS, FUSED>(waves, blockIdx.x, part, gridDim.x, blockIdx.z, smem, pool_k, pool_v, layer_off,
                                  head_stride, q, out, block_tables, max_blocks, context_lens, scale_log2, H_q,
                                  blocks_per_part, num_parts, ws_ml, ws_acc, k_new, v_new, new_slots);
}

// pa_decode's walk without the arithmetic: the same grid, tables, unit
// order and loads, every loaded dword XORed into a per-wave checksum.
template <typename E, int D, int G, int BS, int MAXT>
__global__ void __launch_bounds__(MAXT)
    gather_kernel(char* __restrict__ pool_k, char* __restrict__ pool_v, int64_t layer_off, int64_t head_stride,
                  const int32_t* __restrict__ block_tables, int32_t max_blocks,
                  const int32_t* __restrict__ context_lens, int32_t H_q, int32_t blocks_per_part, int32_t num_parts,
                  int32_t unsplit_cus, int32_t waves, uint32_t* __restrict__ checksums) {
  extern __shared__ float smem[];
  int part = blockIdx.y;
  int b = blockIdx.z;
  int bpp = blocks_per_part;
  if (decode_unsplit(context_lens, gridDim.z, BS, gridDim.x, unsplit_cus)) {
    // the decode's unsplit walk: the first B * H_kv workgroups take partition
    // 0 of one (sequence, KV head) each, whole; the others stand for the
    // empty partitions 1 .. P-1, whose checksums are 0
    const int B = gridDim.z;
    const int rest = blockIdx.y + num_parts * blockIdx.z;
    if (rest >= B) {
      const int e = rest - B;
      if ((threadIdx.x & 63) == 0)
        checksums[((static_cast<int64_t>(e / (num_parts - 1)) * num_parts + 1 + e % (num_parts - 1)) * gridDim.x +
                   blockIdx.x) * waves + (threadIdx.x >> 6)] = 0;
      return;
    }
    b = rest;
    part = 0;
    bpp = max_blocks;
  } else if (num_parts >= 4) {
    part += blockIdx.z & 3;
    if (part >= num_parts) part -= num_parts;
  }
  decode_body<E, D, G, BS, false, false, true>(waves, blockIdx.x, part, gridDim.x, b, smem, pool_k, pool_v,
                                               layer_off, head_stride, nullptr, nullptr, block_tables, max_blocks,
                                               context_lens, 0.0f, H_q, bpp, num_parts,
                                               reinterpret_cast<float*>(checksums), nullptr, nullptr, nullptr,
                                               nullptr);
}

// Combines the partitions of each (sequence, query head):
// out = sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M), M = max_p m_p.
// The (m, l) of all partitions are staged in LDS once; each thread then sums
// its dimension over the partitions with several loads in flight.
template <typename E, int D>
__global__ void __launch_bounds__(D)
    decode_merge_kernel(void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
                        const int32_t* __restrict__ context_lens, int32_t H_q, int32_t H_kv, int32_t xcd_order,
                        int32_t num_parts, int32_t part_tokens, int32_t bs, int32_t unsplit_cus) {
  extern __shared__ float w_lds[];  // [num_parts] weights, then [1] total
  const int64_t bh = xcd_order ? merge_row(blockIdx.x, H_q, H_kv) : blockIdx.x;
  const int b = static_cast<int>(bh / H_q);
  const int e = threadIdx.x;
  if (decode_unsplit(context_lens, gridDim.x / H_q, bs, H_kv, unsplit_cus)) return;  // the decode wrote out
  const int ctx = context_lens[b];
  const int np = min((ctx + part_tokens - 1) / part_tokens, num_parts);
  const float* ml = ws_ml + bh * num_parts * 2;
  const float* ac = ws_acc + bh * num_parts * D;
  float mx = kNegInf;
  for (int p = e; p < np; p += D) mx = fmaxf(mx, ml[2 * p]);
  // block max over D threads (D = 64 or 128: one or two waves)
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  __shared__ float red[2];
  if ((e & 63) == 0) red[e >> 6] = mx;
  __syncthreads();
  mx = D > 64 ? fmaxf(red[0], red[1]) : red[0];
  const float ms = (mx == kNegInf) ? 0.0f : mx;
  float lsum = 0.0f;
  for (int p = e; p < np; p += D) {
    const float wt = exp2_fast(ml[2 * p] - ms);
    w_lds[p] = wt;
    lsum += ml[2 * p + 1] * wt;
  }
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);
  __syncthreads();
  if ((e & 63) == 0) red[e >> 6] = lsum;
  __syncthreads();
  const float lt = D > 64 ? red[0] + red[1] : red[0];
  float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
  int p = 0;
  for (; p + 3 < np; p += 4) {
    a0 += ac[(p + 0) * D + e] * w_lds[p + 0];
    a1 += ac[(p + 1) * D + e] * w_lds[p + 1];
    a2 += ac[(p + 2) * D + e] * w_lds[p + 2];
    a3 += ac[(p + 3) * D + e] * w_lds[p + 3];
  }
  for (; p < np; ++p) a0 += ac[p * D + e] * w_lds[p];
  const float at = (a0 + a1) + (a2 + a3);
  store_elem(E{}, out, bh * D + e, lt > 0.0f ? at / lt : 0.0f);
}

// ------------------------------------------------------------------- host

template <int G>
constexpr int max_threads() {
  return G <= 2 ? 1024 : 512;
}

static int max_waves_for(int G) { return (G <= 2 ? 1024 : 512) / 64; }

// Grid plan from host-side sizes and the device's CU count only (context
// lengths stay on the device).  The tuning overrides (pa_set_tuning) fix the
// wave count and the partition length.
DecodePlan plan_decode(int B, int H_kv, int G, int bs, int max_ctx) {
  const int env_waves = tuning(PA_TUNE_DECODE_WAVES);
  const int env_pb = tuning(PA_TUNE_DECODE_PART_BLOCKS);
  const int cus = device_cus();
  DecodePlan p;
  const int64_t nblk = ceil_div(max_ctx > 0 ? max_ctx : 1, bs);
  const int64_t pairs = static_cast<int64_t>(B) * H_kv;
  if (env_pb > 0) {
    p.blocks_per_part = env_pb;
  } else if (pairs >= cus && nblk <= 256) {
    // Enough (sequence, kv head) pairs to fill the chip and contexts short
    // enough that one workgroup per pair finishes in a few tens of
    // microseconds: a split would only add merge latency.
    p.blocks_per_part = static_cast<int>(nblk);
  } else {
    // Long contexts or few pairs: cut each sequence into partitions of at
    // least 64 blocks, enough that the hardware can balance ~4 per CU.
    const int64_t parts = ceil_div(4 * static_cast<int64_t>(cus), pairs);
    int64_t pb = ceil_div(nblk, parts);
    if (pb < 64) pb = 64;
    p.blocks_per_part = static_cast<int>(pb);
  }
  p.num_parts = static_cast<int>(ceil_div(nblk, p.blocks_per_part));
  // Waves per workgroup: 8 (with the K/V loads non-temporal and the
  // placeholder refills reading block 0, 8 waves against 4: the B=32 GQA
  // 16/8 step 16.0 against 16.1 us, the B=64 MHA-40 decode 104.2 against
  // 105.0 us, the split decode of 63 contexts of 1k-32k tokens 740 against
  // 797 us).
  p.waves = env_waves > 0 ? env_waves : 8;
  p.waves = p.waves > max_waves_for(G) ? max_waves_for(G) : p.waves;
  // A split planned from max_ctx alone may run unsplit on the device
  // (decode_unsplit), unless the partition length is fixed by a tuning
  // override.
  p.unsplit_cus = (p.num_parts > 1 && env_pb <= 0) ? cus : 0;
  return p;
}

size_t workspace_bytes_for(const DecodePlan& pl, int B, int H_kv, int H_q, int D) {
  if (pl.num_parts <= 1) return 0;
  (void)H_kv;
  return static_cast<size_t>(B) * H_q * pl.num_parts * (D + 2) * sizeof(float);
}

Workspace carve(void* ws, const DecodePlan& pl, int B, int H_kv, int H_q) {
  Workspace w{nullptr, nullptr};
  (void)H_kv;
  if (pl.num_parts <= 1) return w;
  w.ml = static_cast<float*>(ws);
  w.acc = w.ml + static_cast<size_t>(B) * H_q * pl.num_parts * 2;
  return w;
}

void launch_decode_merge(int dtype, int D, void* out, const Workspace& ws, const int32_t* ctx, int32_t B, int32_t H_q,
                         int32_t H_kv, const DecodePlan& pl, int bs, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(B) * H_q);
  const size_t lds = pl.num_parts * sizeof(float);
  const int pt = pl.blocks_per_part * bs;
  const int xcd = static_cast<int64_t>(B) * H_q * pl.num_parts * (D + 2) * 4 <= kMergeFromL2Bytes;
#define PA_MERGE(E_, D_) \
  hipLaunchKernelGGL((decode_merge_kernel<E_, D_>), grid, dim3(D_), lds, stream, out, ws.ml, ws.acc, ctx, H_q, \
                     H_kv, xcd, pl.num_parts, pt, bs, pl.unsplit_cus)
  if (dtype == PA_F32 && D == 64) PA_MERGE(F32, 64);
  if (dtype == PA_F32 && D == 128) PA_MERGE(F32, 128);
  if (dtype == PA_BF16 && D == 64) PA_MERGE(BF16, 64);
  if (dtype == PA_BF16 && D == 128) PA_MERGE(BF16, 128);
  if (dtype == PA_F16 && D == 64) PA_MERGE(F16, 64);
  if (dtype == PA_F16 && D == 128) PA_MERGE(F16, 128);
#undef PA_MERGE
}

// New tokens of a fused append: [B][H_kv][D] rows and their slots, or all
// NULL for a plain decode.
struct NewTokens {
  const void* k;
  const void* v;
  const int32_t* slots;
};

template <typename E, int D, int G, int BS, bool FUSED>
static void launch_decode(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t B, int32_t H_q,
                          const int32_t* bt, int32_t max_blocks, const int32_t* ctx, float scale_log2,
                          const DecodePlan& pl, const Workspace& ws, const NewTokens& nt, hipStream_t stream) {
  const int64_t head_stride = static_cast<int64_t>(pool->num_blocks) * BS * D * E::bytes;
  const int64_t layer_off = static_cast<int64_t>(layer) * pool->num_kv_heads * head_stride;
  const size_t lds = static_cast<size_t>(pl.waves) * G * (D + 2) * sizeof(float);
  dim3 grid(pool->num_kv_heads, pl.num_parts, B);
  hipLaunchKernelGGL((decode_kernel<E, D, G, BS, max_threads<G>(), FUSED>), grid, dim3(64 * pl.waves), lds, stream,
                     static_cast<char*>(pool->k), static_cast<char*>(pool->v), layer_off, head_stride,
                     static_cast<const char*>(q), out, bt, max_blocks, ctx, scale_log2, H_q, pl.blocks_per_part,
                     pl.num_parts, pl.unsplit_cus, pl.waves, ws.ml, ws.acc, static_cast<const char*>(nt.k),
                     static_cast<const char*>(nt.v), nt.slots);
  if (pl.num_parts > 1) launch_decode_merge(pool->dtype, D, out, ws, ctx, B, H_q, pool->num_kv_heads, pl, BS, stream);
}

using DecodeFn = void (*)(const pa_kv_pool*, int32_t, void*, const void*, int32_t, int32_t, const int32_t*, int32_t,
                          const int32_t*, float, const DecodePlan&, const Workspace&, const NewTokens&, hipStream_t);

template <typename E, int D, int G, int BS>
static DecodeFn pick_fused(bool fused) {
  return fused ? &launch_decode<E, D, G, BS, true> : &launch_decode<E, D, G, BS, false>;
}
template <typename E, int D, int G>
static DecodeFn pick_bs(int bs, bool fused) {
  switch (bs) {
    case 8: return pick_fused<E, D, G, 8>(fused);
    case 16: return pick_fused<E, D, G, 16>(fused);
    case 32: return pick_fused<E, D, G, 32>(fused);
  }
  return nullptr;
}
template <typename E, int D>
static DecodeFn pick_g(int G, int bs, bool fused) {
  switch (G) {
    case 1: return pick_bs<E, D, 1>(bs, fused);
    case 2: return pick_bs<E, D, 2>(bs, fused);
    case 4: return pick_bs<E, D, 4>(bs, fused);
    case 8: return pick_bs<E, D, 8>(bs, fused);
  }
  return nullptr;
}
template <typename E>
static DecodeFn pick_d(int D, int G, int bs, bool fused) {
  switch (D) {
    case 64: return pick_g<E, 64>(G, bs, fused);
    case 128: return pick_g<E, 128>(G, bs, fused);
  }
  return nullptr;
}
static DecodeFn pick(int dtype, int D, int G, int bs, bool fused) {
  switch (dtype) {
    case PA_F32: return pick_d<F32>(D, G, bs, fused);
    case PA_BF16: return pick_d<BF16>(D, G, bs, fused);
    case PA_F16: return pick_d<F16>(D, G, bs, fused);
  }
  return nullptr;
}


}  // namespace pa

extern "C" size_t pa_decode_workspace_size(const pa_kv_pool* pool, int32_t B, int32_t H_q, int32_t max_ctx) {
  using namespace pa;
  if (!pool || B <= 0 || H_q <= 0 || pool->block_size <= 0 || pool->num_kv_heads <= 0) return 0;
  if (H_q % pool->num_kv_heads) return 0;
  DecodePlan pl = plan_decode(B, pool->num_kv_heads, H_q / pool->num_kv_heads, pool->block_size, max_ctx);
  return workspace_bytes_for(pl, B, pool->num_kv_heads, H_q, pool->head_dim);
}

namespace pa {
int validate_decode(const std::string& w, const pa_kv_pool* pool, int32_t layer, void* out, const void* q,
                    int32_t B, int32_t H_q, const int32_t* block_tables, int32_t max_blocks,
                    const int32_t* context_lens, int32_t max_ctx) {
  if (int e = check_pool(pool, layer)) return e;
  if (B < 0 || H_q <= 0 || max_blocks < 0 || max_ctx < 0) return fail(PA_EINVAL, w + ": negative size");
  if (B == 0) return PA_OK;
  if (!out || !q || !block_tables || !context_lens) return fail(PA_EINVAL, w + ": NULL argument");
  if (H_q % pool->num_kv_heads) return fail(PA_EINVAL, w + ": H_q must be a multiple of num_kv_heads");
  if (static_cast<int64_t>(max_blocks) * pool->block_size < max_ctx)
    return fail(PA_EINVAL, w + ": max_blocks * block_size < max_ctx");
  if (!aligned16(q) || !aligned16(pool->k) || !aligned16(pool->v))
    return fail(PA_EINVAL, w + ": q and pool must be 16-byte aligned");
  if (B > 65535 || pool->num_kv_heads > 65535) return fail(PA_EINVAL, w + ": grid too large");
  return PA_OK;
}

int decode_workspace_check(const std::string& w, const DecodePlan& pl, const pa_kv_pool* pool, int32_t B,
                           int32_t H_q, void* workspace, size_t workspace_bytes, Workspace* ws) {
  if (pl.num_parts > 65535) return fail(PA_EINVAL, w + ": too many partitions for the grid");
  const size_t need = workspace_bytes_for(pl, B, pool->num_kv_heads, H_q, pool->head_dim);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PA_ESPACE, w + ": workspace of " + std::to_string(need) + " bytes needed");
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 3u))
    return fail(PA_EINVAL, w + ": workspace must be 4-byte aligned");
  *ws = carve(workspace, pl, B, pool->num_kv_heads, H_q);
  return PA_OK;
}

static int decode_entry(const char* who, const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t B,
                        int32_t H_q, const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                        int32_t max_ctx, float scale, void* workspace, size_t workspace_bytes, const NewTokens& nt,
                        hipStream_t stream) {
  const std::string w(who);
  if (int e = validate_decode(w, pool, layer, out, q, B, H_q, block_tables, max_blocks, context_lens, max_ctx))
    return e;
  if (B == 0) return PA_OK;
  if (nt.slots && (!aligned16(nt.k) || !aligned16(nt.v)))
    return fail(PA_EINVAL, w + ": k_new and v_new must be 16-byte aligned");
  const int G = H_q / pool->num_kv_heads;
  DecodeFn fn = pick(pool->dtype, pool->head_dim, G, pool->block_size, nt.slots != nullptr);
  if (!fn) return fail(PA_ENOTSUP, w + ": (dtype, head_dim, block_size, H_q/H_kv) not compiled");
  DecodePlan pl = plan_decode(B, pool->num_kv_heads, G, pool->block_size, max_ctx);
  Workspace ws;
  if (int e = decode_workspace_check(w, pl, pool, B, H_q, workspace, workspace_bytes, &ws)) return e;
  if (validate_on())
    if (int e = check_decode_indices(w, pool, B, block_tables, max_blocks, context_lens, max_ctx, nt.slots, stream))
      return e;
  const float scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  fn(pool, layer, out, q, B, H_q, block_tables, max_blocks, context_lens, scale_log2, pl, ws, nt, stream);
  return check_launch(who);
}
}  // namespace pa

extern "C" int pa_decode(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t B, int32_t H_q,
                         const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                         int32_t max_ctx, float scale, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  return pa::decode_entry("pa_decode", pool, layer, out, q, B, H_q, block_tables, max_blocks, context_lens, max_ctx,
                          scale, workspace, workspace_bytes, pa::NewTokens{nullptr, nullptr, nullptr}, stream);
}

extern "C" int pa_decode_append(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, const void* k_new,
                                const void* v_new, const int32_t* slot_mapping, int32_t B, int32_t H_q,
                                const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                                int32_t max_ctx, float scale, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  if (B > 0 && (!k_new || !v_new || !slot_mapping)) return pa::fail(PA_EINVAL, "pa_decode_append: NULL new token input");
  return pa::decode_entry("pa_decode_append", pool, layer, out, q, B, H_q, block_tables, max_blocks, context_lens,
                          max_ctx, scale, workspace, workspace_bytes, pa::NewTokens{k_new, v_new, slot_mapping},
                          stream);
}

// ------------------------------------------------------ gather ceiling
namespace pa {
using GatherFn = void (*)(const pa_kv_pool*, int32_t, int32_t, const int32_t*, int32_t, const int32_t*, int32_t,
                          const DecodePlan&, uint32_t*, hipStream_t);

template <typename E, int D, int G, int BS>
static void launch_gather(const pa_kv_pool* pool, int32_t layer, int32_t B, const int32_t* bt, int32_t max_blocks,
                          const int32_t* ctx, int32_t H_q, const DecodePlan& pl, uint32_t* cs, hipStream_t stream) {
  const int64_t head_stride = static_cast<int64_t>(pool->num_blocks) * BS * D * E::bytes;
  const int64_t layer_off = static_cast<int64_t>(layer) * pool->num_kv_heads * head_stride;
  const size_t lds = static_cast<size_t>(pl.waves) * G * (D + 2) * sizeof(float);
  dim3 grid(pool->num_kv_heads, pl.num_parts, B);
  hipLaunchKernelGGL((gather_kernel<E, D, G, BS, max_threads<G>()>), grid, dim3(64 * pl.waves), lds, stream,
                     static_cast<char*>(pool->k), static_cast<char*>(pool->v), layer_off, head_stride, bt, max_blocks,
                     ctx, H_q, pl.blocks_per_part, pl.num_parts, pl.unsplit_cus, pl.waves, cs);
}
template <typename E, int D, int G>
static GatherFn gather_bs(int bs) {
  switch (bs) {
    case 8: return &launch_gather<E, D, G, 8>;
    case 16: return &launch_gather<E, D, G, 16>;
    case 32: return &launch_gather<E, D, G, 32>;
  }
  return nullptr;
}
template <typename E, int D>
static GatherFn gather_g(int G, int bs) {
  switch (G) {
    case 1: return gather_bs<E, D, 1>(bs);
    case 2: return gather_bs<E, D, 2>(bs);
    case 4: return gather_bs<E, D, 4>(bs);
    case 8: return gather_bs<E, D, 8>(bs);
  }
  return nullptr;
}
static size_t gather_bytes(const DecodePlan& pl, int B, int H_kv) {
  return static_cast<size_t>(B) * pl.num_parts * H_kv * pl.waves * sizeof(uint32_t);
}
}  // namespace pa

extern "C" size_t pa_gather_checksum_size(const pa_kv_pool* pool, int32_t B, int32_t H_q, int32_t max_ctx) {
  using namespace pa;
  if (!pool || B <= 0 || H_q <= 0 || pool->num_kv_heads <= 0 || pool->block_size <= 0 || H_q % pool->num_kv_heads)
    return 0;
  const DecodePlan pl = plan_decode(B, pool->num_kv_heads, H_q / pool->num_kv_heads, pool->block_size, max_ctx);
  return gather_bytes(pl, B, pool->num_kv_heads);
}

extern "C" int pa_gather_checksum(const pa_kv_pool* pool, int32_t layer, int32_t B, int32_t H_q,
                                  const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                                  int32_t max_ctx, uint32_t* checksums, size_t checksum_bytes, hipStream_t stream) {
  using namespace pa;
  const std::string w("pa_gather_checksum");
  // validate_decode wants out and q; the walk reads neither
  if (int e = validate_decode(w, pool, layer, checksums, pool ? pool->k : nullptr, B, H_q, block_tables, max_blocks,
                              context_lens, max_ctx))
    return e;
  if (B == 0) return PA_OK;
  const int G = H_q / pool->num_kv_heads;
  GatherFn fn = nullptr;
  if (pool->dtype == PA_BF16 && pool->head_dim == 128) fn = gather_g<BF16, 128>(G, pool->block_size);
  if (pool->dtype == PA_BF16 && pool->head_dim == 64) fn = gather_g<BF16, 64>(G, pool->block_size);
  if (!fn) return fail(PA_ENOTSUP, w + ": bf16 pools only");
  const DecodePlan pl = plan_decode(B, pool->num_kv_heads, G, pool->block_size, max_ctx);
  if (pl.num_parts > 65535) return fail(PA_EINVAL, w + ": too many partitions for the grid");
  if (checksum_bytes < gather_bytes(pl, B, pool->num_kv_heads) || (reinterpret_cast<uintptr_t>(checksums) & 3u))
    return fail(PA_ESPACE, w + ": checksum buffer too small or misaligned");
  if (validate_on())
    if (int e = check_decode_indices(w, pool, B, block_tables, max_blocks, context_lens, max_ctx, nullptr, stream))
      return e;
  fn(pool, layer, B, block_tables, max_blocks, context_lens, H_q, pl, checksums, stream);
  return check_launch("pa_gather_checksum");
}

// ------------------------------------------------------ allocation-free decode
// pa_decode_noalloc keeps a split decode's partials in this file-scope array
// instead of a caller's workspace.  Each GPU the library runs on holds its
// own copy until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is only a stand-in): the device address is
// looked up once per device, with that device current, and kept.
static __device__ __align__(256) float scratch[PA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace pa {
namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];

int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_EHIP, std::string("pa_decode_noalloc: hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kScratchDevices) return fail(PA_EINVAL, "pa_decode_noalloc: device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(PA_EHIP, std::string("pa_decode_noalloc: hipGetSymbolAddress: ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}
}  // namespace
}  // namespace pa

extern "C" int pa_decode_noalloc(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t B,
                                 int32_t H_q, const int32_t* block_tables, int32_t max_blocks,
                                 const int32_t* context_lens, int32_t max_ctx, float scale, hipStream_t stream) {
  using namespace pa;
  const char* who = "pa_decode_noalloc";
  if (int e = validate_decode(who, pool, layer, out, q, B, H_q, block_tables, max_blocks, context_lens, max_ctx))
    return e;
  if (B == 0) return PA_OK;
  const int G = H_q / pool->num_kv_heads;
  const DecodePlan pl = plan_decode(B, pool->num_kv_heads, G, pool->block_size, max_ctx);
  const size_t need = workspace_bytes_for(pl, B, pool->num_kv_heads, H_q, pool->head_dim);
  if (need > PA_NOALLOC_SCRATCH_BYTES)
    return fail(PA_ESPACE, std::string(who) + ": the split needs " + std::to_string(need) +
                               " bytes of partials, more than the " + std::to_string(PA_NOALLOC_SCRATCH_BYTES) +
                               "-byte static scratch; use pa_decode with a workspace");
  void* ws = nullptr;
  if (need > 0)
    if (int e = scratch_address(&ws)) return e;
  return decode_entry(who, pool, layer, out, q, B, H_q, block_tables, max_blocks, context_lens, max_ctx, scale, ws,
                      need > 0 ? PA_NOALLOC_SCRATCH_BYTES : 0, NewTokens{nullptr, nullptr, nullptr}, stream);
}
