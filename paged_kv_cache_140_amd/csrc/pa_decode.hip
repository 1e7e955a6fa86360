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
//  * grid (partition, kv head, sequence).  A partition is a run of blocks of
//    one sequence; one K/V read serves all G query heads of the KV head.
//  * inside a workgroup each wave takes every W-th unit of U tokens
//    (U <= block size) and keeps the next unit's K and V in flight in
//    registers while it computes on the current one.
//  * lanes split a token row into 16-byte chunks (LPT lanes per token, one
//    128-byte line per 8 lanes), so each wave load covers whole lines of one
//    block; q.k partial sums are combined across the LPT lanes by DPP.
//  * each group of LPT lanes keeps its own online-softmax state (running
//    max m, sum l, weighted V sum acc) in the log2 domain; the groups of a
//    wave are merged by cross-lane shuffles, the waves of a workgroup through
//    LDS.
//  * a sequence split over several partitions writes (m, l, acc) partials
//    to the workspace and a small merge kernel combines them.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>

#include "pa_common.h"

namespace pa {

constexpr float kNegInf = -INFINITY;

template <typename E, int D, int BS>
struct DecodeShape {
  static constexpr int S = E::bytes;
  static constexpr int VEC = 16 / S;                         // elements per lane chunk
  static constexpr int LPT = D / VEC;                        // lanes per token row
  static constexpr int TPW = 64 / LPT;                       // token rows per wave load
  static constexpr int NLD = (BS / TPW) < 4 ? (BS / TPW) : 4;  // loads per unit per side
  static constexpr int U = NLD * TPW;                        // tokens per unit
  static constexpr int UPB = BS / U;                         // units per block
  static_assert(BS % TPW == 0, "block size must hold whole wave loads");
  static_assert(BS % U == 0, "units tile a block");
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename E, int D, int G, int BS>
__global__ void __launch_bounds__(512)
    decode_split_kernel(const char* __restrict__ pool_k, const char* __restrict__ pool_v, int64_t layer_off,
                        int64_t head_stride, const char* __restrict__ q, void* __restrict__ out,
                        const int32_t* __restrict__ block_tables, int32_t max_blocks,
                        const int32_t* __restrict__ context_lens, float scale_log2, int32_t H_q,
                        int32_t blocks_per_part, int32_t num_parts, float* __restrict__ ws_ml,
                        float* __restrict__ ws_acc) {
  using Sh = DecodeShape<E, D, BS>;
  constexpr int S = Sh::S, VEC = Sh::VEC, LPT = Sh::LPT, TPW = Sh::TPW, NLD = Sh::NLD, U = Sh::U,
                UPB = Sh::UPB;
  extern __shared__ float smem[];

  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int W = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = lane / LPT;  // token row inside a wave load
  const int c = lane % LPT;  // 16-byte chunk of the row

  const int ctx = context_lens[b];
  const int nblk = (ctx + BS - 1) / BS;
  const int j0 = part * blocks_per_part;
  const int64_t head0 = static_cast<int64_t>(b) * H_q + static_cast<int64_t>(g) * G;

  if (j0 >= nblk) {
    // Nothing visible in this partition.  With a single partition that means
    // an empty sequence: its rows are zeros.  Split partitions past the end
    // are never read by the merge.
    if (num_parts == 1) {
      for (int i = threadIdx.x; i < G * D; i += blockDim.x) store_elem(E{}, out, head0 * D + i, 0.0f);
    }
    return;
  }
  const int j1 = min(j0 + blocks_per_part, nblk);

  // q of the G heads for this lane's chunk, pre-multiplied by scale*log2(e).
  float qf[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    uint4 raw = load16(q + ((head0 + h) * D + c * VEC) * S);
    widen(E{}, raw, qf[h]);
#pragma unroll
    for (int e = 0; e < VEC; ++e) qf[h][e] *= scale_log2;
  }

  float m[G], l[G], acc[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[h][e] = 0.0f;
  }

  const char* kbase = pool_k + layer_off + static_cast<int64_t>(g) * head_stride;
  const char* vbase = pool_v + layer_off + static_cast<int64_t>(g) * head_stride;
  const int32_t* btrow = block_tables + static_cast<int64_t>(b) * max_blocks;
  const int lane_off = (r * D + c * VEC) * S;  // inside a unit, for load 0

  auto load_unit = [&](int u, uint4* kr, uint4* vr) {
    const int blk = u / UPB;
    const int sub = u % UPB;
    const int64_t phys = btrow[blk];
    const int64_t off = (phys * BS + sub * U) * static_cast<int64_t>(D * S) + lane_off;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      kr[i] = load16(kbase + off + i * TPW * D * S);
      vr[i] = load16(vbase + off + i * TPW * D * S);
    }
  };

  auto process = [&](int u, const uint4* kr, const uint4* vr, bool masked) {
    const int tok0 = u * U + r;  // this lane's first token of the unit
    float s[NLD][G];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      float kf[VEC];
      widen(E{}, kr[i], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) d = fmaf(qf[h][e], kf[e], d);
        s[i][h] = group_sum<LPT>(d);
      }
      if (masked && tok0 + i * TPW >= ctx) {
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = kNegInf;
      }
    }
    float msafe[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = m[h];
#pragma unroll
      for (int i = 0; i < NLD; ++i) mx = fmaxf(mx, s[i][h]);
      msafe[h] = (mx == kNegInf) ? 0.0f : mx;
      const float alpha = exp2_fast(m[h] - msafe[h]);
      m[h] = mx;
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      float vf[VEC];
      widen(E{}, vr[i], vf);
      if (masked && tok0 + i * TPW >= ctx) {
        // unused slots may hold anything (NaN included): select, not multiply
#pragma unroll
        for (int e = 0; e < VEC; ++e) vf[e] = 0.0f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = exp2_fast(s[i][h] - msafe[h]);
        l[h] += p;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
      }
    }
  };

  const int u_end = j1 * UPB;
  int u = j0 * UPB + wave;
  uint4 kc[NLD], vc[NLD];
  if (u < u_end) load_unit(u, kc, vc);
  while (u < u_end) {
    const int un = u + W;
    uint4 kn[NLD], vn[NLD];
    if (un < u_end) load_unit(un, kn, vn);
    const bool masked = (u + 1) * U > ctx;
    if (masked)
      process(u, kc, vc, true);
    else
      process(u, kc, vc, false);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      kc[i] = kn[i];
      vc[i] = vn[i];
    }
    u = un;
  }

  // Merge the TPW row groups of this wave (lanes LPT, 2*LPT, ... apart hold
  // the same dims of different tokens).
#pragma unroll
  for (int step = LPT; step < 64; step <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], step);
      const float lo = __shfl_xor(l[h], step);
      const float mx = fmaxf(m[h], mo);
      const float ms = (mx == kNegInf) ? 0.0f : mx;
      const float a = exp2_fast(m[h] - ms);
      const float bo = exp2_fast(mo - ms);
      l[h] = l[h] * a + lo * bo;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] = acc[h][e] * a + __shfl_xor(acc[h][e], step) * bo;
      m[h] = mx;
    }
  }

  // Waves -> LDS: sm_m[W][G], sm_l[W][G], sm_acc[W][G][D].
  float* sm_m = smem;
  float* sm_l = smem + W * G;
  float* sm_acc = smem + 2 * W * G;
  if (lane < LPT) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm_acc[(wave * G + h) * D + c * VEC + e] = acc[h][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sm_m[wave * G + h] = m[h];
      sm_l[wave * G + h] = l[h];
    }
  }
  __syncthreads();

  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int h = i / D;
    const int e = i % D;
    float mx = kNegInf;
    for (int w = 0; w < W; ++w) mx = fmaxf(mx, sm_m[w * G + h]);
    const float ms = (mx == kNegInf) ? 0.0f : mx;
    float lt = 0.0f, at = 0.0f;
    for (int w = 0; w < W; ++w) {
      const float wt = exp2_fast(sm_m[w * G + h] - ms);
      lt += sm_l[w * G + h] * wt;
      at += sm_acc[(w * G + h) * D + e] * wt;
    }
    if (num_parts == 1) {
      store_elem(E{}, out, (head0 + h) * D + e, lt > 0.0f ? at / lt : 0.0f);
    } else {
      const int64_t slot = (head0 + h) * num_parts + part;
      ws_acc[slot * D + e] = at;
      if (e == 0) {
        ws_ml[2 * slot] = mx;
        ws_ml[2 * slot + 1] = lt;
      }
    }
  }
}

// Combines the partitions of each (sequence, query head):
// out = sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M), M = max_p m_p.
template <typename E, int D>
__global__ void __launch_bounds__(D)
    decode_merge_kernel(void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
                        const int32_t* __restrict__ context_lens, int32_t H_q, int32_t num_parts,
                        int32_t part_tokens) {
  const int64_t bh = blockIdx.x;
  const int b = static_cast<int>(bh / H_q);
  const int e = threadIdx.x;
  const int ctx = context_lens[b];
  const int np = min((ctx + part_tokens - 1) / part_tokens, num_parts);
  const float* ml = ws_ml + bh * num_parts * 2;
  const float* ac = ws_acc + bh * num_parts * D;
  float mx = kNegInf;
  for (int p = 0; p < np; ++p) mx = fmaxf(mx, ml[2 * p]);
  const float ms = (mx == kNegInf) ? 0.0f : mx;
  float lt = 0.0f, at = 0.0f;
  for (int p = 0; p < np; ++p) {
    const float wt = exp2_fast(ml[2 * p] - ms);
    lt += ml[2 * p + 1] * wt;
    at += ac[p * D + e] * wt;
  }
  store_elem(E{}, out, bh * D + e, lt > 0.0f ? at / lt : 0.0f);
}

// ------------------------------------------------------------------- host

struct DecodePlan {
  int waves;
  int blocks_per_part;
  int num_parts;
};

static int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  if (!s || !*s) return dflt;
  return std::atoi(s);
}

// Grid plan from host-side sizes only (context lengths stay on the device):
// aim for about 4 workgroups per CU, never fewer than ~2 blocks per wave.
static DecodePlan plan_decode(int B, int H_kv, int bs, int max_ctx) {
  // Tuning overrides, read on every call so that a process can sweep them.
  const int env_waves = env_int("PA_DECODE_WAVES", 0);
  const int env_pb = env_int("PA_DECODE_PART_BLOCKS", 0);
  DecodePlan p;
  const int64_t nblk = ceil_div(max_ctx > 0 ? max_ctx : 1, bs);
  const int64_t pairs = static_cast<int64_t>(B) * H_kv;
  p.waves = env_waves > 0 ? env_waves : 4;
  if (p.waves > 8) p.waves = 8;
  if (env_pb > 0) {
    p.blocks_per_part = env_pb;
  } else {
    const int64_t target_wgs = 1024;
    int64_t parts = ceil_div(target_wgs, pairs);
    const int64_t min_pb = 2 * p.waves;
    const int64_t max_parts = ceil_div(nblk, min_pb);
    if (parts > max_parts) parts = max_parts;
    if (parts < 1) parts = 1;
    p.blocks_per_part = static_cast<int>(ceil_div(nblk, parts));
  }
  p.num_parts = static_cast<int>(ceil_div(nblk, p.blocks_per_part));
  return p;
}

template <typename E, int D, int G, int BS>
static void launch_split(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t B, int32_t H_q,
                         const int32_t* bt, int32_t max_blocks, const int32_t* ctx, float scale_log2,
                         const DecodePlan& pl, float* ws_ml, float* ws_acc, hipStream_t stream) {
  const int64_t head_stride = static_cast<int64_t>(pool->num_blocks) * BS * D * E::bytes;
  const int64_t layer_off = static_cast<int64_t>(layer) * pool->num_kv_heads * head_stride;
  const size_t lds = static_cast<size_t>(pl.waves) * G * (D + 2) * sizeof(float);
  dim3 grid(pl.num_parts, pool->num_kv_heads, B);
  hipLaunchKernelGGL((decode_split_kernel<E, D, G, BS>), grid, dim3(64 * pl.waves), lds, stream,
                     static_cast<const char*>(pool->k), static_cast<const char*>(pool->v), layer_off, head_stride,
                     static_cast<const char*>(q), out, bt, max_blocks, ctx, scale_log2, H_q, pl.blocks_per_part,
                     pl.num_parts, ws_ml, ws_acc);
  if (pl.num_parts > 1) {
    hipLaunchKernelGGL((decode_merge_kernel<E, D>), dim3(static_cast<uint32_t>(B) * H_q), dim3(D), 0, stream, out,
                       ws_ml, ws_acc, ctx, H_q, pl.num_parts, pl.blocks_per_part * BS);
  }
}

using SplitFn = void (*)(const pa_kv_pool*, int32_t, void*, const void*, int32_t, int32_t, const int32_t*, int32_t,
                         const int32_t*, float, const DecodePlan&, float*, float*, hipStream_t);

template <typename E, int D, int G>
static SplitFn pick_bs(int bs) {
  switch (bs) {
    case 8: return &launch_split<E, D, G, 8>;
    case 16: return &launch_split<E, D, G, 16>;
    case 32: return &launch_split<E, D, G, 32>;
  }
  return nullptr;
}
template <typename E, int D>
static SplitFn pick_g(int G, int bs) {
  switch (G) {
    case 1: return pick_bs<E, D, 1>(bs);
    case 2: return pick_bs<E, D, 2>(bs);
    case 4: return pick_bs<E, D, 4>(bs);
    case 8: return pick_bs<E, D, 8>(bs);
  }
  return nullptr;
}
template <typename E>
static SplitFn pick_d(int D, int G, int bs) {
  switch (D) {
    case 64: return pick_g<E, 64>(G, bs);
    case 128: return pick_g<E, 128>(G, bs);
  }
  return nullptr;
}
static SplitFn pick(int dtype, int D, int G, int bs) {
  switch (dtype) {
    case PA_F32: return pick_d<F32>(D, G, bs);
    case PA_BF16: return pick_d<BF16>(D, G, bs);
    case PA_F16: return pick_d<F16>(D, G, bs);
  }
  return nullptr;
}

static size_t workspace_bytes_for(const DecodePlan& pl, int B, int H_q, int D) {
  if (pl.num_parts <= 1) return 0;
  return static_cast<size_t>(B) * H_q * pl.num_parts * (D + 2) * sizeof(float);
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace pa

extern "C" size_t pa_decode_workspace_size(const pa_kv_pool* pool, int32_t B, int32_t H_q, int32_t max_ctx) {
  using namespace pa;
  if (!pool || B <= 0 || H_q <= 0 || pool->block_size <= 0 || pool->num_kv_heads <= 0) return 0;
  DecodePlan pl = plan_decode(B, pool->num_kv_heads, pool->block_size, max_ctx);
  return workspace_bytes_for(pl, B, H_q, pool->head_dim);
}

extern "C" int pa_decode(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t B, int32_t H_q,
                         const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                         int32_t max_ctx, float scale, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  using namespace pa;
  if (int e = check_pool(pool, layer)) return e;
  if (B < 0 || H_q <= 0 || max_blocks < 0 || max_ctx < 0) return fail(PA_EINVAL, "pa_decode: negative size");
  if (B == 0) return PA_OK;
  if (!out || !q || !block_tables || !context_lens) return fail(PA_EINVAL, "pa_decode: NULL argument");
  if (H_q % pool->num_kv_heads) return fail(PA_EINVAL, "pa_decode: H_q must be a multiple of num_kv_heads");
  if (static_cast<int64_t>(max_blocks) * pool->block_size < max_ctx)
    return fail(PA_EINVAL, "pa_decode: max_blocks * block_size < max_ctx");
  if (!aligned16(q) || !aligned16(pool->k) || !aligned16(pool->v))
    return fail(PA_EINVAL, "pa_decode: q and pool must be 16-byte aligned");
  if (B > 65535 || pool->num_kv_heads > 65535) return fail(PA_EINVAL, "pa_decode: grid too large");
  const int G = H_q / pool->num_kv_heads;
  SplitFn fn = pick(pool->dtype, pool->head_dim, G, pool->block_size);
  if (!fn) return fail(PA_ENOTSUP, "pa_decode: (dtype, head_dim, block_size, H_q/H_kv) not compiled");
  DecodePlan pl = plan_decode(B, pool->num_kv_heads, pool->block_size, max_ctx);
  const size_t need = workspace_bytes_for(pl, B, H_q, pool->head_dim);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PA_ESPACE, "pa_decode: workspace of " + std::to_string(need) + " bytes needed");
  float* ws_ml = static_cast<float*>(workspace);
  float* ws_acc = need ? ws_ml + static_cast<size_t>(B) * H_q * pl.num_parts * 2 : nullptr;
  const float scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  fn(pool, layer, out, q, B, H_q, block_tables, max_blocks, context_lens, scale_log2, pl, ws_ml, ws_acc, stream);
  return check_launch("pa_decode");
}
