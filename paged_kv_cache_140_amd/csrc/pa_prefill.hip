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
// (v_mfma_f32_16x16x32_{bf16,f16}) with fp32 accumulation.
//  * workgroup = 8 waves x 16 query rows of one KV head: TP = 128/G
//    positions x the G query heads that share the KV head, so every K/V tile
//    staged in LDS serves all G heads.  Row r is (position r / G, head r % G).
//    16 rows per wave keep the kernel near 160 VGPRs, so several workgroups
//    share a CU and hide each other's LDS and exp latency.
//  * keys advance 64 at a time.  The tile is gathered through the table
//    (staged once in LDS) into double-buffered LDS, K and V both row-major
//    with an XOR swizzle of the 16-byte chunks that keeps MFMA operand reads
//    and transposing reads free of bank conflicts beyond 2-way.
//  * S^T = K Q^T is computed (keys on the MFMA row axis), so the fp32 result
//    a lane holds -- 4 keys of one query row per 16x16 tile -- is, after the
//    softmax, exactly its B operand of O^T += V^T P^T: P never leaves
//    registers.  The V^T operand comes from two ds_read_b64_tr_b16 reads.
//  * online softmax in the log2 domain with the scale folded into the
//    exponent; the running output is rescaled only when a row's maximum
//    grows, and the causal mask is applied only in the last steps, whose keys
//    can pass a row's position.
#include <hip/hip_runtime.h>

#include <cmath>

#include "pa_common.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

template <typename E>
struct Mfma;
template <>
struct Mfma<BF16> {
  using vec = bf16x8_t;
  __device__ static floatx4_t mma(vec a, vec b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static uint16_t cvt(float x) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x)); }
};
template <>
struct Mfma<F16> {
  using vec = f16x8_t;
  __device__ static floatx4_t mma(vec a, vec b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static uint16_t cvt(float x) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x)); }
};

constexpr int kPrefillWaves = 8;
constexpr int kPrefillThreads = 64 * kPrefillWaves;
constexpr int kKeysPerStep = 64;

// 16-byte chunk position of (key, chunk) inside a K or V tile row in LDS.
// Rows are stored unpadded; the XOR keeps the 16 rows one MFMA operand read
// touches -- and the 4 rows x 2 chunks one transposing read touches -- on
// distinct bank groups.
template <int DCH>
__device__ __forceinline__ int swz(int key, int chunk) {
  if constexpr (DCH >= 16)
    return chunk ^ ((2 * (key & 7) + ((key >> 3) & 1)) & (DCH - 1));
  else
    return chunk ^ ((key >> 1) & (DCH - 1));
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane 4k+q supplies the address of 4 consecutive 16-bit elements and
// lane 4q+e receives element e of lanes q, 4+q, 8+q, 12+q.
__device__ __forceinline__ uint2 lds_read_tr(const char* p) {
  const v4i16_t v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Workgroup ids are handed round-robin to the 8 XCDs, each with its own L2.
// Map id L to work item w so that every XCD gets a contiguous run of work:
// the workgroups of one KV head then share one L2 for that head's K/V.
__device__ __forceinline__ int xcd_contiguous(int L, int total) {
  constexpr int kXcds = 8;
  const int per = (total + kXcds - 1) / kXcds;
  const int full = total - (per - 1) * kXcds;  // XCDs that take `per` items; the rest take per - 1
  const int xcd = L % kXcds, local = L / kXcds;
  return xcd < full ? xcd * per + local : full * per + (xcd - full) * (per - 1) + local;
}

template <typename E, int D, int G, int BS>
__global__ void __launch_bounds__(kPrefillThreads)
    prefill_chunk_kernel(const char* __restrict__ pool_k, const char* __restrict__ pool_v, int64_t layer_off,
                         int64_t head_stride, const uint16_t* __restrict__ q, uint16_t* __restrict__ out,
                         const int32_t* __restrict__ table, int32_t T, int32_t H_q, int32_t ctx_before,
                         float scale_log2) {
  using M = Mfma<E>;
  using vec = typename M::vec;
  constexpr int ROWS = 16 * kPrefillWaves;  // query rows per workgroup, 16 per wave
  constexpr int TP = ROWS / G;              // positions per workgroup
  constexpr int KT = kKeysPerStep;          // keys per step
  constexpr int KS = D / 32;                // MFMA k-steps over the head dim
  constexpr int DT = D / 16;                // 16-dim output tiles
  constexpr int NT = KT / 16;               // 16-key score tiles per step
  constexpr int KK = KT / 32;               // 32-key PV k-steps per step
  constexpr int ROWB = D * 2;               // bytes per K/V row in LDS
  constexpr int DCH = D / 8;                // 16-byte chunks per row
  constexpr int CPT = KT * DCH / kPrefillThreads;  // chunks per thread per side per step
  static_assert(ROWS % G == 0, "query group must divide the workgroup's rows");
  static_assert(KT % BS == 0 || BS % KT == 0, "steps align with blocks");
  static_assert(CPT >= 1 && KT * DCH % kPrefillThreads == 0, "staging covers the tile");

  __shared__ __attribute__((aligned(16))) char lds_k[2][KT * ROWB];
  __shared__ __attribute__((aligned(16))) char lds_v[2][KT * ROWB];
  extern __shared__ int32_t s_table[];  // [ceil(keys needed / BS)]

  // Work item w = (KV head, position tile); tiles of a head run last-first,
  // since later positions see more keys.
  const int ntiles = (T + TP - 1) / TP;
  const int w = xcd_contiguous(blockIdx.x, gridDim.x);  // gridDim.x = ntiles * H_kv
  const int g = w / ntiles;
  const int t0 = (ntiles - 1 - w % ntiles) * TP;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int li = lane & 15;
  const int lg = lane >> 4;
  const int t_last = min(t0 + TP, T) - 1;
  const int kmax = ctx_before + t_last + 1;  // no row of this workgroup sees key kmax or later
  const int nsteps = (kmax + KT - 1) / KT;
  const int first_masked_key = ctx_before + t0 + 1;

  // This lane's query row (MFMA B operand) and its last visible key.
  vec qb[KS];
  const int r = wave * 16 + li;
  const int pos = t0 + r / G;
  const int limit = ctx_before + pos;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (pos < T) raw = load16(q + (static_cast<int64_t>(pos) * H_q + g * G + r % G) * D + ks * 32 + lg * 8);
    qb[ks] = __builtin_bit_cast(vec, raw);
  }

  float m = -INFINITY, lsum = 0.0f;
  floatx4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const char* kbase = pool_k + layer_off + static_cast<int64_t>(g) * head_stride;
  const char* vbase = pool_v + layer_off + static_cast<int64_t>(g) * head_stride;

  // The workgroup's slice of the block table, staged once.
  const int nblk_used = (kmax + BS - 1) / BS;
  for (int i = tid; i < nblk_used; i += kPrefillThreads) s_table[i] = table[i];
  __syncthreads();

  // Staging: thread handles chunk c = tid + i * threads of each tile, i.e.
  // (key c / DCH, chunk c % DCH); consecutive threads read consecutive 16 B
  // of one K/V row.  Keys at or past kmax are zero-filled.
  uint4 kst[CPT], vst[CPT];
  auto gload = [&](int step) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * kPrefillThreads;
      const int key = step * KT + c / DCH;
      if (key < kmax) {
        const int64_t phys = s_table[key / BS];
        const int64_t off = (phys * BS + key % BS) * static_cast<int64_t>(ROWB) + (c % DCH) * 16;
        kst[i] = load16(kbase + off);
        vst[i] = load16(vbase + off);
      } else {
        kst[i] = make_uint4(0, 0, 0, 0);
        vst[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lds_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * kPrefillThreads;
      const int kr = c / DCH;
      const int at = kr * ROWB + swz<DCH>(kr, c % DCH) * 16;
      *reinterpret_cast<uint4*>(&lds_k[buf][at]) = kst[i];
      *reinterpret_cast<uint4*>(&lds_v[buf][at]) = vst[i];
    }
  };

  gload(0);
  lds_store(0);
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    if (step + 1 < nsteps) gload(step + 1);
    const int key0 = step * KT;

    // S^T = K Q^T: NT tiles of 16 keys x this wave's 16 rows.
    floatx4_t st[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      st[n] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
      const int kr = n * 16 + li;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const vec a = *reinterpret_cast<const vec*>(&lds_k[buf][kr * ROWB + swz<DCH>(kr, ks * 4 + lg) * 16]);
        st[n] = M::mma(a, qb[ks], st[n]);
      }
    }

    // Online softmax on unscaled scores (for scale > 0 the max commutes with
    // the scale, which is folded into the exponent).
    if (scale_log2 <= 0.0f) {
#pragma unroll
      for (int n = 0; n < NT; ++n) st[n] *= scale_log2;
    }
    const float c = scale_log2 > 0.0f ? scale_log2 : 1.0f;
    const bool masked = key0 + KT > first_masked_key;
    float mx = -INFINITY;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sv = st[n][i];
        if (masked && key0 + n * 16 + lg * 4 + i > limit) sv = -INFINITY;
        st[n][i] = sv;
        mx = fmaxf(mx, sv);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx * c);
    if (__any(mnew > m)) {
      const float alpha = __builtin_amdgcn_exp2f(m - ((mnew == -INFINITY) ? 0.0f : mnew));
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    const float ms = (m == -INFINITY) ? 0.0f : m;
    vec pb[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint16_t h[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(st[2 * kk][i], c, -ms));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(st[2 * kk + 1][i], c, -ms));
        lsum += p0 + p1;
        h[i] = M::cvt(p0);
        h[4 + i] = M::cvt(p1);
      }
      uint4 raw = make_uint4(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16),
                             h[4] | (uint32_t(h[5]) << 16), h[6] | (uint32_t(h[7]) << 16));
      pb[kk] = __builtin_bit_cast(vec, raw);
    }

    // O^T += V^T P^T.  The lane's P^T operand holds keys kk*32 + lg*4 + [0,4)
    // then kk*32 + 16 + lg*4 + [0,4) of its row; two transposing reads give
    // V^T for the same keys at dim dt*16 + li (lane 4k+q addresses key k,
    // dims 4q..4q+3 of the tile).
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int k4 = li >> 2, q4 = li & 3;
        const int dch = dt * 2 + (q4 >> 1), dsub = (q4 & 1) * 8;
        const int ka = kk * 32 + lg * 4 + k4;
        const int kb = ka + 16;
        const uint2 lo = lds_read_tr(&lds_v[buf][ka * ROWB + swz<DCH>(ka, dch) * 16 + dsub]);
        const uint2 hi = lds_read_tr(&lds_v[buf][kb * ROWB + swz<DCH>(kb, dch) * 16 + dsub]);
        const vec a = __builtin_bit_cast(vec, make_uint4(lo.x, lo.y, hi.x, hi.y));
        o[dt] = M::mma(a, pb[kk], o[dt]);
      }
    }

    if (step + 1 < nsteps) lds_store(buf ^ 1);
    __syncthreads();
  }

  // Normalise and write: the lane holds dims dt*16 + lg*4 + [0,4) of row li.
  float lt = lsum;
  lt += __shfl_xor(lt, 16);
  lt += __shfl_xor(lt, 32);
  if (pos >= T) return;
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  uint16_t* orow = out + (static_cast<int64_t>(pos) * H_q + g * G + r % G) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const uint32_t lo = M::cvt(o[dt][0] * inv) | (uint32_t(M::cvt(o[dt][1] * inv)) << 16);
    const uint32_t hi = M::cvt(o[dt][2] * inv) | (uint32_t(M::cvt(o[dt][3] * inv)) << 16);
    *reinterpret_cast<uint2*>(orow + dt * 16 + lg * 4) = make_uint2(lo, hi);
  }
}

using PrefillFn = void (*)(const pa_kv_pool*, int32_t, void*, const void*, int32_t, int32_t, const int32_t*,
                           int32_t, float, hipStream_t);

template <typename E, int D, int G, int BS>
static void launch_prefill(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t T, int32_t H_q,
                           const int32_t* table, int32_t ctx_before, float scale_log2, hipStream_t stream) {
  constexpr int TP = 16 * kPrefillWaves / G;
  const int64_t head_stride = static_cast<int64_t>(pool->num_blocks) * BS * D * 2;
  const int64_t layer_off = static_cast<int64_t>(layer) * pool->num_kv_heads * head_stride;
  dim3 grid(static_cast<uint32_t>((T + TP - 1) / TP) * pool->num_kv_heads);
  const size_t table_lds = static_cast<size_t>((static_cast<int64_t>(ctx_before) + T + BS - 1) / BS) * sizeof(int32_t);
  hipLaunchKernelGGL((prefill_chunk_kernel<E, D, G, BS>), grid, dim3(kPrefillThreads), table_lds, stream,
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

extern "C" int pa_prefill_chunk(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t T,
                                int32_t H_q, const int32_t* block_table, int32_t nb, int32_t ctx_before, float scale,
                                hipStream_t stream) {
  using namespace pa;
  if (int e = check_pool(pool, layer)) return e;
  if (T < 0 || H_q <= 0 || nb < 0 || ctx_before < 0) return fail(PA_EINVAL, "pa_prefill_chunk: negative size");
  if (T == 0) return PA_OK;
  if (!out || !q || !block_table) return fail(PA_EINVAL, "pa_prefill_chunk: NULL argument");
  if (H_q % pool->num_kv_heads) return fail(PA_EINVAL, "pa_prefill_chunk: H_q must be a multiple of num_kv_heads");
  const int64_t total = static_cast<int64_t>(ctx_before) + T;
  if (total > INT32_MAX) return fail(PA_EINVAL, "pa_prefill_chunk: ctx_before + T overflows");
  if (ceil_div(total, pool->block_size) > nb) return fail(PA_EINVAL, "pa_prefill_chunk: block table too short");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(pool->k) |
       reinterpret_cast<uintptr_t>(pool->v)) & 15u)
    return fail(PA_EINVAL, "pa_prefill_chunk: q, out and pool must be 16-byte aligned");
  if (ceil_div(T, 16) * pool->num_kv_heads > INT32_MAX) return fail(PA_EINVAL, "pa_prefill_chunk: grid too large");
  // The kernel keeps its slice of the block table in LDS next to ~70 KB of K/V tiles.
  if (ceil_div(total, pool->block_size) * 4 > 64 * 1024)
    return fail(PA_ENOTSUP, "pa_prefill_chunk: ctx_before + T needs more than 16,384 table entries");
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
