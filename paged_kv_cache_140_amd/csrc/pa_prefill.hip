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
//  * workgroup = 4 waves = 128 query rows of one KV head: TP = 128/G
//    positions x the G query heads that share the KV head, so every K/V tile
//    staged in LDS serves all G heads.  Row r is (position r / G, head r % G).
//  * keys advance 64 at a time.  The tile is gathered block by block through
//    the table into double-buffered LDS: K row-major (padded rows), V
//    transposed with a key order that makes each lane's PV operand one
//    16-byte read.
//  * S^T = K Q^T is computed (keys on the MFMA row axis), so the fp32 result
//    a lane holds -- 4 keys of one query row per 16x16 tile -- is, after the
//    softmax, exactly its B operand of O^T += V^T P^T: P never leaves
//    registers.
//  * online softmax in the log2 domain; the causal mask is applied only in
//    the last steps, whose keys can pass a row's position.
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

constexpr int kPrefillThreads = 256;

// Byte column inside a V^T row, XOR-swizzled by the dim's 8-row group so that
// the 16 lanes staging one key quad (dims 8 apart, rows 1,152 B apart) spread
// over 8 bank groups instead of one; 16-byte chunks stay intact, so operand
// reads apply the same map to their chunk start.
__device__ __forceinline__ int vt_col(int dim, int colbyte) { return colbyte ^ (((dim >> 3) & 7) << 4); }
constexpr int kKeysPerStep = 64;

template <typename E, int D, int G, int BS>
__global__ void __launch_bounds__(kPrefillThreads)
    prefill_chunk_kernel(const char* __restrict__ pool_k, const char* __restrict__ pool_v, int64_t layer_off,
                         int64_t head_stride, const uint16_t* __restrict__ q, uint16_t* __restrict__ out,
                         const int32_t* __restrict__ table, int32_t T, int32_t H_q, int32_t ctx_before,
                         float scale_log2) {
  using M = Mfma<E>;
  using vec = typename M::vec;
  constexpr int TP = 128 / G;       // positions per workgroup
  constexpr int KT = kKeysPerStep;  // keys per step
  constexpr int RT = 2;             // 16-row tiles per wave
  constexpr int KS = D / 32;        // MFMA k-steps over the head dim
  constexpr int DT = D / 16;        // 16-dim output tiles
  constexpr int KROW = D * 2 + 16;  // LDS bytes per K row (padded against bank conflicts)
  constexpr int VROW = KT * 2 + 16; // LDS bytes per V^T row
  constexpr int DCH = D / 8;        // 16-byte chunks per K/V row
  static_assert(128 % G == 0, "query group must divide 128 rows");
  static_assert(KT % BS == 0 || BS % KT == 0, "steps align with blocks");

  __shared__ __attribute__((aligned(16))) char lds_k[2][KT * KROW];
  __shared__ __attribute__((aligned(16))) char lds_v[2][D * VROW];
  extern __shared__ int32_t s_table[];  // [ceil(keys needed / BS)]

  const int g = blockIdx.y;
  const int t0 = blockIdx.x * TP;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int li = lane & 15;
  const int lg = lane >> 4;
  const int t_last = min(t0 + TP, T) - 1;
  const int kmax = ctx_before + t_last + 1;
  const int nsteps = (kmax + KT - 1) / KT;
  const int first_masked_key = ctx_before + t0 + 1;  // keys beyond this may be masked for some row

  // Query rows of this lane (as the MFMA B operand) and their key limits.
  vec qb[RT][KS];
  int limit[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = wave * 32 + rt * 16 + li;
    const int pos = t0 + r / G;
    const int head = g * G + r % G;
    limit[rt] = ctx_before + pos;  // row sees keys 0 .. limit
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (pos < T) raw = load16(q + (static_cast<int64_t>(pos) * H_q + head) * D + ks * 32 + lg * 8);
      qb[rt][ks] = __builtin_bit_cast(vec, raw);
    }
  }

  float m[RT], lsum[RT];
  floatx4_t o[RT][DT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    lsum[rt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[rt][dt] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const char* kbase = pool_k + layer_off + static_cast<int64_t>(g) * head_stride;
  const char* vbase = pool_v + layer_off + static_cast<int64_t>(g) * head_stride;

  // Staging: K chunks (key, 16-byte dim chunk) and V units (4 keys, 16-byte dim chunk).
  constexpr int KCH = KT * DCH / kPrefillThreads;                         // K chunks per thread
  constexpr int VUNITS = (KT / 4) * DCH;                                  // V units per step
  constexpr int VPT = (VUNITS + kPrefillThreads - 1) / kPrefillThreads;  // V units per thread
  uint4 kst[KCH];
  uint4 vst[VPT][4];

  auto key_addr = [&](const char* base, int key, int dchunk) -> const char* {
    const int64_t phys = s_table[key / BS];
    return base + (phys * BS + key % BS) * static_cast<int64_t>(D * 2) + dchunk * 16;
  };
  // Gathers stop at kmax: no row of this workgroup sees a later key (those
  // tiles are zero-filled), and s_table holds exactly the entries below it.
  auto gload = [&](int step) {
    const int key0 = step * KT;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * kPrefillThreads;
      const int key = key0 + c / DCH;
      kst[i] = key < kmax ? load16(key_addr(kbase, key, c % DCH)) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int u = tid + i * kPrefillThreads;
      if (u < VUNITS) {
        const int keyq = key0 + (u / DCH) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vst[i][j] = keyq + j < kmax ? load16(key_addr(vbase, keyq + j, u % DCH)) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lds_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * kPrefillThreads;
      *reinterpret_cast<uint4*>(&lds_k[buf][(c / DCH) * KROW + (c % DCH) * 16]) = kst[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int u = tid + i * kPrefillThreads;
      if (u < VUNITS) {
        const int kq = (u / DCH) * 4;  // first of 4 keys, relative to the step
        const int local = kq & 31;
        const int pos = (kq & ~31) + ((local & 15) >> 2) * 8 + (local >> 4) * 4;
        const uint32_t w[4][4] = {{vst[i][0].x, vst[i][0].y, vst[i][0].z, vst[i][0].w},
                                  {vst[i][1].x, vst[i][1].y, vst[i][1].z, vst[i][1].w},
                                  {vst[i][2].x, vst[i][2].y, vst[i][2].z, vst[i][2].w},
                                  {vst[i][3].x, vst[i][3].y, vst[i][3].z, vst[i][3].w}};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int sh = (e & 1) * 16;
          const uint32_t a0 = (w[0][e >> 1] >> sh) & 0xFFFFu, a1 = (w[1][e >> 1] >> sh) & 0xFFFFu;
          const uint32_t a2 = (w[2][e >> 1] >> sh) & 0xFFFFu, a3 = (w[3][e >> 1] >> sh) & 0xFFFFu;
          uint2 pk = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
          const int dim = (u % DCH) * 8 + e;
          *reinterpret_cast<uint2*>(&lds_v[buf][dim * VROW + vt_col(dim, pos * 2)]) = pk;
        }
      }
    }
  };

  // The workgroup's slice of the block table, staged once: the per-step
  // gathers then find physical blocks in LDS instead of waiting on a global
  // load before every K/V load.
  const int nblk_used = (kmax + BS - 1) / BS;
  for (int i = tid; i < nblk_used; i += kPrefillThreads) s_table[i] = table[i];
  __syncthreads();

  gload(0);
  lds_store(0);
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    if (step + 1 < nsteps) gload(step + 1);
    const int key0 = step * KT;

    // S^T tiles: 4 key tiles of 16 x RT row tiles.
    floatx4_t st[RT][KT / 16];
#pragma unroll
    for (int n = 0; n < KT / 16; ++n) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) st[rt][n] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const vec a = *reinterpret_cast<const vec*>(&lds_k[buf][(n * 16 + li) * KROW + (ks * 32 + lg * 8) * 2]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) st[rt][n] = M::mma(a, qb[rt][ks], st[rt][n]);
      }
    }

    const bool masked = key0 + KT > first_masked_key;
    vec pb[RT][KT / 32];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float mx = m[rt];
#pragma unroll
      for (int n = 0; n < KT / 16; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s = st[rt][n][i] * scale_log2;
          if (masked && key0 + n * 16 + lg * 4 + i > limit[rt]) s = -INFINITY;
          st[rt][n][i] = s;
          mx = fmaxf(mx, s);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float ms = (mx == -INFINITY) ? 0.0f : mx;
      const float alpha = __builtin_amdgcn_exp2f(m[rt] - ms);
      m[rt] = mx;
      lsum[rt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[rt][dt] *= alpha;
#pragma unroll
      for (int n = 0; n < KT / 16; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(st[rt][n][i] - ms);
          lsum[rt] += p;
          st[rt][n][i] = p;
        }
      }
#pragma unroll
      for (int kk = 0; kk < KT / 32; ++kk) {
        uint16_t h[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[i] = M::cvt(st[rt][2 * kk][i]);
          h[4 + i] = M::cvt(st[rt][2 * kk + 1][i]);
        }
        uint4 raw = make_uint4(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16),
                               h[4] | (uint32_t(h[5]) << 16), h[6] | (uint32_t(h[7]) << 16));
        pb[rt][kk] = __builtin_bit_cast(vec, raw);
      }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int kk = 0; kk < KT / 32; ++kk) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int dim = dt * 16 + li;
        const vec a = *reinterpret_cast<const vec*>(&lds_v[buf][dim * VROW + vt_col(dim, (kk * 32 + lg * 8) * 2)]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) o[rt][dt] = M::mma(a, pb[rt][kk], o[rt][dt]);
      }
    }

    if (step + 1 < nsteps) lds_store(buf ^ 1);
    __syncthreads();
  }

  // Normalise and write: lane holds dims dt*16 + lg*4 + [0,4) of row li.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float lt = lsum[rt];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const int r = wave * 32 + rt * 16 + li;
    const int pos = t0 + r / G;
    if (pos >= T) continue;
    const int head = g * G + r % G;
    uint16_t* orow = out + (static_cast<int64_t>(pos) * H_q + head) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint32_t lo = M::cvt(o[rt][dt][0] * inv) | (uint32_t(M::cvt(o[rt][dt][1] * inv)) << 16);
      const uint32_t hi = M::cvt(o[rt][dt][2] * inv) | (uint32_t(M::cvt(o[rt][dt][3] * inv)) << 16);
      *reinterpret_cast<uint2*>(orow + dt * 16 + lg * 4) = make_uint2(lo, hi);
    }
  }
}

using PrefillFn = void (*)(const pa_kv_pool*, int32_t, void*, const void*, int32_t, int32_t, const int32_t*,
                           int32_t, float, hipStream_t);

template <typename E, int D, int G, int BS>
static void launch_prefill(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t T, int32_t H_q,
                           const int32_t* table, int32_t ctx_before, float scale_log2, hipStream_t stream) {
  constexpr int TP = 128 / G;
  const int64_t head_stride = static_cast<int64_t>(pool->num_blocks) * BS * D * 2;
  const int64_t layer_off = static_cast<int64_t>(layer) * pool->num_kv_heads * head_stride;
  dim3 grid(static_cast<uint32_t>((T + TP - 1) / TP), pool->num_kv_heads);
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
  if (pool->num_kv_heads > 65535) return fail(PA_EINVAL, "pa_prefill_chunk: grid too large");
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
