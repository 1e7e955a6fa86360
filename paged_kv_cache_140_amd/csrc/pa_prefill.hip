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
//  * workgroup = 4 waves x 32 query rows of one KV head: TP = 128/G
//    positions x the G query heads that share the KV head, so every K/V tile
//    staged in LDS serves all G heads.  Row r is (position r / G, head r % G).
//    32 rows per wave make each K/V byte read from LDS feed 32 rows; at 256
//    registers and 64 KiB of LDS two workgroups share a CU, and their
//    independent barriers let one's softmax overlap the other's MFMA.
//  * keys advance 64 at a time.  Each step's K and V tiles go from HBM
//    straight into double-buffered LDS (global_load_lds_dwordx4), row-major
//    with an XOR swizzle of the 16-byte chunks that keeps MFMA operand reads
//    and transposing reads free of bank conflicts.  The block id of every
//    1 KiB load is wave-uniform and read with a scalar load.
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

#include "pa_common.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

// v_mfma_f32_32x32x16_{bf16,f16}.  Lane l supplies A row l%32 and B column
// l%32 at k = (l/32)*8 + [0,8); it receives D column l%32, rows
// 8*(v/4) + (l/32)*4 + v%4 for v = 0..15.
template <typename E>
struct Mfma;
template <>
struct Mfma<BF16> {
  using vec = bf16x8_t;
  __device__ static floatx16_t mma(vec a, vec b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static uint16_t cvt(float x) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x)); }
};
template <>
struct Mfma<F16> {
  using vec = f16x8_t;
  __device__ static floatx16_t mma(vec a, vec b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static uint16_t cvt(float x) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x)); }
};

constexpr int kPrefillWaves = 4;
constexpr int kPrefillThreads = 64 * kPrefillWaves;
constexpr int kRowsPerWave = 32;
constexpr int kKeysPerStep = 64;

// K and V tiles sit in LDS row-major (one key per row, unpadded); the 16-byte
// chunk c of row `row` is stored at chunk position c ^ swz(row).  LDS serves
// a 16-byte read 16 lanes at a time and an 8-byte read 32 lanes at a time,
// each pass over 256 bytes of banks.  The XOR makes both passes touch 256
// distinct bytes: the MFMA operand read (16 consecutive rows, one chunk each)
// and the transposing read (4 consecutive rows, the 4 chunks of one 32-dim
// slice each).  It depends on row & 15 only.
template <int DCH>
__device__ __forceinline__ int swz(int row) {
  if constexpr (DCH >= 16)
    return 4 * (row & 3) + ((row >> 2) & 3);  // 256-byte rows
  else
    return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);  // 128-byte rows: two per 256 bytes
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

// Max / sum of a lane's value and the value of lane l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane l's bytes land at lds + 16*l; lds must be wave-uniform.
__device__ __forceinline__ void load_to_lds(const char* src, char* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
#endif
}
__device__ __forceinline__ void wait_loads_to_lds() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
  constexpr int ROWS = kRowsPerWave * kPrefillWaves;  // query rows per workgroup
  constexpr int TP = ROWS / G;                        // positions per workgroup
  constexpr int KT = kKeysPerStep;                    // keys per step
  constexpr int KS = D / 16;                          // QK k-steps over the head dim
  constexpr int DT = D / 32;                          // 32-dim output tiles
  constexpr int NT = KT / 32;                         // 32-key score tiles per step
  constexpr int ROWB = D * 2;                         // bytes per K/V row
  constexpr int DCH = D / 8;                          // 16-byte chunks per row
  constexpr int TILE = KT * ROWB;                     // bytes of one K or V tile
  constexpr int RPL = 1024 / ROWB;                    // rows per 1 KiB direct load
  constexpr int LPW = TILE / 1024 / kPrefillWaves;    // direct loads per wave per side per step
  static_assert(ROWS % G == 0, "query group must divide the workgroup's rows");
  static_assert(BS % RPL == 0, "the rows of one direct load lie in one block");
  static_assert(LPW >= 1 && TILE % (1024 * kPrefillWaves) == 0, "direct loads cover the tile");
  static_assert(kPrefillWaves == 4 && kRowsPerWave * ROWB <= TILE, "each wave stages its output in one tile array");

  // Double-buffered K and V tiles as four distinct arrays: the compiler can
  // then tell that the next tile's direct loads never alias the tile being
  // read, and adds no wait for them before the reads.
  __shared__ __attribute__((aligned(1024))) char lk0[TILE];
  __shared__ __attribute__((aligned(1024))) char lv0[TILE];
  __shared__ __attribute__((aligned(1024))) char lk1[TILE];
  __shared__ __attribute__((aligned(1024))) char lv1[TILE];

  // Work item w = (KV head, position tile); tiles of a head run last-first,
  // since later positions see more keys.
  const int ntiles = (T + TP - 1) / TP;
  const int w = xcd_contiguous(blockIdx.x, gridDim.x);  // gridDim.x = ntiles * H_kv
  const int g = w / ntiles;
  const int t0 = (ntiles - 1 - w % ntiles) * TP;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int li = lane & 31;
  const int h = lane >> 5;
  const int t_last = min(t0 + TP, T) - 1;
  const int kmax = ctx_before + t_last + 1;  // no row of this workgroup sees key kmax or later
  const int nsteps = (kmax + KT - 1) / KT;
  const int first_masked_key = ctx_before + t0 + 1;

  // This lane's query row (MFMA B operand: dims ks*16 + h*8 + [0,8)) and its
  // last visible key.
  const int r = wave * kRowsPerWave + li;
  const int pos = t0 + r / G;
  const int limit = ctx_before + pos;
  vec qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (pos < T) raw = load16(q + (static_cast<int64_t>(pos) * H_q + g * G + r % G) * D + ks * 16 + h * 8);
    qb[ks] = __builtin_bit_cast(vec, raw);
  }

  const char* kbase = pool_k + layer_off + static_cast<int64_t>(g) * head_stride;
  const char* vbase = pool_v + layer_off + static_cast<int64_t>(g) * head_stride;

  // Direct global -> LDS loads of one step's K and V tiles.  This wave's
  // loads cover rows wave*WROWS + [0, WROWS) of the tile; load i fills 1 KiB
  // of LDS, rows row0 .. row0 + RPL - 1, lane l landing at byte 16*l: it
  // fetches logical chunk (l % DCH) ^ swz(row).  Keys at or past kmax are
  // clamped to kmax - 1 (finite data that every row masks out).
  constexpr int WROWS = LPW * RPL;                  // tile rows per wave
  constexpr int NBW = WROWS >= BS ? WROWS / BS : 1;  // blocks those rows touch
  struct Blocks {
    int32_t b[NBW];
  };
  // Block ids of this wave's rows at `step` (wave-uniform, scalar loads).
  // Entry j serves rows from j*BS on; clamping the key first keeps every
  // clamped row's block.
  auto fetch = [&](int step) {
    Blocks bl;
#pragma unroll
    for (int j = 0; j < NBW; ++j) bl.b[j] = table[min(step * KT + wave * WROWS + j * BS, kmax - 1) / BS];
    return bl;
  };
  auto issue = [&](int step, const Blocks& bl, char* kdst, char* vdst) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int row0 = wave * WROWS + i * RPL;
      const int row = row0 + lane / DCH;
      const int key = min(step * KT + row, kmax - 1);
      const int64_t blk = bl.b[NBW > 1 ? i * RPL / BS : 0];
      const int64_t off = (blk * BS + (key & (BS - 1))) * ROWB + (((lane % DCH) ^ swz<DCH>(row)) * 16);
      load_to_lds(kbase + off, kdst + row0 * ROWB);
      load_to_lds(vbase + off, vdst + row0 * ROWB);
    }
  };

  float m = -INFINITY, lsum = 0.0f;
  floatx16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = floatx16_t{};

  // Transposing-read geometry: this lane, as source lane 4*k4 + q4 of its
  // 16-lane group g16, addresses row 4*(g16/2) + k4 (+8) of a 16-key slice,
  // dims dt*32 + (g16%2)*16 + 4*q4 + [0,4).
  const int g16 = lane >> 4, k4 = (lane >> 2) & 3, q4 = lane & 3;
  const int vrow = 4 * (g16 >> 1) + k4;
  const int vsw_lo = swz<DCH>(vrow), vsw_hi = swz<DCH>(vrow + 8);  // the same for + 16 s + 32 n

  // One step: attend to the tile in (kt, vt) while the next step's tile
  // streams into (kn, vn).
  Blocks next = fetch(0);
  auto step_body = [&](int step, const char* kt, const char* vt, char* kn, char* vn) {
    if (step + 1 < nsteps) issue(step + 1, next, kn, vn);
    const int key0 = step * KT;

    // S^T = K Q^T: NT tiles of 32 keys x this wave's 32 rows.  The lane holds
    // keys n*32 + 8*(v/4) + 4*h + v%4 of row li.
    floatx16_t st[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      st[n] = floatx16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const vec a =
            *reinterpret_cast<const vec*>(kt + (n * 32 + li) * ROWB + (((ks * 2 + h) ^ swz<DCH>(li)) * 16));
        st[n] = M::mma(a, qb[ks], st[n]);
      }
    }
    next = fetch(step + 2);

    // Online softmax on unscaled scores (for scale > 0 the max commutes with
    // the scale, which is folded into the exponent).
    if (scale_log2 <= 0.0f) {
#pragma unroll
      for (int n = 0; n < NT; ++n) st[n] *= scale_log2;
    }
    const float c = scale_log2 > 0.0f ? scale_log2 : 1.0f;
    if (key0 + KT > first_masked_key) {  // uniform: only the last steps reach past a row's position
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (key0 + n * 32 + 8 * (v >> 2) + 4 * h + (v & 3) > limit) st[n][v] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, st[n][v]);
    mx = max_halves(mx);
    const float mnew = fmaxf(m, mx * c);
    if (__any(mnew > m)) {
      const float alpha = __builtin_amdgcn_exp2f(m - ((mnew == -INFINITY) ? 0.0f : mnew));
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    const float ms = (m == -INFINITY) ? 0.0f : m;

    // P^T operand for 16-key slice (n, s): slots 0..7 of this lane are keys
    // n*32 + 16s + 4h + [0,4) and n*32 + 16s + 8 + 4h + [0,4), i.e. its score
    // values 8s .. 8s+7 of tile n.
    vec pb[NT][2];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        uint16_t hh[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(st[n][8 * s2 + i], c, -ms));
          lsum += p;
          hh[i] = M::cvt(p);
        }
        const uint4 raw = make_uint4(hh[0] | (uint32_t(hh[1]) << 16), hh[2] | (uint32_t(hh[3]) << 16),
                                     hh[4] | (uint32_t(hh[5]) << 16), hh[6] | (uint32_t(hh[7]) << 16));
        pb[n][s2] = __builtin_bit_cast(vec, raw);
      }
    }

    // O^T += V^T P^T.  The V^T operand for dims dt*32 + li and the same 8 keys
    // comes from two transposing reads (rows vrow and vrow + 8 of the slice).
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int rw = n * 32 + s2 * 16 + vrow;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int ch = dt * 4 + (g16 & 1) * 2 + (q4 >> 1);
          const uint2 lo = lds_read_tr(vt + rw * ROWB + (ch ^ vsw_lo) * 16 + (q4 & 1) * 8);
          const uint2 hi = lds_read_tr(vt + (rw + 8) * ROWB + (ch ^ vsw_hi) * 16 + (q4 & 1) * 8);
          const vec a = __builtin_bit_cast(vec, make_uint4(lo.x, lo.y, hi.x, hi.y));
          o[dt] = M::mma(a, pb[n][s2], o[dt]);
        }
      }
    }

    wait_loads_to_lds();
    __syncthreads();
  };

  issue(0, next, lk0, lv0);
  next = fetch(1);
  wait_loads_to_lds();
  __syncthreads();
  for (int step = 0; step < nsteps; step += 2) {
    step_body(step, lk0, lv0, lk1, lv1);
    if (step + 1 >= nsteps) break;
    step_body(step + 1, lk1, lv1, lk0, lv0);
  }

  // Normalise; stage the wave's 32 x D output rows in LDS (wave w takes one
  // of the four tile arrays, no longer read) and write whole rows.  The lane
  // holds dims dt*32 + 8*j + 4*h + [0,4) of row li, j = 0..3; chunk c of row
  // rr is stored at chunk position c ^ (rr % DCH).
  const float lt = sum_halves(lsum);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  char* ob = wave == 0 ? lk0 : wave == 1 ? lv0 : wave == 2 ? lk1 : lv1;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = M::cvt(o[dt][4 * j] * inv) | (uint32_t(M::cvt(o[dt][4 * j + 1] * inv)) << 16);
      const uint32_t hi = M::cvt(o[dt][4 * j + 2] * inv) | (uint32_t(M::cvt(o[dt][4 * j + 3] * inv)) << 16);
      const int chunk = (dt * 4 + j) ^ (li % DCH);
      *reinterpret_cast<uint2*>(ob + li * ROWB + chunk * 16 + h * 8) = make_uint2(lo, hi);
    }
  }
  __syncthreads();
  constexpr int OCH = kRowsPerWave * DCH / 64;  // 16-byte chunks per lane
#pragma unroll
  for (int i = 0; i < OCH; ++i) {
    const int idx = i * 64 + lane;
    const int orow = idx / DCH, och = idx % DCH;
    const int rr = wave * kRowsPerWave + orow;
    const int opos = t0 + rr / G;
    if (opos < T) {
      const uint4 val = *reinterpret_cast<const uint4*>(ob + orow * ROWB + ((och ^ (orow % DCH)) * 16));
      *reinterpret_cast<uint4*>(out + (static_cast<int64_t>(opos) * H_q + g * G + rr % G) * D + och * 8) = val;
    }
  }
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
