// Device code of the causal prefill chunk for gfx950: the per-work-item body
// shared by the prefill kernel and the mixed decode + prefill kernel.
//
// What it computes: chunk row t sits at position ctx_before + t and attends
// to keys 0 .. ctx_before + t, gathered through the sequence's block table
// ([ttlab] "llm-kv-cache-02-serving-engine-kv", section "새 문제: 긴 프리필이
// 디코드를 멈춘다"; [icarus] "PagedAttention", sections "KV Cache 为什么难管理"
// and "Block Table 如何工作").  The design notes are in pa_prefill.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

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

constexpr int kPrefillWaves = 8;
constexpr int kPrefillThreads = 64 * kPrefillWaves;
constexpr int kRowsPerWave = 32;
constexpr int kKeysPerStep = 64;
// How far (log2 units) a row's max may pass the softmax reference before the
// prefill rescales its running sum and output: probabilities stay <= 256.
constexpr float kSlack = 8.0f;

// LDS tile layout for K and V (KT keys x D dims, 16-bit): columns of 64
// bytes (4 chunks of 16 bytes, 32 dims) are stored one after another, each
// as KT rows of 64 bytes, and the 4 chunks of row `row` are rotated by
// (row >> 2) & 3.  LDS serves a 16-byte read 16 lanes at a time and an
// 8-byte read 32 lanes at a time, each pass over 256 bytes of banks; this
// layout makes both passes touch 256 distinct bytes for the MFMA operand
// read (16 consecutive rows, one chunk each) and the transposing read (4
// consecutive rows, the 4 chunks of one column each), and every lane's
// address is a per-lane base plus a compile-time offset.
template <int KT>
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return (chunk >> 2) * (KT * 64) + row * 64 + (((chunk & 3) ^ ((row >> 2) & 3)) * 16);
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
// lane l's bytes land at lds + 16*l; lds must be wave-uniform.  Written as
// inline assembly rather than the compiler's builtin: with a builtin load
// into LDS in flight, the compiler's wait-count pass cannot separate LDS
// reads from it and waits for every outstanding LDS read (lgkmcnt(0)) before
// the first MFMA of each unit, instead of only the one that unit needs.  The
// kernel tracks these loads itself (wait_loads_to_lds before the barrier
// that precedes their first reader).  M0 (the LDS byte address, the low half
// of the generic address) is an operand of the statement, so the compiler
// itself writes it and knows its value afterwards.
__device__ __forceinline__ void load_to_lds(const char* src, char* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
#endif
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima), as a builtin
// so that the compiler's own wait tracking knows the loads have landed.
__device__ __forceinline__ void wait_loads_to_lds() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier without a memory fence (a fence would wait for every
// direct load in flight): this wave's LDS reads are complete (lgkmcnt(0), so
// no buffer is overwritten under a pending read), the compiler keeps every
// instruction on its side of it (so the units of the ping-pong stay in their
// phases), and loads into LDS stay in flight.  Each wave waits for its own
// loads before the barrier that precedes their first reader.
__device__ __forceinline__ void barrier_keep_loads() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
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

// LDS of one prefill workgroup: double-buffered K and V tiles, lds[0..1] K,
// lds[2..3] V.  Every access names its buffer with a compile-time index, so
// the compiler sees that direct loads into one buffer never alias reads of
// another.
template <int D>
using PrefillLds = char[4][kKeysPerStep * D * 2];

// One work item of a prefill chunk: w = KV head * ntiles + i, where tile i
// holds positions [(ntiles - 1 - i) * TP, ...) (the tiles of a head run
// last-first, since later positions see more keys).  The caller passes
// the workgroup's LDS and, between two items, a workgroup barrier.
//
// Split over the keys: the item covers its 64-key steps [step_lo, step_hi)
// only (clamped to the steps its rows can see; an empty range returns at
// once) and, with ws_o set, writes its rows' un-normalised output (fp32,
// [T][H_q][D] per split at ws_o) and (running max, sum) pairs ([T][H_q][2]
// at ws_ml) instead of the output; a merge combines the splits.  Without a
// split: step_lo = 0, step_hi >= every item's steps, ws_o = nullptr.
//
// key_end: no row sees key key_end or later (INT32_MAX for a chunk).  With
// ctx_before >= key_end every row sees exactly the keys [0, key_end): the
// shared-prefix pass of a decode, where the rows are the queries of the
// sequences that share those keys' blocks.
template <typename E, int D, int G, int BS>
__device__ __forceinline__ void prefill_tile(int w, PrefillLds<D>& lds, const char* __restrict__ pool_k,
                                             const char* __restrict__ pool_v, int64_t layer_off, int64_t head_stride,
                                             const uint16_t* __restrict__ q, uint16_t* __restrict__ out,
                                             const int32_t* __restrict__ table, int32_t T, int32_t H_q,
                                             int32_t ctx_before, float scale_log2, int step_lo, int step_hi,
                                             float* __restrict__ ws_o, float* __restrict__ ws_ml, int32_t key_end) {
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
  constexpr int RG = KT / 16;                         // 16-row groups per tile (one 1 KiB load each per column)
  constexpr int LPW = TILE / 1024 / kPrefillWaves;    // direct loads per wave per tile
  static_assert(ROWS % G == 0, "query group must divide the workgroup's rows");
  static_assert(LPW >= 1 && TILE % (1024 * kPrefillWaves) == 0 && kPrefillWaves % RG == 0,
                "direct loads cover the tile, one row group per wave");
  static_assert(DCH % 4 == 0 && BS >= 8, "whole 64-byte columns; at most two blocks per row group");
  static_assert(2 * kRowsPerWave * ROWB <= TILE, "two waves stage their output in one tile");

  static_assert(sizeof(PrefillLds<D>) == 4 * TILE, "LDS tile geometry");
  const int ntiles = (T + TP - 1) / TP;
  const int g = w / ntiles;
  const int t0 = (ntiles - 1 - w % ntiles) * TP;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int li = lane & 31;
  const int h = lane >> 5;
  const int t_last = min(t0 + TP, T) - 1;
  const int kmax = min(ctx_before + t_last + 1, key_end);  // no row of this workgroup sees key kmax or later
  // local steps 0 .. nsteps-1 are the item's 64-key steps s0 .. s0+nsteps-1
  const int s0 = step_lo;
  const int nsteps = min((kmax + KT - 1) / KT, step_hi) - s0;
  if (nsteps <= 0) return;  // uniform: this split holds none of the item's keys
  const int first_masked_key = min(ctx_before + t0 + 1, key_end);
  // Waves 0-3 (group A) and 4-7 (group B) share the SIMDs pairwise and run
  // the same work one phase apart.
  const bool group_b = wave >= kPrefillWaves / 2;
  // A wave whose 32 rows all lie past the last row (a tile of few rows, such
  // as a shared-prefix group's few sequences) has nothing to compute: it
  // still issues its share of every tile load and meets every barrier, but
  // skips its MFMA and softmax units.
  const bool live = t0 + (wave * kRowsPerWave) / G < T;

  // This lane's query row (MFMA B operand: dims ks*16 + h*8 + [0,8)) and its
  // last visible key.
  const int r = wave * kRowsPerWave + li;
  const int pos = t0 + r / G;
  const int limit = min(ctx_before + pos, key_end - 1);
  vec qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (pos < T) raw = load16(q + (static_cast<int64_t>(pos) * H_q + g * G + r % G) * D + ks * 16 + h * 8);
    qb[ks] = __builtin_bit_cast(vec, raw);
  }

  const char* kbase = pool_k + layer_off + static_cast<int64_t>(g) * head_stride;
  const char* vbase = pool_v + layer_off + static_cast<int64_t>(g) * head_stride;

  // Direct global -> LDS loads of one K or V tile.  This wave loads row
  // group rg = wave % RG (rows 16*rg + [0,16)) of columns cg0 .. cg0+LPW-1;
  // each load fills 1 KiB of LDS (16 rows x 64 bytes), lane l landing at
  // byte 16*l: row 16*rg + l/4, rotated chunk position l % 4.  Keys at or
  // past kmax are clamped to kmax - 1 (finite data that every row masks out).
  const int rg = wave % RG, cg0 = (wave / RG) * LPW;
  const int lrow = rg * 16 + (lane >> 2);                         // tile row this lane loads
  const int lchunk = ((lane & 3) ^ ((lrow >> 2) & 3)) * 16;       // byte of its chunk within the column
  struct Blocks {
    int32_t lo, hi;  // block ids of rows 16*rg + [0,8) and + [8,16) (the same when BS >= 16)
  };
  // Block ids of this wave's rows at `step` (wave-uniform scalar loads);
  // clamping the key first keeps every clamped row's block.
  auto fetch = [&](int step) __attribute__((always_inline)) {
    Blocks b;
    b.lo = table[min((s0 + step) * KT + rg * 16, kmax - 1) / BS];
    b.hi = BS >= 16 ? b.lo : table[min((s0 + step) * KT + rg * 16 + 8, kmax - 1) / BS];
    return b;
  };
  auto issue = [&](const char* base, int step, const Blocks& bl, char* dst) __attribute__((always_inline)) {
    const int key = min((s0 + step) * KT + lrow, kmax - 1);
    const int64_t blk = (BS >= 16 || (lane >> 2) < 8) ? bl.lo : bl.hi;
    const char* src = base + (blk * BS + (key & (BS - 1))) * ROWB + lchunk;
#pragma unroll
    for (int i = 0; i < LPW; ++i)
      load_to_lds(src + (cg0 + i) * 64, dst + (cg0 + i) * (KT * 64) + rg * 1024);
  };

  float m = -INFINITY, lsum = 0.0f;
  floatx16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = floatx16_t{};
  floatx16_t st[NT];  // scores of the step whose softmax is next
  vec pb[NT][2];      // probabilities of the step whose PV is next

  // Read geometry.  MFMA operand of K: row n*32 + li, chunk 2*ks + h, i.e.
  // column ks/2 at a per-lane base that depends on ks % 2.  Transposing read
  // of V: this lane, as source lane 4*k4 + q4 of its 16-lane group g16,
  // addresses row 4*(g16/2) + k4 (+8) of a 16-key slice, dims
  // dt*32 + (g16%2)*16 + 4*q4 + [0,4): column dt at a per-lane base.
  const int kb_even = tile_off<KT>(li, h), kb_odd = tile_off<KT>(li, 2 + h);
  const int g16 = lane >> 4, k4 = (lane >> 2) & 3, q4 = lane & 3;
  const int vrow = 4 * (g16 >> 1) + k4, vch = (g16 & 1) * 2 + (q4 >> 1);
  const int vb_lo = tile_off<KT>(vrow, vch) + (q4 & 1) * 8, vb_hi = tile_off<KT>(vrow + 8, vch) + (q4 & 1) * 8;

  // MFMA unit: S^T = K Q^T for the next step from tile kt (keys on the MFMA
  // row axis: the lane holds keys n*32 + 8*(v/4) + 4*h + v%4 of row li) and,
  // with PV, O^T += V^T P^T for this step from tile vt.  The V^T operand for
  // dims dt*32 + li and the 8 keys of P's slots comes from two transposing
  // reads (rows vrow and vrow + 8 of the 16-key slice).  Operands are read
  // into arrays and the instruction groups are ordered explicitly so that
  // LDS reads run one group of MFMAs ahead instead of each MFMA waiting for
  // its own read.
  auto gemm = [&](auto with_pv, const char* kt, const char* vt) __attribute__((always_inline)) {
    constexpr bool kPV = decltype(with_pv)::value;
    vec ka[NT][KS];
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ka[n][ks] = *reinterpret_cast<const vec*>(kt + (ks >> 1) * (KT * 64) + n * 32 * 64 +
                                                  ((ks & 1) ? kb_odd : kb_even));
    vec va[NT][2][DT];
    if constexpr (kPV) {
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const char* vs = vt + (n * 32 + s2 * 16) * 64 + dt * (KT * 64);
            const uint2 lo = lds_read_tr(vs + vb_lo);
            const uint2 hi = lds_read_tr(vs + vb_hi);
            va[n][s2][dt] = __builtin_bit_cast(vec, make_uint4(lo.x, lo.y, hi.x, hi.y));
          }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      st[n] = floatx16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) st[n] = M::mma(ka[n][ks], qb[ks], st[n]);
    }
    if constexpr (kPV) {
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[dt] = M::mma(va[n][s2][dt], pb[n][s2], o[dt]);
    }
    // Order: K reads of tile 0; tile-0 MFMAs each followed by one K read of
    // tile 1; with PV, tile-1 MFMAs each followed by two transposing reads,
    // then the first half of the PV MFMAs each followed by two more, then the
    // rest.  (Masks: 0x100 LDS read, 0x008 MFMA.)
    static_assert(NT == 2 && 4 * DT == 2 * KS, "schedule shape");
    __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (kPV) {
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * KS, 0);
    } else {
      __builtin_amdgcn_sched_group_barrier(0x008, KS, 0);
    }
  };

  // Softmax unit j: online softmax of step j's scores into P_j.  Scores are
  // unscaled (for scale > 0 the max commutes with the scale, which is folded
  // into the exponent).  P^T slots 0..7 for 16-key slice (n, s) are keys
  // n*32 + 16s + 4h + [0,4) and n*32 + 16s + 8 + 4h + [0,4): score values
  // 8s .. 8s+7 of tile n.
  auto softmax = [&](int j) __attribute__((always_inline)) {
    const int key0 = (s0 + j) * KT;
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
    // The running max m is the exponent's reference: it is raised (and l,
    // O rescaled) only when a row's max passes it by more than kSlack, so
    // every probability stays <= 2^kSlack and, after the first few steps,
    // the rescale is almost never taken.  l and O share the reference, so
    // O / l is unchanged.
    const float mcand = mx * c;
    if (__any(mcand > m + kSlack)) {
      const float mnew = fmaxf(m, mcand);
      const float alpha = __builtin_amdgcn_exp2f(m - ((mnew == -INFINITY) ? 0.0f : mnew));
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    const float ms = (m == -INFINITY) ? 0.0f : m;
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
  };

  // Schedule.  Every wave runs the same units: gemm(-1), softmax(0),
  // gemm(0), softmax(1), ..., softmax(n-1), gemm(n-1), each closed by a
  // barrier.  Group B passes one extra barrier first, so it runs unit u in
  // phase u + 1 while group A runs it in phase u: in every phase one wave of
  // each SIMD feeds the matrix core and the other runs the softmax on the
  // vector ALU.  (A barrier counts arrivals, not which instruction arrives.)
  // gemm(j-1) reads K_j and V_{j-1}.  Round m = phases 2m and 2m+1: at the
  // start of round m every wave issues its share of K_{m+1} and V_m into the
  // buffers that round m-1 finished reading, and waits for them at the end
  // of the round.  Group A issues round j with its gemm(j-1); group B issues
  // round j+1 with its softmax(j) (round 0 before its extra barrier).
  Blocks blk_v = fetch(0);  // block ids of the V tile of the next round
  Blocks blk_k = fetch(1);  // ... and of its K tile
  auto issue_round = [&](int mr, char* kw, char* vw) __attribute__((always_inline)) {
    if (mr + 1 < nsteps) issue(kbase, mr + 1, blk_k, kw);
    if (mr < nsteps) issue(vbase, mr, blk_v, vw);
    blk_v = blk_k;
    blk_k = fetch(mr + 2);
  };
  issue(kbase, 0, blk_v, lds[0]);
  wait_loads_to_lds();
  barrier_keep_loads();
  if (group_b) {
    issue_round(0, lds[1], lds[2]);
    barrier_keep_loads();
  }
  // gemm(-1): scores of step 0 only.
  if (live) gemm(std::false_type{}, lds[0], lds[3]);
  if (!group_b) issue_round(0, lds[1], lds[2]);
  if (group_b) wait_loads_to_lds();
  barrier_keep_loads();
  // Step j's units: gemm(j-1), then softmax(j) unless j == n.  k_rd / v_rd:
  // the buffers gemm(j-1) reads (K_j, V_{j-1}; at j == n the K tile is stale
  // and its scores unused); A writes K_{j+1}, V_j into (ka, va) right after
  // issuing its reads; B writes K_{j+2}, V_{j+1} into (k_rd, v_rd) once
  // both groups have finished gemm(j-1).  Issuing after the reads keeps the
  // compiler from waiting for these loads before them.
  auto softmax_unit = [&](int j, char* kb, char* vb) __attribute__((always_inline)) {
    if (group_b) issue_round(j + 1, kb, vb);
    if (live) softmax(j);
    if (!group_b) wait_loads_to_lds();
    barrier_keep_loads();
  };
  softmax_unit(0, lds[0], lds[3]);
  auto body = [&](int j, char* k_rd, char* v_rd, char* ka, char* va) __attribute__((always_inline)) {
    if (live) gemm(std::true_type{}, k_rd, v_rd);
    if (!group_b) issue_round(j, ka, va);
    if (group_b) wait_loads_to_lds();
    barrier_keep_loads();
    if (j == nsteps) return;
    softmax_unit(j, k_rd, v_rd);
  };
  for (int j = 1; j <= nsteps; j += 2) {
    body(j, lds[1], lds[2], lds[0], lds[3]);
    if (j + 1 > nsteps) break;
    body(j + 1, lds[0], lds[3], lds[1], lds[2]);
  }
  if (!group_b) barrier_keep_loads();

  const float lt = sum_halves(lsum);
  if (ws_o) {
    // A split: the row's un-normalised output, running max and sum (rows
    // that see none of this split's keys leave m = -inf, l = 0, o = 0).
    if (pos < T) {
      const int64_t row = static_cast<int64_t>(pos) * H_q + g * G + r % G;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<float4*>(ws_o + row * D + dt * 32 + 8 * j + 4 * h) =
              make_float4(o[dt][4 * j], o[dt][4 * j + 1], o[dt][4 * j + 2], o[dt][4 * j + 3]);
      if (h == 0) *reinterpret_cast<float2*>(ws_ml + 2 * row) = make_float2(m, lt);
    }
    return;
  }

  // Normalise; stage the wave's 32 x D output rows in LDS (two waves per
  // tile array, no longer read) and write whole rows.  The lane holds dims
  // dt*32 + 8*j + 4*h + [0,4) of row li, j = 0..3; chunk c of row rr is
  // stored at chunk position c ^ (rr % DCH).
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  char* ob = &lds[wave >> 1][(wave & 1) * kRowsPerWave * ROWB];
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

}  // namespace pa
