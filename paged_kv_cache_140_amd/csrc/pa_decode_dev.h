// Device code of paged decode attention for gfx950: the per-workgroup body
// shared by the decode kernel and the mixed decode + prefill kernel.
//
// What it computes: every sequence's newest query reads all of its visible
// K/V, found through the block table that maps logical to physical blocks,
// and takes softmax(scale * q K^T) V ([icarus] "PagedAttention",
// icarus.shaojiemike.top, sections "Block Table 如何工作" and
// "不会降低单请求的理论读取量"; [ttlab] "llm-kv-cache-02-serving-engine-kv",
// section "블록과 블록 표").  The design notes are in pa_decode.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "pa_common.h"

namespace pa {

constexpr float kNegInf = -INFINITY;

// Unit = NLD wave loads of K and V (TPW tokens each), 2 units in flight per
// wave.  Few query heads per KV head: short units.  Many heads (more
// arithmetic per byte): longer units for more independent work per lane.
// More loads in flight do not raise the streaming rate; they lengthen the
// queues, and the kernel's final loads then wait that much longer (measured:
// 4 units in flight cost ~0.8 us more per launch than 2 on a 75 MB decode).
template <typename E, int D, int BS, int G>
struct DecodeShape {
  static constexpr int S = E::bytes;
  static constexpr int VEC = 16 / S;                             // elements per lane chunk
  static constexpr int LPT = D / VEC;                            // lanes per token row
  static constexpr int TPW = 64 / LPT;                           // token rows per wave load
  static constexpr int NLD_MAX = G <= 2 ? 2 : 4;
  static constexpr int NLD = (BS / TPW) < NLD_MAX ? (BS / TPW) : NLD_MAX;  // loads per unit per side
  static constexpr int U = NLD * TPW;                            // tokens per unit
  static constexpr int UPB = BS / U;                             // units per block
  static constexpr int RING = 2;                                 // units in flight per wave
  static_assert(BS % TPW == 0, "block size must hold whole wave loads");
  static_assert(BS % U == 0, "units tile a block");
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// A lane's value and that of lane ^ S, as a pair whose order differs
// between lanes (callers combine the two symmetrically).  Lanes 16 and 32
// apart: v_permlane16_swap / v_permlane32_swap; 8 apart: DPP row_ror:8.
template <int S>
__device__ __forceinline__ void pair_with(float x, float& a, float& b) {
  static_assert(S == 8 || S == 16 || S == 32, "lane distance");
  if constexpr (S == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else if constexpr (S == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    a = x;
    b = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  }
}


// q.k over one lane's 16-byte chunk.  The query is kept in its storage
// format; bf16 and f16 pairs go through the packed dot instructions (exact
// products, fp32 accumulate), fp32 through FMAs.
template <typename E>
struct QChunk;
template <>
struct QChunk<BF16> {
  uint32_t w[4];
  __device__ void set(const uint4& raw) { w[0] = raw.x, w[1] = raw.y, w[2] = raw.z, w[3] = raw.w; }
  __device__ float dot(const uint4& k) const {
    float d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[0]), __builtin_bit_cast(bf16x2_t, k.x),
                                              0.0f, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[1]), __builtin_bit_cast(bf16x2_t, k.y), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[2]), __builtin_bit_cast(bf16x2_t, k.z), d, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[3]), __builtin_bit_cast(bf16x2_t, k.w), d,
                                           false);
  }
};
template <>
struct QChunk<F16> {
  uint32_t w[4];
  __device__ void set(const uint4& raw) { w[0] = raw.x, w[1] = raw.y, w[2] = raw.z, w[3] = raw.w; }
  __device__ float dot(const uint4& k) const {
    float d = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w[0]), __builtin_bit_cast(f16x2_t, k.x), 0.0f, false);
    d = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w[1]), __builtin_bit_cast(f16x2_t, k.y), d, false);
    d = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w[2]), __builtin_bit_cast(f16x2_t, k.z), d, false);
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w[3]), __builtin_bit_cast(f16x2_t, k.w), d, false);
  }
};
template <>
struct QChunk<F32> {
  float f[4];
  __device__ void set(const uint4& raw) { widen(F32{}, raw, f); }
  __device__ float dot(const uint4& k) const {
    float kf[4];
    widen(F32{}, k, kf);
    float d = f[0] * kf[0];
    d = fmaf(f[1], kf[1], d);
    d = fmaf(f[2], kf[2], d);
    return fmaf(f[3], kf[3], d);
  }
};


// Probabilities packed two tokens to a register in the pool's 16-bit type,
// for P.V as packed dot products (exact products, fp32 accumulate).
template <typename E>
struct PPair;
template <>
struct PPair<BF16> {
  static constexpr uint32_t kOnes = 0x3F803F80u;  // (1, 1)
  __device__ static uint32_t pack(float a, float b) {
    const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static float dot(uint32_t p, uint32_t v, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p), __builtin_bit_cast(bf16x2_t, v), c, false);
  }
};
template <>
struct PPair<F16> {
  static constexpr uint32_t kOnes = 0x3C003C00u;  // (1, 1)
  __device__ static uint32_t pack(float a, float b) {
    const f16x2_t v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static float dot(uint32_t p, uint32_t v, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, p), __builtin_bit_cast(f16x2_t, v), c, false);
  }
};

// Scattered heads: with G >= 4 query heads per KV head, lane bits 5 and 4
// pick a quarter of the heads, so a lane holds G/4 "own" heads: (G/2)*bit5 +
// (G/4)*bit4 + j; with G = 2, bit 5 picks the lane's one head.  gather_heads
// turns the own heads' values into all G heads' values, in head order, in
// every lane: v_permlane16_swap and v_permlane32_swap of a register with
// itself return (the even row's value, the odd row's value) and (the lower
// half's, the upper half's) in every lane.
template <int G>
__device__ __forceinline__ void gather_heads(const uint32_t* own, uint32_t* all) {
  if constexpr (G == 2) {
    const auto t = __builtin_amdgcn_permlane32_swap(own[0], own[0], false, false);
    all[0] = t[0];
    all[1] = t[1];
  } else {
    constexpr int NH = G / 4;
    uint32_t y[2 * NH];
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const auto t = __builtin_amdgcn_permlane16_swap(own[j], own[j], false, false);
      y[j] = t[0];
      y[j + NH] = t[1];
    }
#pragma unroll
    for (int k = 0; k < 2 * NH; ++k) {
      const auto t = __builtin_amdgcn_permlane32_swap(y[k], y[k], false, false);
      all[k] = t[0];
      all[k + 2 * NH] = t[1];
    }
  }
}

// Whether a split decode runs unsplit, one partition per (sequence, KV
// head): when the batch's longest sequence holds no more blocks than one
// CU's share of the whole batch (the sum of all sequences' blocks times H_kv,
// over the CU count), every (sequence, KV head) fits the share a CU would
// stream anyway, and a split only adds partial writes and merge work.  The
// host plans the grid from the longest context alone (the lengths stay on
// the device), so it cannot tell a uniform mix of long contexts from one
// long context among short ones; every workgroup of the decode and of its
// merge reads the B lengths and takes the same decision.  Unsplit, the
// first B * H_kv workgroups of the grid (in launch order) take one
// (sequence, KV head) each and write its output as an unsplit decode does,
// the rest exit, and the merge writes nothing.  cus <= 0: never.
// Wave-uniform; every wave computes it on its own.
__device__ __forceinline__ bool decode_unsplit(const int32_t* __restrict__ lens, int B, int BS, int H_kv, int cus) {
  if (cus <= 0) return false;
  int64_t sum = 0;
  int longest = 0;
  for (int i = threadIdx.x & 63; i < B; i += 64) {
    const int n = (lens[i] + BS - 1) / BS;
    sum += n;
    longest = max(longest, n);
  }
  for (int off = 32; off > 0; off >>= 1) {
    sum += __shfl_xor(sum, off);
    longest = max(longest, __shfl_xor(longest, off));
  }
  return __builtin_amdgcn_readfirstlane(static_cast<int64_t>(longest) * cus <= sum * H_kv);
}

// One workgroup's share of a decode: KV head g of sequence b, partition
// ``part`` (blocks [part, part + 1) * blocks_per_part), H_kv KV heads.  W is
// the workgroup's wave count, passed in rather than read from the dispatch:
// the table entry of a wave's second unit depends on it, and a load of the
// workgroup size would put one more memory round trip (which the scalar
// wait counter cannot separate from the table loads) before the first K/V
// loads.  smem holds W * G * (D + 2) floats.
//
// SUFFIX: the part of a decode that follows the first skip_blocks blocks of
// the sequence (a shared-prefix decode reads those for all its sharers at
// once): partition ``part`` covers blocks skip_blocks + [part, part + 1) *
// blocks_per_part, and the workgroup always writes (m, l, acc) partials,
// which a merge combines with the prefix's; an empty partition writes
// nothing.
//
// CHECKSUM: a measuring variant, not a decode: the same grid, block tables,
// unit walk and K/V loads, but each unit's bytes are XORed into a checksum
// instead of attended to (no q, no softmax, no output).  Each wave writes
// its checksum (uint32) to ws_ml at ((b * num_parts + part) * H_kv + g) * W
// + wave.  It measures what the decode's access pattern alone can stream.
template <typename E, int D, int G, int BS, bool FUSED, bool SUFFIX = false, bool CHECKSUM = false>
__device__ __forceinline__ void decode_body(int W, int g, int part, int H_kv, int b, float* __restrict__ smem,
                                            char* __restrict__ pool_k, char* __restrict__ pool_v, int64_t layer_off,
                                            int64_t head_stride, const char* __restrict__ q, void* __restrict__ out,
                                            const int32_t* __restrict__ block_tables, int32_t max_blocks,
                                            const int32_t* __restrict__ context_lens, float scale_log2, int32_t H_q,
                                            int32_t blocks_per_part, int32_t num_parts, float* __restrict__ ws_ml,
                                            float* __restrict__ ws_acc, const char* __restrict__ k_new,
                                            const char* __restrict__ v_new, const int32_t* __restrict__ new_slots,
                                            int skip_blocks = 0) {
  static_assert(!(SUFFIX && FUSED), "a shared-prefix decode appends beforehand");
  static_assert(!(CHECKSUM && (FUSED || SUFFIX)), "the checksum walk is the plain decode's");
  using Sh = DecodeShape<E, D, BS, G>;
  constexpr int S = Sh::S, VEC = Sh::VEC, LPT = Sh::LPT, TPW = Sh::TPW, NLD = Sh::NLD, U = Sh::U, UPB = Sh::UPB,
                RING = Sh::RING;
  // Wave-uniform by construction; readfirstlane lets the compiler keep the
  // unit walk and the block-table reads in scalar registers / scalar loads,
  // so that a table read never waits on the vector loads in flight.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // Scattered-score layout (16-bit pools, G >= 4): lane bits 4 and 5 pick
  // a quarter of a token row's 16-byte chunks, the CLO lowest bits a chunk
  // inside it (a lane quad still reads 64 contiguous bytes), and the bits in
  // between the token row.  q.k partial sums are then reduced across chunks
  // by swaps 32 and 16 lanes apart that leave each lane the scores of G/4
  // heads, so the softmax runs once per (token, head) per 4 lanes instead of
  // once per lane of the row, and P.V takes packed dot products over token
  // pairs.  Otherwise a row's chunks sit in adjacent lanes and every lane
  // keeps all G heads' scores.
  constexpr bool kScatter = S == 2 && G >= 2 && NLD % 2 == 0;
  constexpr int NS = kScatter ? (G >= 4 ? G / 4 : 1) : G;  // softmax states per lane
  constexpr int CLO = LPT / 4;              // scattered layout: chunks in the low lane bits
  static_assert(!kScatter || TPW == 4 || TPW == 8, "scattered layout: 4 or 8 token rows");
  const int r = kScatter ? (lane / CLO) % TPW : lane / LPT;            // token row inside a wave load
  const int c = kScatter ? lane % CLO + CLO * (lane / 16) : lane % LPT;  // 16-byte chunk of the row

  const int j0 = (SUFFIX ? skip_blocks : 0) + part * blocks_per_part;
  const int u_begin = j0 * UPB;
  const int32_t* btrow = block_tables + static_cast<int64_t>(b) * max_blocks;
  // Table entries of this wave's first RING units, read in parallel with the
  // sequence length instead of after it (the index is clamped to the row; an
  // entry past the sequence's end is simply not used).
  // Fused: the new token's slot, read with the length and the table entries
  // (one memory round trip for all of them, before the first K/V loads).
  const int new_slot = FUSED ? __builtin_amdgcn_readfirstlane(new_slots[b]) : -1;
  int32_t ph[RING];
#pragma unroll
  for (int p = 0; p < RING; ++p)
    ph[p] = max_blocks > 0 ? btrow[min((u_begin + wave + p * W) / UPB, max_blocks - 1)] : 0;
  const int ctx = __builtin_amdgcn_readfirstlane(context_lens[b]);
  const int nblk = (ctx + BS - 1) / BS;
  const int64_t head0 = static_cast<int64_t>(b) * H_q + static_cast<int64_t>(g) * G;

  if (j0 >= nblk) {
    // Nothing visible in this partition.  With a single partition that means
    // an empty sequence: its rows are zeros.  Split partitions past the end
    // are not counted by the merge.
    if constexpr (CHECKSUM) {
      if (lane == 0)
        reinterpret_cast<uint32_t*>(ws_ml)[((static_cast<int64_t>(b) * num_parts + part) * H_kv + g) * W + wave] = 0;
    } else if (!SUFFIX && num_parts == 1) {
      for (int i = threadIdx.x; i < G * D; i += W * 64) store_elem(E{}, out, head0 * D + i, 0.0f);
    }
    return;
  }
  const int j1 = min(j0 + blocks_per_part, nblk);

  // Fused append: this sequence's new token sits at position ctx - 1.  The
  // partition holding that position processes the unit holding it last, as
  // its masked tail, with that position masked out (vis = ctx - 1: the pool
  // row may be read, stale, but never counts); wave 0 adds the new token from
  // the input and writes it into its slot at the end.  Which unit is the
  // tail depends on ctx only, so the first K/V loads do not wait for the
  // slot, and the units streamed before it need no mask.  A negative slot
  // writes nothing and lets the tail read the pool's own row, as a plain
  // decode would.
  int vis = ctx;
  bool holds_new = false;
  bool owns_new = false;
  uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
  if constexpr (FUSED) {
    holds_new = (ctx - 1) / BS >= j0 && (ctx - 1) / BS < j1;
    owns_new = holds_new && new_slot >= 0;
    const int64_t new_row = (static_cast<int64_t>(b) * H_kv + g) * D * S;  // [B][H_kv][D] inputs
    kx = load16(k_new + new_row + c * 16);  // every lane: a fixed number of loads keeps the waits exact
    vx = load16(v_new + new_row + c * 16);
    if (owns_new) vis = ctx - 1;
  }

  QChunk<E> qc[G];
  if constexpr (!CHECKSUM) {
#pragma unroll
    for (int h = 0; h < G; ++h) qc[h].set(load16(q + ((head0 + h) * D + c * VEC) * S));
  }

  float m[NS], l[NS], acc[G][VEC];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    m[j] = kNegInf;
    l[j] = 0.0f;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[h][e] = 0.0f;
  }

  const char* kbase = pool_k + layer_off + static_cast<int64_t>(g) * head_stride;
  const char* vbase = pool_v + layer_off + static_cast<int64_t>(g) * head_stride;
  const int lane_off = (r * D + c * VEC) * S;

  // A placeholder load (a ring slot past the wave's last unit, or the tail
  // slot of a wave without the tail) keeps the count of loads in flight
  // fixed, so the waits stay exact.  It reads the head's block 0 rather than
  // re-reading a unit of K/V: every placeholder of the launch reads the same
  // few lines, which stay in L2, where a re-read of the non-temporal stream
  // would go back to HBM.
  auto load_unit = [&](int u, uint4* kr, uint4* vr, int32_t phys_id, bool dummy) {
    const int64_t phys = dummy ? 0 : __builtin_amdgcn_readfirstlane(phys_id);
    const int64_t off = (phys * BS + (dummy ? 0 : u % UPB) * U) * static_cast<int64_t>(D * S) + lane_off;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      kr[i] = load16_stream(kbase + off + i * TPW * D * S);
      vr[i] = load16_stream(vbase + off + i * TPW * D * S);
    }
  };

  uint32_t cs = 0;  // CHECKSUM: XOR of every loaded dword

  // One unit: NLD tokens per lane row, online-softmax update for G heads;
  // with ``masked``, tokens at positions >= vis_ take no part.
  auto process = [&](int u, const uint4* kr, const uint4* vr, bool masked, int vis_) {
    if constexpr (CHECKSUM) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) cs ^= kr[i].x ^ kr[i].y ^ kr[i].z ^ kr[i].w ^ vr[i].x ^ vr[i].y ^ vr[i].z ^ vr[i].w;
      return;
    }
    const int tok0 = u * U + r;
    if constexpr (kScatter) {
      constexpr int NH = NS;
      float x[NLD][NH];
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        float sp[G];
#pragma unroll
        for (int h = 0; h < G; ++h) sp[h] = qc[h].dot(kr[i]);
        // Chunks 32 lanes apart: the lower half keeps heads [0, G/2), the
        // upper half [G/2, G); then 16 apart: a quarter each.
        float w[G / 2];
#pragma unroll
        for (int h = 0; h < G / 2; ++h) {
          const auto t =
              __builtin_amdgcn_permlane32_swap(__float_as_uint(sp[h]), __float_as_uint(sp[h + G / 2]), false, false);
          w[h] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
        }
        const bool dead = masked && tok0 + i * TPW >= vis_;
#pragma unroll
        for (int j = 0; j < NH; ++j) {
          // G >= 4: chunks 16 lanes apart split the heads again; G = 2: they
          // are summed (each lane keeps its one head).
          uint32_t w2;
          if constexpr (G >= 4) {
            w2 = __float_as_uint(w[j + NH]);
          } else {
            w2 = __float_as_uint(w[j]);
          }
          const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(w[j]), w2, false, false);
          float y = __uint_as_float(t[0]) + __uint_as_float(t[1]);
          // the remaining chunk bits: the lowest lane bits
          y += dpp_move<kDppXor1>(y);
          if constexpr (CLO == 4) y += dpp_move<kDppXor2>(y);
          x[i][j] = dead ? kNegInf : y * scale_log2;
        }
      }
      float mx[NH];
      bool grew = false;
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        mx[j] = m[j];
#pragma unroll
        for (int i = 0; i < NLD; ++i) mx[j] = fmaxf(mx[j], x[i][j]);
        grew |= mx[j] > m[j];
      }
      if (__any(grew)) {
        uint32_t al[NH], alg[G];
#pragma unroll
        for (int j = 0; j < NH; ++j) {
          const float alpha = exp2_fast(m[j] - ((mx[j] == kNegInf) ? 0.0f : mx[j]));
          m[j] = mx[j];
          l[j] *= alpha;
          al[j] = __float_as_uint(alpha);
        }
        gather_heads<G>(al, alg);
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[h][e] *= __uint_as_float(alg[h]);
        }
      }
      float msafe[NH];
#pragma unroll
      for (int j = 0; j < NH; ++j) msafe[j] = (m[j] == kNegInf) ? 0.0f : m[j];
#pragma unroll
      for (int q2 = 0; q2 < NLD / 2; ++q2) {
        // Tokens 2*q2 and 2*q2+1 of the lane: probabilities packed per own
        // head (l sums the packed values, so it weighs what P.V weighs),
        // then gathered for all heads.
        uint32_t pk[NH], pg[G];
#pragma unroll
        for (int j = 0; j < NH; ++j) {
          pk[j] = PPair<E>::pack(exp2_fast(x[2 * q2][j] - msafe[j]), exp2_fast(x[2 * q2 + 1][j] - msafe[j]));
          l[j] = PPair<E>::dot(pk[j], PPair<E>::kOnes, l[j]);
        }
        gather_heads<G>(pk, pg);
        uint4 va = vr[2 * q2], vb = vr[2 * q2 + 1];
        // unused slots may hold anything (NaN included): select, not multiply
        if (masked && tok0 + 2 * q2 * TPW >= vis_) va = make_uint4(0, 0, 0, 0);
        if (masked && tok0 + (2 * q2 + 1) * TPW >= vis_) vb = make_uint4(0, 0, 0, 0);
        const uint32_t a4[4] = {va.x, va.y, va.z, va.w};
        const uint32_t b4[4] = {vb.x, vb.y, vb.z, vb.w};
        uint32_t vp[VEC];  // (element e of token 2*q2, element e of token 2*q2+1)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          vp[2 * d] = __builtin_amdgcn_perm(b4[d], a4[d], 0x05040100u);
          vp[2 * d + 1] = __builtin_amdgcn_perm(b4[d], a4[d], 0x07060302u);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[h][e] = PPair<E>::dot(pg[h], vp[e], acc[h][e]);
        }
      }
      return;
    }
    float s[NLD][G];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const bool dead = masked && tok0 + i * TPW >= vis_;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float d = group_sum<LPT>(qc[h].dot(kr[i])) * scale_log2;
        s[i][h] = dead ? kNegInf : d;
      }
    }
    // Running max: rescale (l, acc) only when some lane's max grew, which
    // after the first few units of a sequence is rare.
    float mx[G];
    bool grew = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mx[h] = m[h];
#pragma unroll
      for (int i = 0; i < NLD; ++i) mx[h] = fmaxf(mx[h], s[i][h]);
      grew |= mx[h] > m[h];
    }
    if (__any(grew)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float alpha = exp2_fast(m[h] - ((mx[h] == kNegInf) ? 0.0f : mx[h]));
        m[h] = mx[h];
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] *= alpha;
      }
    }
    float msafe[G];
#pragma unroll
    for (int h = 0; h < G; ++h) msafe[h] = (m[h] == kNegInf) ? 0.0f : m[h];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      float vf[VEC];
      widen(E{}, vr[i], vf);
      if (masked && tok0 + i * TPW >= vis_) {
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

  // Units of this partition: unmasked ones [u_first, u_full), stepping by W
  // per wave, streamed through a ring of RING loads in flight; then at most
  // one masked unit (partly visible, or, fused, the one holding ctx - 1),
  // handled by the wave that owns it.
  const int u_stop = min(j1 * UPB, (ctx + U - 1) / U);
  const int u_full = FUSED && holds_new ? (ctx - 1) / U : min(u_stop, ctx / U);
  const int u_first = u_begin + wave;
  const int n_w = u_full > u_first ? (u_full - u_first + W - 1) / W : 0;  // this wave's full units
  // The partly visible last unit (if this partition has it) is loaded first,
  // by the wave it falls to, and processed last with masking.
  const bool has_tail = u_full < u_stop && u_full >= u_first && (u_full - u_first) % W == 0;
  // Fused: the new token's share of the attention, added right after the
  // wave's first K/V loads are in flight (so its own input load overlaps
  // them): a unit whose only live token is row 0 of its first load, taken
  // from the input.  With N full units over W waves, waves 0 .. N mod W
  // (the last of them also takes the masked tail) hold one unit more than
  // the rest: the new token goes to wave W - 1 when it is one of the rest.
  const int new_wave = max(0, u_full - u_begin) % W < W - 1 ? W - 1 : 0;
  auto add_new_token = [&]() {
    if constexpr (FUSED) {
      if (owns_new && wave == new_wave) {
        uint4 kxa[NLD], vxa[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i) kxa[i] = kx, vxa[i] = vx;
        process(0, kxa, vxa, true, 1);
      }
    }
  };
  uint4 kt[NLD], vt[NLD];
  // The tail's table entry depends on ctx, one more dependent read than the
  // ring's first entries: its loads go after the ring's so that they do not
  // hold the ring's back.  Unconditional (a wave without the tail issues
  // placeholder loads): every wave then has the same loads in flight, and
  // the waits below stay exact.
  auto load_tail = [&]() __attribute__((always_inline)) {
    const int ut = has_tail ? u_full : u_begin;
    load_unit(ut, kt, vt, btrow[ut / UPB], !has_tail);
  };
  if (n_w > 0) {
    // Refills are unconditional (past the wave's last unit, placeholder
    // loads), so each ring slot stays in fixed registers and no load ever
    // waits for a later one.
    uint4 kr[RING][NLD], vr[RING][NLD];
#pragma unroll
    for (int p = 0; p < RING; ++p) {
      const bool live = p < n_w;
      load_unit(live ? u_first + p * W : u_first, kr[p], vr[p], live ? ph[p] : ph[0], !live);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_tail();
    add_new_token();
    for (int k = 0; k < n_w; k += RING) {
#pragma unroll
      for (int p = 0; p < RING; ++p) {
        const int idx = k + p;
        if (idx < n_w) {
          const int u = u_first + idx * W;
          process(u, kr[p], vr[p], false, vis);
        }
        // Keep refills in ring order: the in-order load counter then only
        // ever waits for the oldest slot.
        __builtin_amdgcn_sched_barrier(0);
        const int un = u_first + min(idx + RING, n_w - 1) * W;
        load_unit(un, kr[p], vr[p], btrow[un / UPB], idx + RING >= n_w);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (n_w <= 0) {
    load_tail();
    add_new_token();
  }
  if (has_tail) process(u_full, kt, vt, true, vis);

  if constexpr (CHECKSUM) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cs ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(cs), off));
    if (lane == 0)
      reinterpret_cast<uint32_t*>(ws_ml)[((static_cast<int64_t>(b) * num_parts + part) * H_kv + g) * W + wave] = cs;
    return;
  }

  // Softmax state of all G heads in every lane: mg, lg.
  float mg[G], lg[G];
  if constexpr (kScatter) {
    uint32_t mo[NS], lo[NS], ma[G], la[G];
#pragma unroll
    for (int j = 0; j < NS; ++j) mo[j] = __float_as_uint(m[j]), lo[j] = __float_as_uint(l[j]);
    gather_heads<G>(mo, ma);
    gather_heads<G>(lo, la);
#pragma unroll
    for (int h = 0; h < G; ++h) mg[h] = __uint_as_float(ma[h]), lg[h] = __uint_as_float(la[h]);
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) mg[h] = m[h], lg[h] = l[h];
  }

  // Merge the TPW row groups of this wave (lanes holding the same dims of
  // different tokens) with cross-lane VALU moves: pair_with gives a lane its
  // own value and its partner's, in either order, and the combine is
  // symmetric in the two.
  auto combine = [&](auto pair) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float m0, m1, l0, l1;
      pair(mg[h], m0, m1);
      pair(lg[h], l0, l1);
      const float mx = fmaxf(m0, m1);
      const float ms = (mx == kNegInf) ? 0.0f : mx;
      const float w0 = exp2_fast(m0 - ms);
      const float w1 = exp2_fast(m1 - ms);
      lg[h] = l0 * w0 + l1 * w1;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float a0, a1;
        pair(acc[h][e], a0, a1);
        acc[h][e] = a0 * w0 + a1 * w1;
      }
      mg[h] = mx;
    }
  };
  auto dpp_pair = [](auto ctl) {
    return [](float x, float& a, float& b) __attribute__((always_inline)) {
      a = x;
      b = dpp_move<decltype(ctl)::value>(x);
    };
  };
  auto swap_pair = [](auto dist) {
    return [](float x, float& a, float& b) __attribute__((always_inline)) { pair_with<decltype(dist)::value>(x, a, b); };
  };
  if constexpr (kScatter) {
    // rows in lane bits log2(CLO)..3: lane 2 apart (8 rows), then rotations
    // by 4 and 8 inside each 16, which reach all rows of bits 2 and 3
    if constexpr (CLO == 2) combine(dpp_pair(std::integral_constant<int, kDppXor2>{}));
    combine(dpp_pair(std::integral_constant<int, kDppRor4>{}));
    combine(dpp_pair(std::integral_constant<int, kDppRor8>{}));
  } else {
    // rows in lane bits log2(LPT)..5
    static_assert(LPT >= 8, "row groups are at least 8 lanes wide");
    if constexpr (LPT <= 8) combine(swap_pair(std::integral_constant<int, 8>{}));
    if constexpr (LPT <= 16) combine(swap_pair(std::integral_constant<int, 16>{}));
    if constexpr (LPT <= 32) combine(swap_pair(std::integral_constant<int, 32>{}));
  }

  // Waves -> LDS: sm_m[W][G], sm_l[W][G], sm_acc[W][G][D].
  float* sm_m = smem;
  float* sm_l = smem + W * G;
  float* sm_acc = smem + 2 * W * G;
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm_acc[(wave * G + h) * D + c * VEC + e] = acc[h][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sm_m[wave * G + h] = mg[h];
      sm_l[wave * G + h] = lg[h];
    }
  }
  __syncthreads();

  for (int i = threadIdx.x; i < G * D; i += W * 64) {
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
    if (!SUFFIX && num_parts == 1) {
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

  if constexpr (FUSED) {
    // The new token's row into its slot, last: nothing in this launch reads
    // it back, and a barrier after these stores would wait for them.
    if (owns_new && wave == 0 && r == 0) {
      const int64_t dst =
          layer_off + static_cast<int64_t>(g) * head_stride + static_cast<int64_t>(new_slot) * D * S + c * 16;
      *reinterpret_cast<uint4*>(pool_k + dst) = kx;
      *reinterpret_cast<uint4*>(pool_v + dst) = vx;
    }
  }
}

}  // namespace pa
