// Shared pieces of the gfx950 library: element traits, 16-byte vector
// loads, fp32 <-> bf16/f16 conversion, cross-lane sums and error plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_host.h"

namespace pa {

// ---------------------------------------------------------------- elements
// Storage types: fp32 as float, bf16 and f16 as raw 16-bit patterns.
struct F32 {
  using storage = float;
  static constexpr int bytes = 4;
};
struct BF16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
};
struct F16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
};

// Widen the elements of one 16-byte chunk (4 dwords) to fp32.
__device__ __forceinline__ void widen(F32, const uint4& c, float* out) {
  out[0] = __uint_as_float(c.x);
  out[1] = __uint_as_float(c.y);
  out[2] = __uint_as_float(c.z);
  out[3] = __uint_as_float(c.w);
}

// bf16 is the upper half of a binary32: the low element of a dword is
// widened by a shift, the high one by masking off the low half.
__device__ __forceinline__ void widen_dword_bf16(uint32_t u, float* out) {
  out[0] = __uint_as_float(u << 16);
  out[1] = __uint_as_float(u & 0xFFFF0000u);
}
__device__ __forceinline__ void widen(BF16, const uint4& c, float* out) {
  widen_dword_bf16(c.x, out + 0);
  widen_dword_bf16(c.y, out + 2);
  widen_dword_bf16(c.z, out + 4);
  widen_dword_bf16(c.w, out + 6);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, static_cast<uint16_t>(h));
  return static_cast<float>(v);
}
__device__ __forceinline__ void widen(F16, const uint4& c, float* out) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = half_bits_to_float(w[i] & 0xFFFFu);
    out[2 * i + 1] = half_bits_to_float(w[i] >> 16);
  }
}

// fp32 -> bf16, round to nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  _Float16 h = static_cast<_Float16>(f);  // v_cvt_f16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ void store_elem(F32, void* base, int64_t i, float v) {
  static_cast<float*>(base)[i] = v;
}
__device__ __forceinline__ void store_elem(BF16, void* base, int64_t i, float v) {
  static_cast<uint16_t*>(base)[i] = float_to_bf16_bits(v);
}
__device__ __forceinline__ void store_elem(F16, void* base, int64_t i, float v) {
  static_cast<uint16_t*>(base)[i] = float_to_half_bits(v);
}

__device__ __forceinline__ uint4 load16(const void* p) { return *static_cast<const uint4*>(p); }
// The same load marked non-temporal (the K/V stream: each byte is read once
// per launch, and should not push the block tables and lengths, which every
// launch reads first, out of the L2).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Two 16-bit floats in one dword, for the packed dot products.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- lanes
// Cross-lane moves inside a row of 16 lanes through DPP (no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i inside each 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i inside each 16
constexpr int kDppRor4 = 0x124;        // rotate by 4 lanes inside each 16
constexpr int kDppRor8 = 0x128;        // lane i <-> i^8 inside each 16

// Sum over aligned groups of N consecutive lanes (N = 2..64); every lane of
// the group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  if constexpr (N >= 2) x += dpp_move<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp_move<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp_move<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_move<kDppMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// The row (sequence or position, query head) a merge workgroup takes, in an
// order that runs KV head g's rows on XCD g mod 8 (workgroup L runs on XCD
// L mod 8): the decode, shared-prefix and split prefill kernels run KV head
// g's workgroups there too (KV head fastest in their grids), so with H_kv a
// multiple of 8 the merge reads the partials from the L2 they were written
// through.  Only while the partials fit the L2s: larger ones come from HBM
// either way, and the plain row order reads them as one stream.
constexpr int64_t kMergeFromL2Bytes = int64_t{16} << 20;  // half of the 8 XCDs' 4 MiB L2s
__device__ __forceinline__ int64_t merge_row(int64_t L, int32_t H_q, int32_t H_kv) {
  const int G = H_q / H_kv;
  const int g = static_cast<int>(L % H_kv);
  const int64_t rest = L / H_kv;
  return (rest / G) * H_q + g * G + rest % G;
}

}  // namespace pa
