// Decode attention of a batch whose sequences share prefixes, reading every
// shared block once for all of its sharers.
//
// What it computes: exactly what pa_decode computes -- each sequence's
// newest query reads all of its visible K/V through its block table
// ([icarus] "PagedAttention", icarus.shaojiemike.top, sections "Block Table
// 如何工作" and "不会降低单请求的理论读取量").  Parallel sampling, beam search
// and common prompt prefixes leave several sequences whose tables start
// with the same physical blocks, shared by reference count ([icarus] "支持块
// 级共享"; [ttlab] "llm-kv-cache-02-serving-engine-kv", section "블록을 함께
// 쓰기").  A plain decode reads such a block once per sharer; here it is read
// once per step for all of them.
//
// How: the caller names groups of consecutive batch rows and how many
// leading blocks each group's rows share.
//  * prefix pass: for a group of n rows the shared keys [0, shared_blocks *
//    block_size) are the same for all n * G query rows of a KV head, so
//    S = Q K^T and O = P V over them are dense contractions.  They run on
//    the matrix cores through the prefill tile (no causal mask, all rows see
//    every shared key), cut into key splits that write (m, l, o) partials.
//    A group whose rows times query heads fit one 32-row MFMA tile (a few
//    samples or beams of one prompt) takes a streaming 32-row tile instead,
//    which also reads each row's own keys past the shared blocks (its
//    suffix) as further steps, masked to that row.
//  * suffix pass: the remaining blocks of every other row through the
//    decode body, which writes (m, l, acc) partials per partition.
//  * both passes are one launch, prefix workgroups first; a merge launch
//    combines each row's prefix and suffix partials into its output.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <string>
#include <vector>

#include "pa_decode_dev.h"
#include "pa_prefill_dev.h"

namespace pa {

constexpr int kMaxGroups = 64;

// The groups of a launch (those with shared blocks), in the kernel
// arguments, in the order of their first rows.
struct GroupList {
  int32_t n;
  int32_t first_row[kMaxGroups];
  int32_t n_rows[kMaxGroups];
  int32_t shared_blocks[kMaxGroups];
  int32_t splits[kMaxGroups];          // key splits of the group's prefix
  int32_t steps_per_split[kMaxGroups];  // key steps per split (64 or 32 keys)
  // 32-row tile: 32-key steps per row of the rows' own keys past the shared
  // blocks, streamed by the tile after the shared ones; -1: those keys go
  // through the suffix pass.
  int32_t tile_suffix[kMaxGroups];
  int32_t pre_before[kMaxGroups + 1];  // prefix workgroups before group c
  int64_t row_off[kMaxGroups];         // first partial row of group c ([split][row][head] rows)
};

template <typename E, int D, int G, int BS>
__global__ void __launch_bounds__(kPrefillThreads)
    shared_decode_kernel(char* __restrict__ pool_k, char* __restrict__ pool_v, int64_t layer_off,
                         int64_t head_stride, int32_t H_kv, int32_t H_q, float scale_log2, const char* __restrict__ q,
                         const int32_t* __restrict__ block_tables, int32_t max_blocks,
                         const int32_t* __restrict__ context_lens, int32_t blocks_per_part, int32_t num_parts,
                         float* __restrict__ ws_ml, float* __restrict__ ws_acc, float* __restrict__ pre_o,
                         float* __restrict__ pre_ml, int32_t n_pre, GroupList gl) {
  static_assert(8 * G * (D + 2) * sizeof(float) <= sizeof(PrefillLds<D>), "decode merge fits the prefill LDS");
  __shared__ __attribute__((aligned(1024))) PrefillLds<D> lds;
  const int id = blockIdx.x;
  if (id < n_pre) {
    // Prefix: group c, (split, item) with the items of one split adjacent.
    int c = 0;
    while (id >= gl.pre_before[c + 1]) ++c;
    constexpr int TP = kRowsPerWave * kPrefillWaves / G;
    const int n = gl.n_rows[c];
    const int items = (n + TP - 1) / TP * H_kv;
    const int local = id - gl.pre_before[c];
    const int split = local / items;
    const int sps = gl.steps_per_split[c];
    const int key_end = gl.shared_blocks[c] * BS;
    const int64_t roff = gl.row_off[c] + static_cast<int64_t>(split) * n * H_q;
    prefill_tile<E, D, G, BS>(local % items, lds, pool_k, pool_v, layer_off, head_stride,
                              reinterpret_cast<const uint16_t*>(q) + static_cast<int64_t>(gl.first_row[c]) * H_q * D,
                              nullptr, block_tables + static_cast<int64_t>(gl.first_row[c]) * max_blocks, n, H_q,
                              key_end, scale_log2, split * sps, (split + 1) * sps, pre_o + roff * D,
                              pre_ml + roff * 2, key_end);
    return;
  }
  // Suffix: the decode kernel's order (kv head fastest, then the rotated
  // partition slot, then the sequence), past the row's shared blocks.
  const int j = id - n_pre;
  const int g = j % H_kv;
  const int rest = j / H_kv;
  const int b = rest / num_parts;
  int part = rest % num_parts;
  if (num_parts >= 4) {
    part += b & 3;
    if (part >= num_parts) part -= num_parts;
  }
  int skip = 0;
  for (int c = 0; c < gl.n; ++c)
    if (b >= gl.first_row[c] && b < gl.first_row[c] + gl.n_rows[c]) skip = gl.shared_blocks[c];
  decode_body<E, D, G, BS, false, true>(kPrefillWaves, g, part, H_kv, b, reinterpret_cast<float*>(&lds[0][0]), pool_k,
                                        pool_v, layer_off, head_stride, q, nullptr, block_tables, max_blocks,
                                        context_lens, scale_log2, H_q, blocks_per_part, num_parts, ws_ml, ws_acc,
                                        nullptr, nullptr, nullptr, skip);
}

// ----------------------------------------------------- the 32-row prefix tile
// A group whose rows times query heads fit one 32-row MFMA tile (the usual
// case: a few samples or beams of one prompt) reads its shared keys with a
// tile built for streaming rather than for the matrix cores: the pass is
// bound by HBM (each K/V byte feeds only the group's 32 rows), so what
// matters is how many loads are in flight.  A workgroup of 4 waves takes one
// (group, KV head, key split); the waves take every 4th 32-key step of the
// split, each with its next step's K and V in flight in a ring of its own in
// LDS, with no barrier between steps.  Every global load goes straight into
// LDS (global_load_lds_dwordx4) and is waited for by explicit counts, so
// that the compiler's own load tracking never makes a step wait for the
// step behind it.  Each load reads whole 128-byte lines (8 rows of one
// line-wide part), non-temporal, into a swizzled layout on which the MFMA
// operand reads and the transposing V reads stay on distinct banks.  At the
// end the 4 waves merge their (m, l, O) through LDS into one partial.
constexpr int kShWaves = 4;
constexpr int kShThreads = 64 * kShWaves;
constexpr int kShKT = 32;     // keys per step
constexpr int kShStages = 2;  // steps in flight per wave

// LDS layout of a 32-row K, V or q tile: the row's bytes [128 p, 128 p +
// 128) (one 128-byte line of global memory) lie in part p, 4 KiB of 32
// rows x 128 bytes, and inside a row's 128 bytes the 16-byte chunk c sits
// at position c ^ sw(row).  Each direct load fills 8 rows of one part:
// lane l lands at byte 16 l (row 8 i + l / 8, position l % 8), so every
// load reads 8 whole lines of global memory.  The swizzle keeps the MFMA
// operand reads (16 rows, one chunk each, per pass) and the transposing V
// reads (32 lanes: 4 rows x 8 chunk halves per pass) on distinct banks.
template <int D>
struct ShLayout {
  static constexpr int ROWB = D * 2;                 // bytes of a K/V/q row
  static constexpr int TILE = kShKT * ROWB;          // one 32-row tile
  static constexpr int PARTS = ROWB / 128;           // 128-byte parts of a row
  static constexpr int PART = kShKT * 128;           // bytes of one part
  static constexpr int LOADS = TILE / 1024;          // 1 KiB direct loads per tile
  static constexpr int STAGE = 2 * TILE;             // K then V
  static constexpr int RING = kShStages * STAGE;     // one wave's ring
  static constexpr int QOFF = kShWaves * RING;       // the 32 query rows
  static constexpr int BYTES = QOFF + TILE;
  static_assert(PARTS >= 1 && LOADS == 4 * PARTS, "four 8-row loads per part");
  static constexpr int OS = D + 4;                   // floats per row of a wave's staged o (a 16-byte pad:
                                                      // the rows' writes fall on distinct banks)
  static_assert(32 * OS * 4 + 2 * 32 * 4 <= RING, "a wave's (o, m, l) fit its ring");
};
__device__ __forceinline__ int sh_swizzle(int row) {
  const int x = (row >> 1) & 7;  // bit-reversed: rows 2 apart land 4 chunks apart
  return ((x & 1) << 2) | (x & 2) | (x >> 2);
}
// Byte of the tile at which row `row`, byte `b` of the row (16-byte chunk
// units and the offset inside the chunk) is stored.
__device__ __forceinline__ int sh_off(int row, int b) {
  return (b >> 7) * (kShKT * 128) + row * 128 + ((((b >> 4) & 7) ^ sh_swizzle(row)) << 4) + (b & 15);
}

// global_load_lds_dwordx4 with the non-temporal bit: K and V of the tile are
// read once per launch, and every 128-byte line by one load.
__device__ __forceinline__ void load_to_lds_stream(const char* src, char* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "{m0}"(m0) : "memory");
#endif
}

// s_waitcnt vmcnt(n), expcnt and lgkmcnt at their maxima (gfx9 encoding).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Steps of a group: P = ceil(S / 32) steps over the shared keys [0, S),
// all rows' (table: the group's first row), then, with U >= 0, U steps per
// row over its own keys [S, S + 32 U) (table: that row's; keys at or past
// its length are masked, and rows of the other samples see none of them).
// The tile takes steps [v_lo, v_hi).
template <typename E, int D, int G, int BS>
__device__ __forceinline__ void prefix_tile32(int g, int n_rows, int v_lo, int v_hi, int S, int U,
                                              char* __restrict__ lds, const char* __restrict__ pool_k,
                                              const char* __restrict__ pool_v, int64_t layer_off, int64_t head_stride,
                                              const char* __restrict__ q, const int32_t* __restrict__ table,
                                              int32_t max_blocks, const int32_t* __restrict__ lens, int32_t H_q,
                                              float scale_log2, float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  using M = Mfma<E>;
  using vec = typename M::vec;
  using L = ShLayout<D>;
  constexpr int KT = kShKT;
  constexpr int KS = D / 16;  // QK k-steps over the head dim
  constexpr int DT = D / 32;  // 32-dim output tiles
  constexpr int LPS = 2 * L::LOADS;  // direct loads per step (K and V)
  static_assert(BS >= 8, "at most two blocks per 16-row group");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int li = lane & 31;
  const int h = lane >> 5;
  const int rows = n_rows * G;  // live query rows: (sample r / G, head g * G + r % G)

  const char* kbase = pool_k + layer_off + static_cast<int64_t>(g) * head_stride;
  const char* vbase = pool_v + layer_off + static_cast<int64_t>(g) * head_stride;
  char* ring = lds + wave * L::RING;
  char* qt = lds + L::QOFF;

  // Direct loads: load (p, i) of a tile fills rows 8 i + [0, 8) of part p;
  // lane l takes row 8 i + l / 8 and the row's chunk 8 p + ((l % 8) ^
  // sw(row)), which lands at byte 16 l of the load's 1 KiB.
  const int lrow = lane >> 3;
  auto chunk_byte = [&](int row, int p) { return p * 128 + (((lane & 7) ^ sh_swizzle(row)) << 4); };

  // The 32 query rows, loaded once per workgroup: wave w issues loads
  // w, w + 4, ... of the q tile.  Rows past the group's are clamped (never
  // stored).
#pragma unroll
  for (int n = wave; n < L::LOADS; n += kShWaves) {
    const int p = n / 4, i = n % 4;
    const int r = min(i * 8 + lrow, rows - 1);
    const char* src = q + ((static_cast<int64_t>(r / G) * H_q + g * G + r % G) * D) * 2 + chunk_byte(i * 8 + lrow, p);
    load_to_lds(src, qt + p * L::PART + i * 1024);
  }

  // Steps of this wave: steps v_lo + wave, v_lo + wave + 4, ... (an index
  // past the wave's last is clamped to it; no loads are issued for it).
  const int nsteps = v_hi - v_lo;
  const int nw = nsteps > wave ? (nsteps - wave + kShWaves - 1) / kShWaves : 0;
  const int P = (S + KT - 1) / KT;
  const int Us = max(U, 1);
  auto v_of = [&](int j) { return v_lo + wave + min(j, nw - 1) * kShWaves; };
  // A step's first key and key limit, and its table row (-1: the shared
  // keys) -- all wave-uniform.
  auto row_of = [&](int v) { return v < P ? -1 : (v - P) / Us; };
  auto key0_of = [&](int v) { return v < P ? v * KT : S + (v - P) % Us * KT; };
  const int32_t spare = table[0];  // a block of the group: loads past a row's end read it, unused
  struct Step {
    int32_t b[2][2];  // [row group][rows 0-7 / 8-15]
    int32_t k0, lim;  // first key; keys at or past lim are not the step's
  };
  // The step's table entries and the row's length (scalar loads, waited
  // for with the LDS reads of a later step).  Entries are read at their
  // index clamped to the table; one past the row's length is never used.
  auto fetch = [&](int j) __attribute__((always_inline)) {
    Step st;
    const int v = v_of(j);
    const int row = row_of(v);
    st.k0 = key0_of(v);
    st.lim = row < 0 ? S : lens[row];
    const int32_t* tab = table + static_cast<int64_t>(max(row, 0)) * max_blocks;
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      st.b[rg][0] = tab[min((st.k0 + rg * 16) / BS, max_blocks - 1)];
      st.b[rg][1] = BS >= 16 ? st.b[rg][0] : tab[min((st.k0 + rg * 16 + 8) / BS, max_blocks - 1)];
    }
    return st;
  };
  auto issue = [&](const Step& st, int slot) __attribute__((always_inline)) {
    char* kt = ring + slot * L::STAGE;
    char* vt = kt + L::TILE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // A load's 8 rows sit in one block (S is a multiple of the block
      // size, steps start 32 keys apart): past the limit, the spare.
      const bool past = st.k0 + i * 8 >= st.lim;
      const int key = past ? 0 : min(st.k0 + i * 8 + lrow, st.lim - 1);
      const int64_t blk = past ? spare : st.b[i >> 1][i & 1];
      const int64_t off = (blk * BS + (key & (BS - 1))) * L::ROWB;
#pragma unroll
      for (int p = 0; p < L::PARTS; ++p) {
        const int cb = chunk_byte(i * 8 + lrow, p);
        load_to_lds_stream(kbase + off + cb, kt + p * L::PART + i * 1024);
        load_to_lds_stream(vbase + off + cb, vt + p * L::PART + i * 1024);
      }
    }
  };

  // The key limit the next step computed needs, loaded a step ahead.  Every
  // value loaded here is used once, in the next iteration, and reloaded
  // only after that use: a value carried further would make the loop wait
  // for the scalar loads it has just issued.
  auto lim_of = [&](int j) __attribute__((always_inline)) {
    const int row = row_of(v_of(j));
    return row < 0 ? S : lens[row];
  };
  Step next{};
  int limc = 0;
  if (nw > 0) {
    issue(fetch(0), 0);
    if (nw > 1) issue(fetch(1), 1);
    next = fetch(2);
    limc = lim_of(0);
  }
  // q landed (each wave waits for its own q loads; the steps behind them may
  // stay in flight), then the workgroup's q loads are all visible.
  if (nw > 1) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LPS));
  } else if (nw == 1) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPS));
  } else {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  }
  barrier_keep_loads();

  // MFMA operand of K and q: row li, chunk 2 ks + h, at a per-lane offset
  // for each ks % 4 plus part ks / 4.
  vec qb[KS];
  int kb[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) kb[k] = sh_off(li, (2 * k + h) * 16);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qb[ks] = *reinterpret_cast<const vec*>(qt + (ks >> 2) * L::PART + kb[ks & 3]);
  // Transposing V reads of a 16-key slice s2 and dims dt * 32 + [0, 32):
  // this lane, as source lane 4 k4 + q4 of its 16-lane group g16, addresses
  // 4 dims of row s2 * 16 + vrow (+ 8), at a per-lane offset for each
  // (row half, dt % 2) plus part dt / 2 and 16 rows per s2.
  const int g16 = lane >> 4, k4 = (lane >> 2) & 3, q4 = lane & 3;
  const int vrow = 4 * (g16 >> 1) + k4, vch = (g16 & 1) * 2 + (q4 >> 1);
  int vb[2][2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2) vb[hi][d2] = sh_off(vrow + 8 * hi, d2 * 64 + vch * 16 + (q4 & 1) * 8);

  float m = -INFINITY, lsum = 0.0f;
  floatx16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = floatx16_t{};
  const float c = scale_log2 > 0.0f ? scale_log2 : 1.0f;

  for (int j = 0; j < nw; ++j) {
    const int slot = j & 1;
    const char* kt = ring + slot * L::STAGE;
    const char* vt = kt + L::TILE;
    // step j has landed; step j + 1 (LPS loads), if any, may still be in
    // flight
    if (j + 1 < nw) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPS));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    vec ka[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[ks] = *reinterpret_cast<const vec*>(kt + (ks >> 2) * L::PART + kb[ks & 3]);
    vec va[2][DT];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const char* vs = vt + s2 * 16 * 128 + (dt >> 1) * L::PART;
        const uint2 lo = lds_read_tr(vs + vb[0][dt & 1]);
        const uint2 hi = lds_read_tr(vs + vb[1][dt & 1]);
        va[s2][dt] = __builtin_bit_cast(vec, make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
    // Every read of this slot is back before its refill (step j + 2) lands
    // in it.  A wave's last two steps refill nothing, so a step's wait
    // above leaves one step in flight, or none at the last.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
    if (j + 2 < nw) issue(next, slot);
    next = fetch(j + 3);
    __builtin_amdgcn_sched_barrier(0);
    const int lim = limc;
    const int vj = v_of(j);
    const int key0 = key0_of(vj);
    if (key0 < lim) {  // uniform: not a step wholly past its row's length
      floatx16_t st = floatx16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) st = M::mma(ka[ks], qb[ks], st);
      // online softmax of this step's 32 keys (lane: 16 keys of row li, the
      // other 16 in lane li + 32): log2 domain, scale folded into the exponent
      if (scale_log2 <= 0.0f) st *= scale_log2;
      const int row = row_of(vj);
      if (row >= 0 || key0 + KT > lim) {  // uniform: a row's own keys, or a partial step
        const bool mine = row < 0 || li / G == row;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!mine || key0 + 8 * (i >> 2) + 4 * h + (i & 3) >= lim) st[i] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, st[v]);
      mx = max_halves(mx);
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
      vec pb[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        uint16_t hh[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(st[8 * s2 + i], c, -ms));
          lsum += p;
          hh[i] = M::cvt(p);
        }
        pb[s2] = __builtin_bit_cast(vec, make_uint4(hh[0] | (uint32_t(hh[1]) << 16), hh[2] | (uint32_t(hh[3]) << 16),
                                                    hh[4] | (uint32_t(hh[5]) << 16), hh[6] | (uint32_t(hh[7]) << 16)));
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] = M::mma(va[s2][dt], pb[s2], o[dt]);
    }
    __builtin_amdgcn_sched_barrier(0);
    limc = lim_of(j + 1);
  }

  // Merge the 4 waves through LDS (each wave's ring, once its own loads
  // have all landed): o as [32 rows][D] fp32, rows L::OS floats apart, then
  // m and l per row.
  const float lt = sum_halves(lsum);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  float* wo = reinterpret_cast<float*>(ring);
  float* wm = wo + 32 * L::OS;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      *reinterpret_cast<float4*>(wo + li * L::OS + dt * 32 + 8 * jj + 4 * h) =
          make_float4(o[dt][4 * jj], o[dt][4 * jj + 1], o[dt][4 * jj + 2], o[dt][4 * jj + 3]);
  if (h == 0) {
    wm[li] = m;
    wm[32 + li] = lt;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < rows * D; idx += kShThreads) {
    const int r = idx / D, e = idx % D;
    float mw[kShWaves], mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kShWaves; ++w) {
      mw[w] = reinterpret_cast<const float*>(lds + w * L::RING)[32 * L::OS + r];
      mx = fmaxf(mx, mw[w]);
    }
    const float msafe = (mx == -INFINITY) ? 0.0f : mx;
    float acc = 0.0f, lw = 0.0f;
#pragma unroll
    for (int w = 0; w < kShWaves; ++w) {
      const float* base = reinterpret_cast<const float*>(lds + w * L::RING);
      const float wt = __builtin_amdgcn_exp2f(mw[w] - msafe);
      acc += base[r * L::OS + e] * wt;
      lw += base[32 * L::OS + 32 + r] * wt;
    }
    const int64_t row = static_cast<int64_t>(r / G) * H_q + g * G + r % G;
    ws_o[row * D + e] = acc;
    if (e == 0) *reinterpret_cast<float2*>(ws_ml + 2 * row) = make_float2(mx, lw);
  }
}

// Prefix tiles of 32 rows (groups whose rows times query heads fit one MFMA
// tile) and the suffix decode, 4 waves per workgroup.  Workgroup i takes
// prefix item i (group, KV head, split) if there is one, then the suffix
// items i, i + grid, i + 2 grid, ... in the decode kernel's order over the
// rows whose suffix the tile does not stream: a workgroup's LDS takes most
// of a CU, so a suffix item of a few blocks launched as a workgroup of its
// own would hold a CU for a whole dispatch.
template <typename E, int D, int G, int BS>
__global__ void __launch_bounds__(kShThreads)
    shared_decode32_kernel(char* __restrict__ pool_k, char* __restrict__ pool_v, int64_t layer_off,
                           int64_t head_stride, int32_t H_kv, int32_t H_q, float scale_log2, const char* __restrict__ q,
                           const int32_t* __restrict__ block_tables, int32_t max_blocks,
                           const int32_t* __restrict__ context_lens, int32_t blocks_per_part, int32_t num_parts,
                           float* __restrict__ ws_ml, float* __restrict__ ws_acc, float* __restrict__ pre_o,
                           float* __restrict__ pre_ml, int32_t n_pre, int32_t n_dec, GroupList gl) {
  static_assert(kShWaves * G * (D + 2) * sizeof(float) <= ShLayout<D>::BYTES, "decode merge fits the LDS");
  __shared__ __attribute__((aligned(1024))) char lds[ShLayout<D>::BYTES];
  const int id = blockIdx.x;
  if (id < n_pre) {
    int c = 0;
    while (id >= gl.pre_before[c + 1]) ++c;
    const int local = id - gl.pre_before[c];
    const int g = local % H_kv;  // KV head fastest: the heads of one split spread over the XCDs
    const int split = local / H_kv;
    const int n = gl.n_rows[c];
    const int S = gl.shared_blocks[c] * BS;
    const int U = gl.tile_suffix[c];
    const int steps = (S + kShKT - 1) / kShKT + (U > 0 ? n * U : 0);
    const int v_lo = split * gl.steps_per_split[c];
    const int v_hi = min(steps, v_lo + gl.steps_per_split[c]);
    const int64_t roff = gl.row_off[c] + static_cast<int64_t>(split) * n * H_q;
    prefix_tile32<E, D, G, BS>(g, n, v_lo, v_hi, S, U, lds, pool_k, pool_v, layer_off, head_stride,
                               q + static_cast<int64_t>(gl.first_row[c]) * H_q * D * 2,
                               block_tables + static_cast<int64_t>(gl.first_row[c]) * max_blocks, max_blocks,
                               context_lens + gl.first_row[c], H_q, scale_log2, pre_o + roff * D, pre_ml + roff * 2);
  }
  for (int j = id; j < n_dec; j += gridDim.x) {
    __syncthreads();  // the previous tile's or item's last LDS reads are done
    const int g = j % H_kv;
    const int rest = j / H_kv;
    // the (rest / num_parts)-th row outside the groups whose suffix the
    // tile streams (groups in row order)
    int b = rest / num_parts;
    for (int c = 0; c < gl.n; ++c)
      if (gl.tile_suffix[c] >= 0 && b >= gl.first_row[c]) b += gl.n_rows[c];
    int part = rest % num_parts;
    if (num_parts >= 4) {
      part += b & 3;
      if (part >= num_parts) part -= num_parts;
    }
    int skip = 0;
    for (int c = 0; c < gl.n; ++c)
      if (b >= gl.first_row[c] && b < gl.first_row[c] + gl.n_rows[c]) skip = gl.shared_blocks[c];
    decode_body<E, D, G, BS, false, true>(kShWaves, g, part, H_kv, b, reinterpret_cast<float*>(lds), pool_k, pool_v,
                                          layer_off, head_stride, q, nullptr, block_tables, max_blocks, context_lens,
                                          scale_log2, H_q, blocks_per_part, num_parts, ws_ml, ws_acc, nullptr,
                                          nullptr, nullptr, skip);
  }
}

// Combines each (sequence, query head)'s partials: the prefix splits of its
// group (if any) and the suffix partitions that hold some of its blocks:
// out = sum_k o_k 2^(m_k - M) / sum_k l_k 2^(m_k - M), M = max_k m_k.  Every
// load is issued before any result is used -- each thread's first kPre
// partial outputs and one partial's (m, l) -- so the merge waits for one
// memory round trip; the weights go through LDS.
template <typename E, int D>
__global__ void __launch_bounds__(D)
    shared_merge_kernel(void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
                        const float* __restrict__ pre_o, const float* __restrict__ pre_ml,
                        const int32_t* __restrict__ context_lens, int32_t H_q, int32_t H_kv, int32_t xcd_order,
                        int32_t num_parts, int32_t blocks_per_part, int32_t bs, GroupList gl) {
  extern __shared__ float wt[];  // [max splits + num_parts] weights
  __shared__ float red[2];
  const int64_t bh = xcd_order ? merge_row(blockIdx.x, H_q, H_kv) : blockIdx.x;
  const int b = static_cast<int>(bh / H_q);
  const int hd = static_cast<int>(bh % H_q);
  const int e = threadIdx.x;
  int c = -1;
  for (int k = 0; k < gl.n; ++k)
    if (b >= gl.first_row[k] && b < gl.first_row[k] + gl.n_rows[k]) c = k;
  const int skip = c >= 0 ? gl.shared_blocks[c] : 0;
  const int ns = c >= 0 ? gl.splits[c] : 0;
  // a row whose suffix the 32-row tile streamed has its splits only
  const bool streamed = c >= 0 && gl.tile_suffix[c] >= 0;
  const int nblk = streamed ? 0 : (context_lens[b] + bs - 1) / bs;
  const int np = streamed ? 0 : max(0, min(num_parts, (nblk - skip + blocks_per_part - 1) / blocks_per_part));
  const int nk = ns + np;
  // partial k: prefix split k (k < ns) or suffix partition k - ns
  const int64_t prow0 = c >= 0 ? gl.row_off[c] + static_cast<int64_t>(b - gl.first_row[c]) * H_q + hd : 0;
  const int64_t pstride = c >= 0 ? static_cast<int64_t>(gl.n_rows[c]) * H_q : 0;  // rows per split
  auto row_of = [&](int k) { return k < ns ? prow0 + k * pstride : bh * num_parts + (k - ns); };
  auto o_of = [&](int k) { return k < ns ? pre_o[row_of(k) * D + e] : ws_acc[row_of(k) * D + e]; };
  constexpr int kPre = 16;
  float pre[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) pre[i] = i < nk ? o_of(i) : 0.0f;
  float2 ml = make_float2(kNegInf, 0.0f);
  if (e < nk) {
    const float* src = e < ns ? pre_ml : ws_ml;
    ml = *reinterpret_cast<const float2*>(src + 2 * row_of(e));
  }
  float mx = ml.x;
  for (int k = e + D; k < nk; k += D) mx = fmaxf(mx, (k < ns ? pre_ml : ws_ml)[2 * row_of(k)]);
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((e & 63) == 0) red[e >> 6] = mx;
  __syncthreads();
  mx = D > 64 ? fmaxf(red[0], red[1]) : red[0];
  const float ms = (mx == kNegInf) ? 0.0f : mx;
  float lsum = 0.0f;
  if (e < nk) {
    const float w = exp2_fast(ml.x - ms);
    wt[e] = w;
    lsum = ml.y * w;
  }
  for (int k = e + D; k < nk; k += D) {
    const float* src = (k < ns ? pre_ml : ws_ml) + 2 * row_of(k);
    const float w = exp2_fast(src[0] - ms);
    wt[k] = w;
    lsum += src[1] * w;
  }
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);
  __syncthreads();
  if ((e & 63) == 0) red[e >> 6] = lsum;
  __syncthreads();
  const float lt = D > 64 ? red[0] + red[1] : red[0];
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int i = 0; i < kPre; i += 2) {
    if (i < nk) a0 += pre[i] * wt[i];
    if (i + 1 < nk) a1 += pre[i + 1] * wt[i + 1];
  }
  for (int k = kPre; k < nk; ++k) a0 += o_of(k) * wt[k];
  store_elem(E{}, out, bh * D + e, lt > 0.0f ? (a0 + a1) / lt : 0.0f);
}

// ------------------------------------------------------------------ host

struct SharedPlan {
  DecodePlan dec;
  GroupList gl;
  int32_t n_pre;
  int64_t pre_rows;  // prefix partial rows (sum over groups of splits * n_rows * H_q)
  int32_t max_splits;
  int32_t loose_rows;  // rows whose suffix goes through the suffix pass
  bool tile32;         // every group fits one 32-row tile: the streaming prefix tile
};

// Host checks of a group list and the launch plan (PA_OK or an error).
static int plan_shared(const std::string& w, const pa_kv_pool* pool, int32_t B, int32_t H_q, int32_t max_ctx,
                       int32_t max_blocks, const pa_share_group* groups, int32_t n_groups, SharedPlan* p) {
  if (n_groups < 0 || n_groups > kMaxGroups)
    return fail(PA_EINVAL, w + ": n_groups must be in [0, " + std::to_string(kMaxGroups) + "]");
  if (n_groups > 0 && !groups) return fail(PA_EINVAL, w + ": NULL groups");
  const int G = H_q / pool->num_kv_heads;
  const int bs = pool->block_size;
  std::vector<std::pair<int, int>> spans;
  for (int c = 0; c < n_groups; ++c) {
    const pa_share_group& gr = groups[c];
    if (gr.first_row < 0 || gr.n_rows < 1 || static_cast<int64_t>(gr.first_row) + gr.n_rows > B)
      return fail(PA_EINVAL, w + ": group " + std::to_string(c) + " rows outside the batch");
    if (gr.shared_blocks < 0 || gr.shared_blocks > max_blocks ||
        static_cast<int64_t>(gr.shared_blocks) * bs > max_ctx)
      return fail(PA_EINVAL, w + ": group " + std::to_string(c) + " shared_blocks out of range");
    spans.emplace_back(gr.first_row, gr.first_row + gr.n_rows);
  }
  std::sort(spans.begin(), spans.end());
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i].first < spans[i - 1].second) return fail(PA_EINVAL, w + ": groups overlap");

  // Groups of at most 32 query rows per KV head (rows times query heads)
  // take the streaming 32-row tile; any larger group sends the whole launch
  // through the prefill tile.
  p->tile32 = pool->head_dim == 128 || pool->head_dim == 64;
  for (int c = 0; c < n_groups; ++c)
    if (groups[c].shared_blocks > 0 && static_cast<int64_t>(groups[c].n_rows) * G > 32) p->tile32 = false;
  p->dec = plan_decode(B, pool->num_kv_heads, G, bs, max_ctx);
  p->dec.waves = p->tile32 ? kShWaves : kPrefillWaves;  // the fused kernel's workgroup size
  if (p->dec.num_parts > 65535) return fail(PA_EINVAL, w + ": too many partitions for the grid");
  // Groups with shared blocks, in row order.  The 32-row tile also streams
  // a group's own keys past the shared blocks, U = ceil((max_ctx - S) / 32)
  // steps per row (a bound: a row's steps past its length are skipped), when
  // those are at most as many as its shared steps; otherwise, and for the
  // prefill tile, they go through the suffix pass.
  std::vector<int> order;
  for (int c = 0; c < n_groups; ++c)
    if (groups[c].shared_blocks > 0) order.push_back(c);
  std::sort(order.begin(), order.end(),
            [&](int a, int b2) { return groups[a].first_row < groups[b2].first_row; });
  const int KT = p->tile32 ? kShKT : kKeysPerStep;
  const int TP = p->tile32 ? 32 / G : kRowsPerWave * kPrefillWaves / G;
  std::vector<int64_t> steps(order.size());
  std::vector<int32_t> tile_suffix(order.size(), -1);
  int64_t item_steps = 0;
  int64_t loose = B;
  for (size_t k = 0; k < order.size(); ++k) {
    const pa_share_group& gr = groups[order[k]];
    const int64_t S = static_cast<int64_t>(gr.shared_blocks) * bs;
    steps[k] = ceil_div(S, KT);
    const int64_t U = ceil_div(std::max<int64_t>(0, max_ctx - S), kShKT);
    if (p->tile32 && gr.n_rows * U <= steps[k]) {
      tile_suffix[k] = static_cast<int32_t>(U);
      steps[k] += gr.n_rows * U;
      loose -= gr.n_rows;
    }
    item_steps += ceil_div(gr.n_rows, TP) * pool->num_kv_heads * steps[k];
  }
  // Key splits.  Prefill tile: about two workgroups per CU, at least two
  // 64-key steps each.  32-row tile: about one workgroup per CU (its LDS
  // holds one), at least one 32-key step per wave.
  const int64_t target = (p->tile32 ? 1 : 2) * static_cast<int64_t>(device_cus());
  const int sps = static_cast<int>(std::max<int64_t>(p->tile32 ? kShWaves : 2, ceil_div(item_steps, target)));
  GroupList& gl = p->gl;
  gl = GroupList{};
  gl.pre_before[0] = 0;
  int64_t pre = 0, rows = 0;
  int max_splits = 0;
  for (size_t k = 0; k < order.size(); ++k) {
    const pa_share_group& gr = groups[order[k]];
    gl.n = static_cast<int32_t>(k + 1);
    gl.first_row[k] = gr.first_row;
    gl.n_rows[k] = gr.n_rows;
    gl.shared_blocks[k] = gr.shared_blocks;
    gl.steps_per_split[k] = sps;
    gl.tile_suffix[k] = tile_suffix[k];
    gl.splits[k] = static_cast<int32_t>(ceil_div(steps[k], sps));
    gl.row_off[k] = rows;
    rows += static_cast<int64_t>(gl.splits[k]) * gr.n_rows * H_q;
    pre += ceil_div(gr.n_rows, TP) * pool->num_kv_heads * gl.splits[k];
    gl.pre_before[k + 1] = static_cast<int32_t>(std::min<int64_t>(pre, INT32_MAX));
    max_splits = std::max(max_splits, gl.splits[k]);
  }
  const int64_t n_dec = static_cast<int64_t>(pool->num_kv_heads) * p->dec.num_parts * loose;
  if (pre + n_dec > INT32_MAX) return fail(PA_EINVAL, w + ": grid too large");
  p->n_pre = static_cast<int32_t>(pre);
  p->pre_rows = rows;
  p->max_splits = max_splits;
  p->loose_rows = static_cast<int32_t>(loose);
  return PA_OK;
}

static size_t shared_ws_bytes(const SharedPlan& p, int32_t B, int32_t H_q, int D) {
  return (static_cast<size_t>(p.pre_rows) + static_cast<size_t>(B) * H_q * p.dec.num_parts) * (D + 2) *
         sizeof(float);
}

using SharedFn = void (*)(const pa_kv_pool*, int32_t, void*, const void*, int32_t, int32_t, const int32_t*, int32_t,
                          const int32_t*, float, const SharedPlan&, float*, hipStream_t);

template <typename E, int D, int G, int BS>
static void launch_shared(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t B, int32_t H_q,
                          const int32_t* bt, int32_t max_blocks, const int32_t* ctx, float scale_log2,
                          const SharedPlan& p, float* ws, hipStream_t stream) {
  const int64_t head_stride = static_cast<int64_t>(pool->num_blocks) * BS * D * 2;
  const int64_t layer_off = static_cast<int64_t>(layer) * pool->num_kv_heads * head_stride;
  // Workspace: prefix o [rows][D] first (its 16-byte stores need the
  // caller's 16-byte alignment), prefix (m, l) [rows][2], then the suffix's
  // acc [B][H_q][P][D] and (m, l) [B][H_q][P][2].
  const int64_t dec_rows = static_cast<int64_t>(B) * H_q * p.dec.num_parts;
  float* pre_o = ws;
  float* pre_ml = pre_o + p.pre_rows * D;
  float* ws_acc = pre_ml + p.pre_rows * 2;
  float* ws_ml = ws_acc + dec_rows * D;
  const int64_t n_dec = static_cast<int64_t>(pool->num_kv_heads) * p.dec.num_parts * p.loose_rows;
  if (p.tile32) {
    // One workgroup per prefix item, at least one per CU while suffix items
    // remain; the suffix items are spread over them.
    const int64_t grid = std::max<int64_t>(p.n_pre, std::min<int64_t>(n_dec, device_cus()));
    if (grid > 0)
      hipLaunchKernelGGL((shared_decode32_kernel<E, D, G, BS>), dim3(static_cast<uint32_t>(grid)), dim3(kShThreads),
                         0, stream, static_cast<char*>(pool->k), static_cast<char*>(pool->v), layer_off, head_stride,
                         pool->num_kv_heads, H_q, scale_log2, static_cast<const char*>(q), bt, max_blocks, ctx,
                         p.dec.blocks_per_part, p.dec.num_parts, ws_ml, ws_acc, pre_o, pre_ml, p.n_pre,
                         static_cast<int32_t>(n_dec), p.gl);
  } else {
    hipLaunchKernelGGL((shared_decode_kernel<E, D, G, BS>), dim3(static_cast<uint32_t>(p.n_pre + n_dec)),
                       dim3(kPrefillThreads), 0, stream, static_cast<char*>(pool->k), static_cast<char*>(pool->v),
                       layer_off, head_stride, pool->num_kv_heads, H_q, scale_log2, static_cast<const char*>(q), bt,
                       max_blocks, ctx, p.dec.blocks_per_part, p.dec.num_parts, ws_ml, ws_acc, pre_o, pre_ml,
                       p.n_pre, p.gl);
  }
  const size_t lds = (p.max_splits + p.dec.num_parts) * sizeof(float);
  hipLaunchKernelGGL((shared_merge_kernel<E, D>), dim3(static_cast<uint32_t>(B) * H_q), dim3(D), lds, stream, out,
                     ws_ml, ws_acc, pre_o, pre_ml, ctx, H_q, pool->num_kv_heads,
                     static_cast<int64_t>(shared_ws_bytes(p, B, H_q, D)) <= kMergeFromL2Bytes, p.dec.num_parts,
                     p.dec.blocks_per_part, BS, p.gl);
}

template <typename E, int D, int G>
static SharedFn shared_bs(int bs) {
  switch (bs) {
    case 8: return &launch_shared<E, D, G, 8>;
    case 16: return &launch_shared<E, D, G, 16>;
    case 32: return &launch_shared<E, D, G, 32>;
  }
  return nullptr;
}
template <typename E, int D>
static SharedFn shared_g(int G, int bs) {
  switch (G) {
    case 1: return shared_bs<E, D, 1>(bs);
    case 2: return shared_bs<E, D, 2>(bs);
    case 4: return shared_bs<E, D, 4>(bs);
    case 8: return shared_bs<E, D, 8>(bs);
  }
  return nullptr;
}
template <typename E>
static SharedFn shared_d(int D, int G, int bs) {
  switch (D) {
    case 64: return shared_g<E, 64>(G, bs);
    case 128: return shared_g<E, 128>(G, bs);
  }
  return nullptr;
}

}  // namespace pa

extern "C" size_t pa_decode_shared_workspace_size(const pa_kv_pool* pool, int32_t B, int32_t H_q, int32_t max_ctx,
                                                  const pa_share_group* groups, int32_t n_groups) {
  using namespace pa;
  if (!pool || B <= 0 || H_q <= 0 || pool->num_kv_heads <= 0 || pool->block_size <= 0 || H_q % pool->num_kv_heads)
    return 0;
  SharedPlan p;
  const int32_t max_blocks = static_cast<int32_t>(ceil_div(std::max(max_ctx, 1), pool->block_size));
  if (plan_shared("pa_decode_shared_workspace_size", pool, B, H_q, max_ctx, max_blocks, groups, n_groups, &p))
    return 0;
  return shared_ws_bytes(p, B, H_q, pool->head_dim);
}

extern "C" int pa_decode_shared(const pa_kv_pool* pool, int32_t layer, void* out, const void* q, int32_t B,
                                int32_t H_q, const int32_t* block_tables, int32_t max_blocks,
                                const int32_t* context_lens, int32_t max_ctx, const pa_share_group* groups,
                                int32_t n_groups, float scale, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  using namespace pa;
  const std::string w("pa_decode_shared");
  if (int e = validate_decode(w, pool, layer, out, q, B, H_q, block_tables, max_blocks, context_lens, max_ctx))
    return e;
  if (B == 0) return PA_OK;
  const int G = H_q / pool->num_kv_heads;
  SharedFn fn = nullptr;
  if (pool->dtype == PA_BF16) fn = shared_d<BF16>(pool->head_dim, G, pool->block_size);
  if (pool->dtype == PA_F16) fn = shared_d<F16>(pool->head_dim, G, pool->block_size);
  if (!fn) return fail(PA_ENOTSUP, w + ": needs a bf16/f16 pool, head_dim 64/128, block 8/16/32, H_q/H_kv in {1,2,4,8}");
  SharedPlan p;
  if (int e = plan_shared(w, pool, B, H_q, max_ctx, max_blocks, groups, n_groups, &p)) return e;
  const size_t need = shared_ws_bytes(p, B, H_q, pool->head_dim);
  if (!workspace || workspace_bytes < need)
    return fail(PA_ESPACE, w + ": workspace of " + std::to_string(need) + " bytes needed");
  if (reinterpret_cast<uintptr_t>(workspace) & 15u) return fail(PA_EINVAL, w + ": workspace must be 16-byte aligned");
  if (validate_on()) {
    if (int e = check_decode_indices(w, pool, B, block_tables, max_blocks, context_lens, max_ctx, nullptr, stream))
      return e;
    if (int e = check_share_groups(w, pool, B, block_tables, max_blocks, context_lens, groups, n_groups, stream))
      return e;
  }
  const float scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  fn(pool, layer, out, q, B, H_q, block_tables, max_blocks, context_lens, scale_log2, p, static_cast<float*>(workspace),
     stream);
  return check_launch("pa_decode_shared");
}

extern "C" int pa_share_groups(const int32_t* block_tables, int32_t B, int32_t max_blocks,
                               const int32_t* context_lens, int32_t block_size, int32_t min_rows, int32_t min_blocks,
                               pa_share_group* out, int32_t cap, int32_t* n_out) {
  using namespace pa;
  if (B < 0 || max_blocks < 0 || block_size <= 0 || min_rows < 2 || min_blocks < 1 || cap < 0 || !n_out ||
      (B > 0 && (!block_tables || !context_lens)) || (cap > 0 && !out))
    return fail(PA_EINVAL, "pa_share_groups: bad argument");
  // Full blocks of row r that its context covers (padding never counts).
  auto full = [&](int r) {
    return std::min<int64_t>(max_blocks, std::max(0, context_lens[r]) / block_size);
  };
  int n = 0;
  int i = 0;
  while (i < B) {
    const int32_t* ti = block_tables + static_cast<int64_t>(i) * max_blocks;
    int64_t k = full(i);
    int j = i + 1;
    // Greedy: extend the run while its rows keep >= min_blocks common
    // leading blocks.
    while (j < B) {
      const int32_t* tj = block_tables + static_cast<int64_t>(j) * max_blocks;
      int64_t kk = std::min(k, full(j)), m = 0;
      while (m < kk && tj[m] == ti[m]) ++m;
      if (m < min_blocks) break;
      k = m;
      ++j;
    }
    if (j - i >= min_rows && k >= min_blocks) {
      if (n >= cap) return fail(PA_ESPACE, "pa_share_groups: more groups than cap");
      out[n++] = pa_share_group{i, j - i, static_cast<int32_t>(k)};
      i = j;
    } else {
      ++i;
    }
  }
  *n_out = n;
  return PA_OK;
}
