// Validate mode: the device-side indices every entry point trusts (block
// ids, slots, copy pairs, context lengths) are copied to the host on the
// call's stream and checked before anything is launched.  Off by default;
// PA_VALIDATE=1 in the environment at load time or pa_set_validate(1) turns
// it on.  The copies synchronise the stream, so the mode is for debugging
// and cannot run under graph capture.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdlib>
#include <string>
#include <unordered_set>
#include <vector>

#include "pa_host.h"

namespace pa {

static std::atomic<int> g_validate{-1};

bool validate_on() {
  int v = g_validate.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* s = std::getenv("PA_VALIDATE");
    v = (s && *s && std::atoi(s) != 0) ? 1 : 0;
    g_validate.store(v, std::memory_order_relaxed);
  }
  return v != 0;
}

static int fetch(const std::string& who, const int32_t* dev, size_t n, std::vector<int32_t>& host,
                 hipStream_t stream) {
  host.resize(n);
  if (n == 0) return PA_OK;
  hipError_t e = hipMemcpyAsync(host.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(PA_EHIP, who + ": validate copy failed: " + hipGetErrorString(e));
  return PA_OK;
}

int check_slots(const std::string& who, const pa_kv_pool* pool, const int32_t* slots, int32_t T,
                hipStream_t stream) {
  std::vector<int32_t> h;
  if (int e = fetch(who, slots, T, h, stream)) return e;
  const int64_t n_slots = static_cast<int64_t>(pool->num_blocks) * pool->block_size;
  std::unordered_set<int32_t> seen;
  for (int32_t t = 0; t < T; ++t) {
    if (h[t] < 0) continue;
    if (h[t] >= n_slots) return fail(PA_EINVAL, who + ": slot " + std::to_string(h[t]) + " out of range");
    if (!seen.insert(h[t]).second) return fail(PA_EINVAL, who + ": slot " + std::to_string(h[t]) + " repeated");
  }
  return PA_OK;
}

int check_pairs(const std::string& who, const pa_kv_pool* pool, const int32_t* pairs, int32_t n, hipStream_t stream) {
  std::vector<int32_t> h;
  if (int e = fetch(who, pairs, 2 * static_cast<size_t>(n), h, stream)) return e;
  std::unordered_set<int32_t> dst, src;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = h[2 * i], d = h[2 * i + 1];
    if (s < 0 || s >= pool->num_blocks || d < 0 || d >= pool->num_blocks)
      return fail(PA_EINVAL, who + ": pair " + std::to_string(i) + " has a block id out of range");
    if (s == d || !dst.insert(d).second) return fail(PA_EINVAL, who + ": destination " + std::to_string(d) + " reused");
    src.insert(s);
  }
  for (int32_t d : dst)
    if (src.count(d)) return fail(PA_EINVAL, who + ": block " + std::to_string(d) + " is both a source and a destination");
  return PA_OK;
}

int check_decode_indices(const std::string& who, const pa_kv_pool* pool, int32_t B, const int32_t* block_tables,
                         int32_t max_blocks, const int32_t* context_lens, int32_t max_ctx, const int32_t* new_slots,
                         hipStream_t stream) {
  std::vector<int32_t> lens, tab, slots;
  if (int e = fetch(who, context_lens, B, lens, stream)) return e;
  if (int e = fetch(who, block_tables, static_cast<size_t>(B) * max_blocks, tab, stream)) return e;
  if (new_slots)
    if (int e = fetch(who, new_slots, B, slots, stream)) return e;
  const int32_t bs = pool->block_size;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t ctx = lens[b];
    if (ctx < 0 || ctx > max_ctx || static_cast<int64_t>(ctx) > static_cast<int64_t>(max_blocks) * bs)
      return fail(PA_EINVAL, who + ": context_lens[" + std::to_string(b) + "] = " + std::to_string(ctx) +
                                 " outside [0, max_ctx] or past the table");
    for (int32_t j = 0; j < (ctx + bs - 1) / bs; ++j) {
      const int32_t id = tab[static_cast<size_t>(b) * max_blocks + j];
      if (id < 0 || id >= pool->num_blocks)
        return fail(PA_EINVAL, who + ": block_tables[" + std::to_string(b) + "][" + std::to_string(j) + "] = " +
                                   std::to_string(id) + " out of range");
    }
    if (new_slots && slots[b] >= 0) {
      if (ctx < 1) return fail(PA_EINVAL, who + ": a new token needs context_lens >= 1");
      const int32_t p = ctx - 1;
      const int64_t want = static_cast<int64_t>(tab[static_cast<size_t>(b) * max_blocks + p / bs]) * bs + p % bs;
      if (slots[b] != want)
        return fail(PA_EINVAL, who + ": slot_mapping[" + std::to_string(b) + "] is not the slot of position " +
                                   "context_lens - 1");
    }
  }
  if (new_slots) return check_slots(who, pool, new_slots, B, stream);
  return PA_OK;
}

int check_share_groups(const std::string& who, const pa_kv_pool* pool, int32_t B, const int32_t* block_tables,
                       int32_t max_blocks, const int32_t* context_lens, const pa_share_group* groups, int32_t n_groups,
                       hipStream_t stream) {
  std::vector<int32_t> lens, tab;
  if (int e = fetch(who, context_lens, B, lens, stream)) return e;
  if (int e = fetch(who, block_tables, static_cast<size_t>(B) * max_blocks, tab, stream)) return e;
  for (int32_t c = 0; c < n_groups; ++c) {
    const pa_share_group& g = groups[c];
    const int32_t* t0 = tab.data() + static_cast<size_t>(g.first_row) * max_blocks;
    for (int32_t r = g.first_row; r < g.first_row + g.n_rows; ++r) {
      if (static_cast<int64_t>(g.shared_blocks) * pool->block_size > lens[r])
        return fail(PA_EINVAL, who + ": group " + std::to_string(c) + " shares blocks row " + std::to_string(r) +
                                   " does not fully see");
      const int32_t* tr = tab.data() + static_cast<size_t>(r) * max_blocks;
      for (int32_t j = 0; j < g.shared_blocks; ++j)
        if (tr[j] != t0[j])
          return fail(PA_EINVAL, who + ": group " + std::to_string(c) + " rows differ at block " + std::to_string(j));
    }
  }
  return PA_OK;
}

int check_prefill_indices(const std::string& who, const pa_kv_pool* pool, const int32_t* table, int32_t nb,
                          int32_t T, int32_t ctx_before, hipStream_t stream) {
  std::vector<int32_t> tab;
  if (int e = fetch(who, table, nb, tab, stream)) return e;
  const int64_t need = ceil_div(static_cast<int64_t>(ctx_before) + T, pool->block_size);
  for (int64_t j = 0; j < need; ++j)
    if (tab[j] < 0 || tab[j] >= pool->num_blocks)
      return fail(PA_EINVAL, who + ": block_table[" + std::to_string(j) + "] = " + std::to_string(tab[j]) +
                                 " out of range");
  return PA_OK;
}

}  // namespace pa

extern "C" int pa_set_validate(int on) {
  const int old = pa::validate_on() ? 1 : 0;
  pa::g_validate.store(on ? 1 : 0, std::memory_order_relaxed);
  return old;
}
