// Status codes, the thread-local last-error text, pool validation, the
// tuning overrides and the device's CU count.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdlib>
#include <mutex>
#include <string>

#include "pa_host.h"

namespace pa {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_EHIP, std::string(what) + ": " + hipGetErrorString(e));
  return PA_OK;
}

int check_pool(const pa_kv_pool* pool, int32_t layer) {
  if (!pool) return fail(PA_EINVAL, "pool is NULL");
  if (!pool->k || !pool->v) return fail(PA_EINVAL, "pool k/v pointer is NULL");
  if (!aligned16(pool->k) || !aligned16(pool->v)) return fail(PA_EINVAL, "pool k and v must be 16-byte aligned");
  if (pool->num_layers <= 0 || pool->num_kv_heads <= 0 || pool->num_blocks <= 0 || pool->block_size <= 0 ||
      pool->head_dim <= 0)
    return fail(PA_EINVAL, "pool sizes must be positive");
  if (pool->dtype != PA_F32 && pool->dtype != PA_BF16 && pool->dtype != PA_F16)
    return fail(PA_EINVAL, "unknown pool dtype");
  if (layer < 0 || layer >= pool->num_layers) return fail(PA_EINVAL, "layer out of range");
  if (pool->head_dim != 64 && pool->head_dim != 128)
    return fail(PA_ENOTSUP, "head_dim must be 64 or 128");
  const int64_t slots = static_cast<int64_t>(pool->num_blocks) * pool->block_size;
  if (slots > INT32_MAX) return fail(PA_EINVAL, "num_blocks * block_size must fit in int32 slots");
  return PA_OK;
}

// ---------------------------------------------------------------- tuning
namespace {
constexpr int kTuneKeys = 3;
const char* const kTuneEnv[kTuneKeys] = {"PA_DECODE_WAVES", "PA_DECODE_PART_BLOCKS", "PA_PREFILL_SPLITS"};
std::atomic<int> g_tune[kTuneKeys];
std::once_flag g_tune_once;

void tune_init() {
  std::call_once(g_tune_once, [] {
    for (int k = 0; k < kTuneKeys; ++k) {
      const char* s = std::getenv(kTuneEnv[k]);
      const int v = (s && *s) ? std::atoi(s) : 0;
      g_tune[k].store(v > 0 ? v : 0, std::memory_order_relaxed);
    }
  });
}
}  // namespace

int tuning(int key) {
  tune_init();
  return g_tune[key].load(std::memory_order_relaxed);
}

// ---------------------------------------------------------------- devices
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace pa

extern "C" int pa_set_tuning(int key, int value) {
  if (key < 0 || key >= pa::kTuneKeys || value < 0) return pa::fail(PA_EINVAL, "pa_set_tuning: bad key or value");
  pa::tune_init();
  return pa::g_tune[key].exchange(value, std::memory_order_relaxed);
}

extern "C" const char* pa_status_string(int status) {
  static thread_local std::string msg;
  const char* base = "unknown status";
  switch (status) {
    case PA_OK: base = "ok"; break;
    case PA_EINVAL: base = "invalid argument"; break;
    case PA_ENOTSUP: base = "not supported"; break;
    case PA_ENOMEM: base = "out of free blocks"; break;
    case PA_EHIP: base = "HIP error"; break;
    case PA_ENOENT: base = "no such sequence"; break;
    case PA_ESPACE: base = "buffer too small"; break;
  }
  msg = base;
  if (status != PA_OK && !pa::g_last_error.empty()) msg += ": " + pa::g_last_error;
  return msg.c_str();
}
