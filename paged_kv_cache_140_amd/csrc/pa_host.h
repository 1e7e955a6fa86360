// Host-side helpers shared by every source of the library: error text,
// launch checks and pool validation.
#pragma once

#include <stdint.h>

#include <string>

#include "../../include/pa.h"

namespace pa {

void set_error(const std::string& msg);
int fail(int code, const std::string& msg);
int check_launch(const char* what);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Validates the pool struct and the layer index.
int check_pool(const pa_kv_pool* pool, int32_t layer);

}  // namespace pa
