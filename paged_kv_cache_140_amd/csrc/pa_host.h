// Host-side helpers shared by every source of the library: error text,
// launch checks and pool validation.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <string>

#include "../../include/pa.h"

namespace pa {

void set_error(const std::string& msg);
int fail(int code, const std::string& msg);
int check_launch(const char* what);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Validates the pool struct and the layer index.
int check_pool(const pa_kv_pool* pool, int32_t layer);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Tuning overrides of the grid plans (0 = the library's own choice): read
// once from PA_DECODE_WAVES, PA_DECODE_PART_BLOCKS and PA_PREFILL_SPLITS at
// first use, changed by pa_set_tuning.
int tuning(int key);

// Compute units of the current device (queried once per device).
int device_cus();

// ---------------------------------------------------------------- validate
// Validate mode (pa_set_validate / PA_VALIDATE): host checks of the device
// indices a call trusts, before it launches anything (each synchronises the
// stream).  Each returns PA_OK or PA_EINVAL with a message.
bool validate_on();
int check_slots(const std::string& who, const pa_kv_pool* pool, const int32_t* slots, int32_t T, hipStream_t stream);
int check_pairs(const std::string& who, const pa_kv_pool* pool, const int32_t* pairs, int32_t n, hipStream_t stream);
int check_decode_indices(const std::string& who, const pa_kv_pool* pool, int32_t B, const int32_t* block_tables,
                         int32_t max_blocks, const int32_t* context_lens, int32_t max_ctx, const int32_t* new_slots,
                         hipStream_t stream);
int check_share_groups(const std::string& who, const pa_kv_pool* pool, int32_t B, const int32_t* block_tables,
                       int32_t max_blocks, const int32_t* context_lens, const pa_share_group* groups, int32_t n_groups,
                       hipStream_t stream);
int check_prefill_indices(const std::string& who, const pa_kv_pool* pool, const int32_t* table, int32_t nb,
                          int32_t T, int32_t ctx_before, hipStream_t stream);

// ---------------------------------------------------------------- decode
// Grid plan of a decode from host-side sizes only (context lengths stay on
// the device): waves per workgroup, and the split of each sequence into
// partitions of blocks_per_part blocks (num_parts of them for max_ctx).
struct DecodePlan {
  int waves;
  int blocks_per_part;
  int num_parts;
  // > 0: the device may run the split plan unsplit (decode_unsplit), given
  // this CU count; 0: the partitions are as planned.
  int unsplit_cus;
};
DecodePlan plan_decode(int B, int H_kv, int G, int bs, int max_ctx);

// Workspace of a split decode: (m, l) partials [B][H_q][P][2], then the
// un-normalised weighted V sums [B][H_q][P][D], fp32.
struct Workspace {
  float* ml;
  float* acc;
};
size_t workspace_bytes_for(const DecodePlan& pl, int B, int H_kv, int H_q, int D);
Workspace carve(void* ws, const DecodePlan& pl, int B, int H_kv, int H_q);

// Host-side checks of a decode call's arguments (PA_OK for B == 0).
int validate_decode(const std::string& who, const pa_kv_pool* pool, int32_t layer, void* out, const void* q,
                    int32_t B, int32_t H_q, const int32_t* block_tables, int32_t max_blocks,
                    const int32_t* context_lens, int32_t max_ctx);
// Checks the caller's workspace against the plan and carves it.
int decode_workspace_check(const std::string& who, const DecodePlan& pl, const pa_kv_pool* pool, int32_t B,
                           int32_t H_q, void* workspace, size_t workspace_bytes, Workspace* ws);
// Enqueues the kernel that merges the partitions of a split decode.
void launch_decode_merge(int dtype, int D, void* out, const Workspace& ws, const int32_t* ctx, int32_t B,
                         int32_t H_q, int32_t H_kv, const DecodePlan& pl, int bs, hipStream_t stream);

// ---------------------------------------------------------------- prefill
// Host-side checks of a prefill chunk's arguments (PA_OK for T == 0).
int validate_prefill(const std::string& who, const pa_kv_pool* pool, int32_t layer, void* out, const void* q,
                     int32_t T, int32_t H_q, const int32_t* block_table, int32_t nb, int32_t ctx_before);

}  // namespace pa
