// Internal declarations of the cache-group (multi-layer, multi-group) kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pba.h"

namespace pba {

// One group of a bundle append.  Strides are in elements; task counts fit in
// int32 because the host splits the tokens over launches.
struct GroupAppend {
  char* k;
  char* v;
  const char* k_new;      // [n][layers][heads][head_dim]
  const char* v_new;
  const int64_t* slots;   // [n]
  int64_t k_sl, k_sb, k_sh, v_sl, v_sb, v_sh;
  int32_t task0;          // first task of the group: K tasks, then V tasks
  int32_t per_kind;       // K tasks: n * layers * heads * pieces
  int32_t v_tasks;        // V tasks: token groups (runs of 8) * layers * heads * pieces
  int32_t layers, heads, head_dim, log2P, esize;
};

struct BundleAppendArgs {
  GroupAppend g[PBA_MAX_GROUPS];
  int32_t n_groups;
  int32_t n;       // tokens of this launch
  int32_t total;   // tasks of this launch
};

// One group of a bundle copy.  Strides are in bytes.
struct GroupCopy {
  char* k;
  char* v;
  const int32_t* src;
  const int32_t* dst;
  int64_t k_sl, k_sb, k_sh, v_sl, v_sb, v_sh;
  int32_t wg0;      // first work-group of the group
  int32_t layers, heads;
  int32_t tile16;   // 16-byte pieces per (layer, block, head) tile
};

struct BundleCopyArgs {
  GroupCopy g[PBA_MAX_GROUPS];
  int32_t n_groups;
  int32_t total;    // work-groups
};

hipError_t launch_kv_append_bundle(const BundleAppendArgs& a, hipStream_t stream);
hipError_t launch_block_copy_bundle(const BundleCopyArgs& a, hipStream_t stream);

}  // namespace pba
