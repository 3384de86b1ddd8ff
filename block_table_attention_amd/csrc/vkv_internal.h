// Validate-mode checks against the mapped frontiers of contiguous arenas.
#pragma once

#include <stdint.h>

namespace pba {

// Each returns PBA_OK when k_base lies in no arena, or when every row the call
// would touch lies below its slot's mapped frontier; PBA_ERR_OUT_OF_RANGE
// otherwise.
int vkv_check_rows(const void* k_base, const int32_t* slots, const int32_t* lens, int64_t n);
int vkv_check_slot_ids(const void* k_base, const int64_t* ids, int64_t n);
int vkv_check_blocks(const void* k_base, const int32_t* ids, int64_t n);

}  // namespace pba
