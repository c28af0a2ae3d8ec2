// Router + index creation in one launch (single-workgroup batches): the
// per-dtype instance sets, each compiled in a translation unit of its own
// (route_index_*.hip) so that the many instances build in parallel.
#pragma once

#include "common.hpp"

namespace moe {

struct IndexOutputs {
  uint32_t* order;
  uint32_t* starts;
  uint32_t* restore;
  int32_t* expert_ids;
  uint32_t* stats;
  uint32_t* scales_offset;  // NULL: no aligned offsets
  uint32_t scale_align;
};

// Launches the fused kernel for scores of type DS and bias of type DB.
template <typename DS, typename DB>
moe_status_t launch_route_index_dt(int32_t fn, int32_t E, int32_t* idx, void* w, const void* s,
                                   const void* b, int64_t T, int32_t K, int32_t G, int32_t TG,
                                   int32_t norm, float scale, int32_t mode, IndexOutputs io,
                                   hipStream_t stream);

// Largest T that one workgroup routes for E experts (0: no one-launch form,
// E not a power of two or above 1024).
int64_t route_index_max_tokens(int32_t E);

}  // namespace moe
