// Router and index creation in one launch (single-workgroup batches): dtype
// dispatch. The kernel is in route_index_impl.hpp, the batch limit in
// plan.hip.
#include "route_index.hpp"

namespace moe {

moe_status_t launch_route_index(int32_t* idx, void* w, const void* s, const void* b,
                                moe_dtype_t sd, moe_dtype_t bd, int32_t fn, int64_t T, int32_t E,
                                int32_t K, int32_t G, int32_t TG, int32_t norm, float scale,
                                int32_t mode, uint32_t* token_expert_order,
                                uint32_t* expert_start_indices, uint32_t* restore_token_order,
                                int32_t* expert_ids, uint32_t* expert_usage_stats,
                                uint32_t* scales_offset, uint32_t scale_align,
                                hipStream_t stream) {
  const IndexOutputs io{token_expert_order, expert_start_indices, restore_token_order,
                        expert_ids, expert_usage_stats, scales_offset, scale_align};
#define MOE_D(DS, DB)                                                                        \
  return launch_route_index_dt<DS, DB>(fn, E, idx, w, s, b, T, K, G, TG, norm, scale, mode, io, \
                                       stream)
  if (sd == MOE_DTYPE_F32 && bd == MOE_DTYPE_F32) MOE_D(DF32, DF32);
  if (sd == MOE_DTYPE_BF16 && bd == MOE_DTYPE_BF16) MOE_D(DBF16, DBF16);
  if (sd == MOE_DTYPE_BF16 && bd == MOE_DTYPE_F32) MOE_D(DBF16, DF32);
  if (sd == MOE_DTYPE_F16 && bd == MOE_DTYPE_F16) MOE_D(DF16, DF16);
  if (sd == MOE_DTYPE_F16 && bd == MOE_DTYPE_F32) MOE_D(DF16, DF32);
#undef MOE_D
  return MOE_ERR_UNSUPPORTED;
}

}  // namespace moe
