// Instances of the fused router + index kernel for fp16 scores with fp16 or fp32 bias.
#include "route_index_impl.hpp"

namespace moe {
template moe_status_t launch_route_index_dt<DF16, DF16>(int32_t, int32_t, int32_t*, void*,
                                                   const void*, const void*, int64_t, int32_t,
                                                   int32_t, int32_t, int32_t, float, int32_t,
                                                   IndexOutputs, hipStream_t);
template moe_status_t launch_route_index_dt<DF16, DF32>(int32_t, int32_t, int32_t*, void*,
                                                   const void*, const void*, int64_t, int32_t,
                                                   int32_t, int32_t, int32_t, float, int32_t,
                                                   IndexOutputs, hipStream_t);

}  // namespace moe
