// Instances of the fused router + index kernel for fp32 scores and bias.
#include "route_index_impl.hpp"

namespace moe {
template moe_status_t launch_route_index_dt<DF32, DF32>(int32_t, int32_t, int32_t*, void*,
                                                   const void*, const void*, int64_t, int32_t,
                                                   int32_t, int32_t, int32_t, float, int32_t,
                                                   IndexOutputs, hipStream_t);

}  // namespace moe
