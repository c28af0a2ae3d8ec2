// Router and index creation fused into one launch, for small batches where
// the launch gap between the two stages is a large share of the step.
//
// Same results as moe_router_group_limited followed by moe_create_indices on
// its expert_indices: the routing routine is the router kernel's, and the
// index outputs come from the same single-chunk routine that
// moe_create_indices runs when all slots fit one workgroup.
//
// Hand-over between the stages: each workgroup writes its tokens'
// expert_indices / expert_weights, then takes a ticket with one
// acquire-release atomic add (agent scope) on a caller-provided counter.
// The workgroup that draws the last ticket has acquired every other
// workgroup's writes; it reads all T * K ids, runs the index creation, and
// puts the counter back to zero for the next call. Workgroups run to completion independently, so no workgroup ever
// waits for another and the launch cannot deadlock whatever the occupancy.
#pragma once

#include "index_block.hpp"
#include "route_index.hpp"
#include "router_tokens.hpp"

namespace moe {
namespace {

// Waves per workgroup: as many as the index step's per-wave LDS table allows
// (W * E <= 4096 words), at most 16.
template <int E>
constexpr int route_index_waves() {
  return E <= 256 ? 16 : 4096 / E;
}

template <typename DS, typename DB, int EPL, int LPT, int FN>
__global__ __launch_bounds__(route_index_waves<EPL * LPT>() * kWave) void route_index_kernel(
    int32_t* out_idx, typename DS::storage* __restrict__ out_w,
    const typename DS::storage* __restrict__ scores, const typename DB::storage* __restrict__ bias,
    int64_t T, int32_t K, int32_t n_groups, int32_t topk_group, int32_t norm_weights,
    float scale, int32_t mode, IndexOutputs io, uint32_t* ticket, int rounds) {
  constexpr int E = EPL * LPT;
  constexpr int W = route_index_waves<E>();
  route_tokens<DS, DB, EPL, LPT, FN, W>(out_idx, out_w, scores, bias, T, K, n_groups, topk_group,
                                        norm_weights, scale, mode);
  // The workgroup barrier makes every wave's expert_indices visible to
  // thread 0; its agent-scope acquire-release count then publishes them
  // device-wide and, for the last workgroup, acquires every earlier
  // workgroup's; the second barrier hands that on to the other waves.
  __shared__ uint32_t is_last;
  __syncthreads();
  if (threadIdx.x == 0)
    is_last = (__hip_atomic_fetch_add(ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
               gridDim.x - 1u)
                  ? 1u
                  : 0u;
  __syncthreads();
  if (is_last == 0u) return;  // uniform over the workgroup
  const int64_t N = T * K;
  scatter_chunk<W>(io.order, io.starts, io.restore, io.expert_ids, io.stats, io.scales_offset,
                   io.scale_align, out_idx, nullptr, N, E,
                   static_cast<int64_t>(rounds) * W * kWave, 1, rounds, 0);
  if (threadIdx.x == 0)
    __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename DS, typename DB, int EPL, int LPT, int FN>
struct RouteIndexLaunch {
  static moe_status_t run(int32_t* idx, void* w, const void* s, const void* b, int64_t T,
                          int32_t K, int32_t G, int32_t TG, int32_t norm, float scale,
                          int32_t mode, IndexOutputs io, uint32_t* ticket, hipStream_t stream) {
    constexpr int W = route_index_waves<EPL * LPT>();
    constexpr int TPB = W * (kWave / LPT);  // tokens per workgroup
    const int64_t blocks = (T + TPB - 1) / TPB;
    const int64_t per_round = static_cast<int64_t>(W) * kWave;
    const int rounds = static_cast<int>((T * K + per_round - 1) / per_round);
    hipLaunchKernelGGL((route_index_kernel<DS, DB, EPL, LPT, FN>),
                       dim3(static_cast<uint32_t>(blocks)), dim3(W * kWave), 0,
                       stream, idx, static_cast<typename DS::storage*>(w),
                       static_cast<const typename DS::storage*>(s),
                       static_cast<const typename DB::storage*>(b), T, K, G, TG, norm, scale,
                       mode, io, ticket, rounds);
    return check_launch();
  }
};

}  // namespace

template <typename DS, typename DB>
moe_status_t launch_route_index_dt(int32_t fn, int32_t E, int32_t* idx, void* w, const void* s,
                                   const void* b, int64_t T, int32_t K, int32_t G, int32_t TG,
                                   int32_t norm, float scale, int32_t mode, IndexOutputs io,
                                   uint32_t* ticket, hipStream_t stream) {
  return dispatch_router_fn<RouteIndexLaunch, DS, DB>(fn, E, idx, w, s, b, T, K, G, TG, norm,
                                                      scale, mode, io, ticket, stream);
}

}  // namespace moe
