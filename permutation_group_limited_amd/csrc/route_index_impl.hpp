// Router and index creation in one launch for batches that one workgroup
// routes on its own (T at most W * 64 / LPT tokens: 16 at E = 256, 128 at
// E = 8), where the second launch is a large part of the step.
//
// Same results as moe_router_group_limited followed by moe_create_indices on
// its expert_indices: the routing routine is the router kernel's, and the
// index outputs come from the single-chunk routine that moe_create_indices
// runs when all slots fit one workgroup. Between the two stages a
// workgroup barrier is all the hand-over there is (every wave's
// expert_indices are then visible to the whole workgroup).
//
// A version for several workgroups, with the last one to finish (counted
// by an acquire-release atomic ticket) building the index outputs, was
// measured and dropped: the device-scope hand-over cost as much as the
// launch it saved, so larger batches take the two-launch form.
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
    float scale, int32_t mode, IndexOutputs io, int rounds) {
  constexpr int E = EPL * LPT;
  constexpr int W = route_index_waves<E>();
  route_tokens<DS, DB, EPL, LPT, FN, W>(out_idx, out_w, scores, bias, T, K, n_groups, topk_group,
                                        norm_weights, scale, mode, 0u);
  __syncthreads();
  const int64_t N = T * K;
  scatter_chunk<W>(io.order, io.starts, io.restore, io.expert_ids, io.stats, io.scales_offset,
                   io.scale_align, out_idx, nullptr, N, E,
                   static_cast<int64_t>(rounds) * W * kWave, 1, rounds, 0);
}

template <typename DS, typename DB, int EPL, int LPT, int FN>
struct RouteIndexLaunch {
  static constexpr int kTokens = route_index_waves<EPL * LPT>() * (kWave / LPT);

  static moe_status_t run(int32_t* idx, void* w, const void* s, const void* b, int64_t T,
                          int32_t K, int32_t G, int32_t TG, int32_t norm, float scale,
                          int32_t mode, IndexOutputs io, hipStream_t stream) {
    constexpr int W = route_index_waves<EPL * LPT>();
    if (T < 1 || T > kTokens) return MOE_ERR_UNSUPPORTED;  // one workgroup only
    const int64_t per_round = static_cast<int64_t>(W) * kWave;
    const int rounds = static_cast<int>((T * K + per_round - 1) / per_round);
    hipLaunchKernelGGL((route_index_kernel<DS, DB, EPL, LPT, FN>), dim3(1), dim3(W * kWave), 0,
                       stream, idx, static_cast<typename DS::storage*>(w),
                       static_cast<const typename DS::storage*>(s),
                       static_cast<const typename DB::storage*>(b), T, K, G, TG, norm, scale,
                       mode, io, rounds);
    return check_launch();
  }
};

}  // namespace

template <typename DS, typename DB>
moe_status_t launch_route_index_dt(int32_t fn, int32_t E, int32_t* idx, void* w, const void* s,
                                   const void* b, int64_t T, int32_t K, int32_t G, int32_t TG,
                                   int32_t norm, float scale, int32_t mode, IndexOutputs io,
                                   hipStream_t stream) {
  return dispatch_router_fn<RouteIndexLaunch, DS, DB>(fn, E, idx, w, s, b, T, K, G, TG, norm,
                                                      scale, mode, io, stream);
}

}  // namespace moe
