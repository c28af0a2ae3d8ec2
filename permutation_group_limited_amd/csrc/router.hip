// Group-limited top-k router for gfx950.
//
// Computes what the group_limited_router_kernel page (Modular MAX Mojo API,
// nn/moe) describes: biased scores for selection, the best topk_group of
// n_groups expert groups, the top-K experts inside them, and weights from
// the unbiased scores, optionally normalised, times routed_scaling_factor.
//
// Mapping (CDNA-specific; the page's one-thread-per-expert block is not
// used): a token is owned by LPT consecutive lanes of a wave64, each lane
// holding EPL consecutive experts (E = LPT * EPL). For E >= 64 a token fills
// a whole wave (E = 256: 4 experts, one 16-byte load per lane); for E < 64
// several tokens share a wave, and so do two tokens of 32 lanes each in
// large batches at E = 64 ... 256 (RouterWideLaunch). E that is not a power of two takes a general
// form (router_any_e_kernel): one wave per token with EPL * 64 >= E, absent
// experts never candidates, and the group stage below replaced by a scan of
// each group's scores staged in LDS.
//
//  * group score: lane-local top-2, then a top-2 merge over the LPG = S/EPL
//    lanes of a group through DPP (quad_perm, row_half_mirror, row_mirror),
//    ds_swizzle and, for 64-lane groups, ds_bpermute; groups are ranked by
//    counting the groups that beat each one (ties: lower group index).
//  * top-K: each lane sorts its EPL (key, expert) pairs (key = biased score
//    mapped to an order-preserving uint32) with Batcher's odd-even merge
//    sort; then K rounds of: segment max of the lane heads (DPP max steps
//    and v_readlane), a ballot of the lanes whose head equals it, the lowest
//    such lane wins (lowest expert id: the lower-index tie rule) and pops its
//    head (two tokens per wave: the sorted lists sit in LDS and a pop
//    advances a position). Round k fills slot k, so the slots come out in
//    (score desc, id asc) order.
//  * weights: the K winners' unbiased scores (read back from LDS or the
//    owner lane's registers), normalised in binary64 with the sum taken in
//    slot order, times the scaling factor, rounded once.
#include "router_tokens.hpp"

namespace moe {
namespace {

template <typename DS, typename DB, int EPL, int LPT, int FN>
__global__ __launch_bounds__(kBlock) void router_kernel(
    int32_t* __restrict__ out_idx, typename DS::storage* __restrict__ out_w,
    const typename DS::storage* __restrict__ scores, const typename DB::storage* __restrict__ bias,
    int64_t T, int32_t K, int32_t n_groups, int32_t topk_group, int32_t norm_weights,
    float scale, int32_t mode, RouterHist hist) {
  route_tokens<DS, DB, EPL, LPT, FN, kWavesPerBlock>(out_idx, out_w, scores, bias, T, K, n_groups,
                                                     topk_group, norm_weights, scale, mode,
                                                     linear_block(), 0, hist);
}

template <typename DS, typename DB, int EPL, int LPT, int FN>
struct RouterLaunch {
  static moe_status_t run(int32_t* idx, void* w, const void* s, const void* b, int64_t T,
                          int32_t K, int32_t G, int32_t TG, int32_t norm, float scale,
                          int32_t mode, RouterHist hist, hipStream_t stream) {
    constexpr int TPB = kWavesPerBlock * (kWave / LPT);  // tokens per block
    const int64_t blocks = (T + TPB - 1) / TPB;
    hipLaunchKernelGGL((router_kernel<DS, DB, EPL, LPT, FN>), grid_1d(blocks, kBlock),
                       dim3(kBlock), 0, stream, idx, static_cast<typename DS::storage*>(w),
                       static_cast<const typename DS::storage*>(s),
                       static_cast<const typename DB::storage*>(b), T, K, G, TG, norm, scale,
                       mode, hist);
    return check_launch();
  }
};

// Two tokens per wave for E = 64 ... 256 (32 lanes per token, 2 * EPL
// experts per lane): the K selection rounds serve two tokens at once and
// the histogram merge sees twice the slots per workgroup, so a token costs
// fewer instructions, but each wave's chain is longer. Reached through
// dispatch_router with the one-token mapping (EPL, 64); used for large
// batches only, where throughput rather than one wave's latency decides.
template <typename DS, typename DB, int EPL, int LPT, int FN>
struct RouterWideLaunch {
  static moe_status_t run(int32_t* idx, void* w, const void* s, const void* b, int64_t T,
                          int32_t K, int32_t G, int32_t TG, int32_t norm, float scale,
                          int32_t mode, RouterHist hist, hipStream_t stream) {
    if constexpr (LPT != kWave || EPL > 4) {
      return MOE_ERR_UNSUPPORTED;
    } else {
      constexpr int TPB = kWavesPerBlock * 2;  // tokens per block
      const int64_t blocks = (T + TPB - 1) / TPB;
      hipLaunchKernelGGL((router_kernel<DS, DB, 2 * EPL, kWave / 2, FN>), grid_1d(blocks, kBlock),
                         dim3(kBlock), 0, stream, idx, static_cast<typename DS::storage*>(w),
                         static_cast<const typename DS::storage*>(s),
                         static_cast<const typename DB::storage*>(b), T, K, G, TG, norm, scale,
                         mode, hist);
      return check_launch();
    }
  }
};

// Any E up to 1024 (not a power of two): one wave per token, EPL experts
// per lane with EPL * 64 >= E, group stage through LDS.
template <typename DS, typename DB, int EPL, int FN>
__global__ __launch_bounds__(kBlock) void router_any_e_kernel(
    int32_t* __restrict__ out_idx, typename DS::storage* __restrict__ out_w,
    const typename DS::storage* __restrict__ scores, const typename DB::storage* __restrict__ bias,
    int64_t T, int32_t K, int32_t n_groups, int32_t topk_group, int32_t norm_weights,
    float scale, int32_t mode, int32_t E, RouterHist hist) {
  route_tokens<DS, DB, EPL, kWave, FN, kWavesPerBlock, true>(
      out_idx, out_w, scores, bias, T, K, n_groups, topk_group, norm_weights, scale, mode,
      linear_block(), E, hist);
}

// Reached through dispatch_router with the padded expert count
// max(64, next power of two >= E), so LPT is always a full wave here.
template <typename DS, typename DB, int EPL, int LPT, int FN>
struct RouterAnyELaunch {
  static moe_status_t run(int32_t* idx, void* w, const void* s, const void* b, int64_t T,
                          int32_t K, int32_t G, int32_t TG, int32_t norm, float scale,
                          int32_t mode, int32_t E, RouterHist hist, hipStream_t stream) {
    if constexpr (LPT != kWave) {
      return MOE_ERR_UNSUPPORTED;
    } else {
      const int64_t blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
      hipLaunchKernelGGL((router_any_e_kernel<DS, DB, EPL, FN>), grid_1d(blocks, kBlock),
                         dim3(kBlock), 0, stream, idx,
                         static_cast<typename DS::storage*>(w),
                         static_cast<const typename DS::storage*>(s),
                         static_cast<const typename DB::storage*>(b), T, K, G, TG, norm, scale,
                         mode, E, hist);
      return check_launch();
    }
  }
};

}  // namespace

moe_status_t launch_router(int32_t* idx, void* w, const void* s, const void* b,
                           moe_dtype_t sd, moe_dtype_t bd, int32_t fn, int64_t T, int32_t E,
                           int32_t K, int32_t G, int32_t TG, int32_t norm, float scale,
                           int32_t mode, RouterHist hist, hipStream_t stream) {
  if ((E & (E - 1)) == 0) {
    const bool counting = hist.counts != nullptr || hist.fine != nullptr;
    if (router_two_tokens_per_wave(T, E, K, G, counting))
      return dispatch_router<RouterWideLaunch>(sd, bd, fn, E, idx, w, s, b, T, K, G, TG, norm,
                                               scale, mode, hist, stream);
    return dispatch_router<RouterLaunch>(sd, bd, fn, E, idx, w, s, b, T, K, G, TG, norm, scale,
                                         mode, hist, stream);
  }
  int32_t padded = kWave;
  while (padded < E) padded <<= 1;
  return dispatch_router<RouterAnyELaunch>(sd, bd, fn, padded, idx, w, s, b, T, K, G, TG, norm,
                                           scale, mode, E, hist, stream);
}

}  // namespace moe
