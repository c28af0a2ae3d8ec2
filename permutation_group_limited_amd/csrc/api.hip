// C ABI of the routing path: argument validation, then one launcher per
// stage on the caller's stream. Nothing here allocates, synchronises or
// touches device memory from the host.
#include <limits.h>

#include "common.hpp"

namespace moe {
namespace {
thread_local int g_last_hip_error = 0;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
size_t dtype_bytes(moe_dtype_t d) { return d == MOE_DTYPE_F32 ? 4 : 2; }
bool dtype_ok(moe_dtype_t d) {
  return d == MOE_DTYPE_F32 || d == MOE_DTYPE_BF16 || d == MOE_DTYPE_F16;
}
// score/bias dtype pairs with a router instance: equal, or fp32 bias
bool router_dtypes_supported(moe_dtype_t s, moe_dtype_t b) {
  return s == b || b == MOE_DTYPE_F32;
}
}  // namespace

moe_status_t hip_failure(hipError_t err) {
  g_last_hip_error = static_cast<int>(err);
  return MOE_ERR_HIP;
}

moe_status_t check_launch() {
  const hipError_t err = hipGetLastError();
  return err == hipSuccess ? MOE_OK : hip_failure(err);
}

}  // namespace moe

using namespace moe;

extern "C" {

static moe_status_t router_check(int32_t* expert_indices, void* expert_weights,
                                 const void* expert_scores, const void* expert_bias,
                                 moe_dtype_t scores_dtype, moe_dtype_t bias_dtype, int64_t T,
                                 int32_t E, int32_t K, int32_t n_groups, int32_t topk_group,
                                 moe_group_score_t group_score) {
  if (T < 0 || E < 1 || n_groups < 1 || n_groups > 64 || E % n_groups != 0)
    return MOE_ERR_INVALID_ARG;
  if (topk_group < 1 || topk_group > n_groups) return MOE_ERR_INVALID_ARG;
  const int64_t S = E / n_groups;
  if (K < 1 || K > topk_group * S || K > 64) return MOE_ERR_INVALID_ARG;
  if (group_score != MOE_GROUP_TOP2_SUM && group_score != MOE_GROUP_MAX)
    return MOE_ERR_INVALID_ARG;
  if (!dtype_ok(scores_dtype) || !dtype_ok(bias_dtype)) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!expert_indices || !expert_weights || !expert_scores || !expert_bias))
    return MOE_ERR_INVALID_ARG;
  if (T > (int64_t)UINT32_MAX / K) return MOE_ERR_INVALID_ARG;
  if (!router_dtypes_supported(scores_dtype, bias_dtype)) return MOE_ERR_UNSUPPORTED;
  if (E > 1024) return MOE_ERR_UNSUPPORTED;
  if (!aligned(expert_scores, 16) || !aligned(expert_bias, 16) || !aligned(expert_indices, 4) ||
      !aligned(expert_weights, dtype_bytes(scores_dtype)))
    return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

static moe_status_t router_common(int32_t* expert_indices, void* expert_weights,
                                  const void* expert_scores, const void* expert_bias,
                                  moe_dtype_t scores_dtype, moe_dtype_t bias_dtype,
                                  int32_t score_fn, int64_t T, int32_t E, int32_t K,
                                  int32_t n_groups, int32_t topk_group, int32_t norm_weights,
                                  float routed_scaling_factor, moe_group_score_t group_score,
                                  void* stream) {
  const moe_status_t st = router_check(expert_indices, expert_weights, expert_scores, expert_bias,
                                       scores_dtype, bias_dtype, T, E, K, n_groups, topk_group,
                                       group_score);
  if (st != MOE_OK || T == 0) return st;
  return launch_router(expert_indices, expert_weights, expert_scores, expert_bias, scores_dtype,
                       bias_dtype, score_fn, T, E, K, n_groups, topk_group, norm_weights ? 1 : 0,
                       routed_scaling_factor, static_cast<int32_t>(group_score),
                       RouterHist{nullptr, 0u}, static_cast<hipStream_t>(stream));
}

moe_status_t moe_router_group_limited(int32_t* expert_indices, void* expert_weights,
                                      const void* expert_scores, const void* expert_bias,
                                      moe_dtype_t scores_dtype, moe_dtype_t bias_dtype,
                                      int64_t T, int32_t E, int32_t K, int32_t n_groups,
                                      int32_t topk_group, int32_t norm_weights,
                                      float routed_scaling_factor, moe_group_score_t group_score,
                                      void* stream) {
  return router_common(expert_indices, expert_weights, expert_scores, expert_bias, scores_dtype,
                       bias_dtype, 0, T, E, K, n_groups, topk_group, norm_weights,
                       routed_scaling_factor, group_score, stream);
}

moe_status_t moe_router_group_limited_logits(int32_t* expert_indices, void* expert_weights,
                                             const void* router_logits, const void* expert_bias,
                                             moe_dtype_t logits_dtype, moe_dtype_t bias_dtype,
                                             moe_score_fn_t score_fn, int64_t T, int32_t E,
                                             int32_t K, int32_t n_groups, int32_t topk_group,
                                             int32_t norm_weights, float routed_scaling_factor,
                                             moe_group_score_t group_score, void* stream) {
  if (score_fn != MOE_SCORE_SIGMOID && score_fn != MOE_SCORE_SOFTMAX) return MOE_ERR_INVALID_ARG;
  return router_common(expert_indices, expert_weights, router_logits, expert_bias, logits_dtype,
                       bias_dtype, static_cast<int32_t>(score_fn), T, E, K, n_groups, topk_group,
                       norm_weights, routed_scaling_factor, group_score, stream);
}

// A plan of several chunks never has more than kMaxChunks of them, so this
// bound serves every N' <= N: the size never decreases as N grows.
static size_t counts_bound(int32_t E) {
  return static_cast<size_t>(kMaxChunks) * static_cast<size_t>(E) * sizeof(uint32_t);
}

size_t moe_create_indices_workspace_size(int64_t N, int32_t E) {
  if (N < 0 || N > (int64_t)UINT32_MAX || E < 1 || E > 1024) return 0;
  return plan_indices(N, E).nchunks > 1 ? counts_bound(E) : 0;
}

// Index-output checks shared by the index entry points and the fused one
// (which has no topk_ids input: pass a non-NULL stand-in).
static moe_status_t index_outputs_check(uint32_t* token_expert_order,
                                        uint32_t* expert_start_indices,
                                        uint32_t* restore_token_order, int32_t* expert_ids,
                                        uint32_t* expert_usage_stats, const int32_t* topk_ids,
                                        int64_t N, int32_t E, uint32_t* scales_offset,
                                        uint32_t scale_align) {
  if (N < 0 || N > (int64_t)UINT32_MAX || E < 1 || E > 1024) return MOE_ERR_INVALID_ARG;
  if (!expert_start_indices || !expert_ids || !expert_usage_stats) return MOE_ERR_INVALID_ARG;
  if (N > 0 && (!token_expert_order || !restore_token_order || !topk_ids))
    return MOE_ERR_INVALID_ARG;
  if (scales_offset != nullptr &&
      (scale_align == 0 || N + static_cast<int64_t>(E) * (scale_align - 1) > (int64_t)UINT32_MAX))
    return MOE_ERR_INVALID_ARG;
  if (!aligned(token_expert_order, 4) || !aligned(expert_start_indices, 4) ||
      !aligned(restore_token_order, 4) || !aligned(expert_ids, 4) ||
      !aligned(expert_usage_stats, 4) || !aligned(topk_ids, 4) || !aligned(scales_offset, 4))
    return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

static moe_status_t indices_common(uint32_t* token_expert_order,
                                   uint32_t* expert_start_indices, uint32_t* restore_token_order,
                                   int32_t* expert_ids, uint32_t* expert_usage_stats,
                                   const int32_t* topk_ids, int64_t N, int32_t E,
                                   void* workspace, size_t workspace_bytes,
                                   uint32_t* scales_offset, uint32_t scale_align, void* stream) {
  const moe_status_t st =
      index_outputs_check(token_expert_order, expert_start_indices, restore_token_order,
                          expert_ids, expert_usage_stats, topk_ids, N, E, scales_offset,
                          scale_align);
  if (st != MOE_OK) return st;
  const IndexPlan plan = plan_indices(N, E);
  if (plan.workspace_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.workspace_bytes))
    return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, 4)) return MOE_ERR_ALIGNMENT;
  return launch_indices(token_expert_order, expert_start_indices, restore_token_order, expert_ids,
                        expert_usage_stats, scales_offset, scale_align, topk_ids, N, E,
                        workspace, plan, false, nullptr, static_cast<hipStream_t>(stream));
}

moe_status_t moe_create_indices(uint32_t* token_expert_order, uint32_t* expert_start_indices,
                                uint32_t* restore_token_order, int32_t* expert_ids,
                                uint32_t* expert_usage_stats, const int32_t* topk_ids,
                                int64_t N, int32_t E, void* workspace, size_t workspace_bytes,
                                uint32_t* scales_offset_p, void* stream) {
  if (scales_offset_p != nullptr) return MOE_ERR_UNSUPPORTED;
  return indices_common(token_expert_order, expert_start_indices, restore_token_order,
                        expert_ids, expert_usage_stats, topk_ids, N, E, workspace,
                        workspace_bytes, nullptr, 0, stream);
}

moe_status_t moe_create_indices_aligned(uint32_t* token_expert_order,
                                        uint32_t* expert_start_indices,
                                        uint32_t* restore_token_order, int32_t* expert_ids,
                                        uint32_t* expert_usage_stats, const int32_t* topk_ids,
                                        int64_t N, int32_t E, void* workspace,
                                        size_t workspace_bytes, uint32_t* scales_offset,
                                        uint32_t scale_align, void* stream) {
  if (scales_offset == nullptr) return MOE_ERR_INVALID_ARG;
  return indices_common(token_expert_order, expert_start_indices, restore_token_order,
                        expert_ids, expert_usage_stats, topk_ids, N, E, workspace,
                        workspace_bytes, scales_offset, scale_align, stream);
}

// Workspace of moe_route_and_index: a 256-byte header (word 0 the ticket of
// the scatter's workgroups, word 1 the status word), then room for a counts
// matrix of kMaxChunks rows (zero between calls, with the ticket; rows of E
// words in the chunked form, of ranked_stride(E) in the ranked form), then,
// for the ranked form, room for the router's fine rows of counts (scratch:
// fully rewritten by every call that uses them). Sized for the largest plan of
// any T' <= T, so the size never decreases as T grows.
static constexpr size_t kTicketBytes = 256;

static bool two_launch_possible(int64_t T, int32_t E) { return T > route_index_max_tokens(E); }

static size_t ranked_counts_bytes(int32_t E) {
  return static_cast<size_t>(kMaxChunks) * static_cast<size_t>(ranked_stride(E)) *
         sizeof(uint32_t);
}

static size_t route_index_workspace(int64_t T, int32_t K, int32_t E) {
  const bool ranked = E <= kRankedMaxExperts && two_launch_possible(T, E);
  const bool chunked = plan_indices(T * K, E, true).nchunks > 1;
  size_t bytes = kTicketBytes;
  if (ranked)
    bytes += ranked_counts_bytes(E);
  else if (chunked)
    bytes += counts_bound(E);
  if (ranked)
    bytes += static_cast<size_t>(ranked_fine_rows_bound(T)) *
             static_cast<size_t>(ranked_stride(E)) * sizeof(uint32_t);
  return bytes;
}

size_t moe_route_and_index_workspace_size(int64_t T, int32_t K, int32_t E) {
  if (T < 0 || K < 1 || E < 1 || E > 1024 || T > (int64_t)UINT32_MAX / K) return 0;
  return route_index_workspace(T, K, E);
}

moe_status_t moe_route_and_index(int32_t* expert_indices, void* expert_weights,
                                 uint32_t* token_expert_order, uint32_t* expert_start_indices,
                                 uint32_t* restore_token_order, int32_t* expert_ids,
                                 uint32_t* expert_usage_stats, uint32_t* scales_offset,
                                 uint32_t scale_align, const void* router_input,
                                 const void* expert_bias, moe_dtype_t input_dtype,
                                 moe_dtype_t bias_dtype, moe_score_fn_t score_fn, int64_t T,
                                 int32_t E, int32_t K, int32_t n_groups, int32_t topk_group,
                                 int32_t norm_weights, float routed_scaling_factor,
                                 moe_group_score_t group_score, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (score_fn != MOE_SCORE_NONE && score_fn != MOE_SCORE_SIGMOID &&
      score_fn != MOE_SCORE_SOFTMAX)
    return MOE_ERR_INVALID_ARG;
  moe_status_t st = router_check(expert_indices, expert_weights, router_input, expert_bias,
                                 input_dtype, bias_dtype, T, E, K, n_groups, topk_group,
                                 group_score);
  if (st != MOE_OK) return st;
  const int64_t N = T * K;  // < 2^32 after router_check
  st = index_outputs_check(token_expert_order, expert_start_indices, restore_token_order,
                           expert_ids, expert_usage_stats, expert_indices, N, E, scales_offset,
                           scale_align);
  if (st != MOE_OK) return st;
  if (workspace == nullptr || workspace_bytes < route_index_workspace(T, K, E))
    return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, 4)) return MOE_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* ticket = static_cast<uint32_t*>(workspace);
  uint32_t* counts = ticket + kTicketBytes / sizeof(uint32_t);
  const IndexPlan plan = plan_indices(N, E, true);
  if (T == 0)  // nothing to route: the index step alone writes the metadata
    return launch_indices(token_expert_order, expert_start_indices, restore_token_order,
                          expert_ids, expert_usage_stats, scales_offset, scale_align,
                          expert_indices, 0, E, nullptr, plan, false, nullptr, s);
  if (T <= route_index_max_tokens(E))  // one workgroup routes it all: one launch
    return launch_route_index(expert_indices, expert_weights, router_input, expert_bias,
                              input_dtype, bias_dtype, static_cast<int32_t>(score_fn), T, E, K,
                              n_groups, topk_group, norm_weights ? 1 : 0, routed_scaling_factor,
                              static_cast<int32_t>(group_score), token_expert_order,
                              expert_start_indices, restore_token_order, expert_ids,
                              expert_usage_stats, scales_offset, scale_align, s);
  const RankedPlan rp = plan_ranked(T, K, E, n_groups);
  if (rp.ok && aligned(workspace, 16)) {  // its rows of counts move in 16-byte pieces
    // two launches, ranked form: the router ranks every slot within its
    // workgroup and records its row of counts (and adds it into the counts
    // matrix when there are several chunks); the index step places each
    // slot from those alone
    uint32_t* fine = counts + ranked_counts_bytes(E) / sizeof(uint32_t);
    uint32_t* coarse = counts;  // the ranked form always has several chunks
    const moe_status_t rs = launch_router(
        expert_indices, expert_weights, router_input, expert_bias, input_dtype, bias_dtype,
        static_cast<int32_t>(score_fn), T, E, K, n_groups, topk_group, norm_weights ? 1 : 0,
        routed_scaling_factor, static_cast<int32_t>(group_score),
        RouterHist{coarse, 0u, fine, restore_token_order, rp.R}, s);
    if (rs != MOE_OK) return rs;
    return launch_indices_ranked(token_expert_order, expert_start_indices, restore_token_order,
                                 expert_ids, expert_usage_stats, scales_offset, scale_align, N, E,
                                 fine, coarse, ticket, rp, s);
  }
  // two launches, chunked form: the router also fills the index step's
  // counts matrix, then the scatter (which clears the matrix again) takes
  // no histogram pass
  const bool multi = plan.nchunks > 1;
  const moe_status_t rs = launch_router(
      expert_indices, expert_weights, router_input, expert_bias, input_dtype, bias_dtype,
      static_cast<int32_t>(score_fn), T, E, K, n_groups, topk_group, norm_weights ? 1 : 0,
      routed_scaling_factor, static_cast<int32_t>(group_score),
      RouterHist{multi ? counts : nullptr, static_cast<uint32_t>(plan.chunk)}, s);
  if (rs != MOE_OK) return rs;
  return launch_indices(token_expert_order, expert_start_indices, restore_token_order, expert_ids,
                        expert_usage_stats, scales_offset, scale_align, expert_indices, N, E,
                        counts, plan, multi, ticket, s);
}

moe_status_t moe_finalize(void* output, moe_dtype_t out_dtype, const void* down,
                          moe_dtype_t down_dtype, const uint32_t* restore_order,
                          const void* router_weight, moe_dtype_t weight_dtype, int64_t T,
                          int32_t K, int64_t H, void* stream) {
  if (T < 0 || K < 1 || H < 0) return MOE_ERR_INVALID_ARG;
  if (!dtype_ok(out_dtype) || !dtype_ok(down_dtype) || !dtype_ok(weight_dtype))
    return MOE_ERR_INVALID_ARG;
  if (T > (int64_t)UINT32_MAX / K) return MOE_ERR_INVALID_ARG;
  // an output row must stay below 2^31 bytes (its stores address it in 32 bits)
  if (H > (int64_t)INT32_MAX ||
      H * static_cast<int64_t>(dtype_bytes(out_dtype)) > (int64_t)INT32_MAX - 16)
    return MOE_ERR_UNSUPPORTED;
  if (T > 0 && H > 0 && (!output || !down || !restore_order || !router_weight))
    return MOE_ERR_INVALID_ARG;
  if ((H * static_cast<int64_t>(dtype_bytes(down_dtype))) % 16 != 0) return MOE_ERR_ALIGNMENT;
  if (!aligned(output, 16) || !aligned(down, 16) || !aligned(restore_order, 4) ||
      !aligned(router_weight, dtype_bytes(weight_dtype)))
    return MOE_ERR_ALIGNMENT;
  if (T == 0 || H == 0) return MOE_OK;
  return launch_finalize(output, out_dtype, down, down_dtype, restore_order, router_weight,
                         weight_dtype, T, K, H, static_cast<hipStream_t>(stream));
}

const char* moe_status_string(moe_status_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_ALIGNMENT: return "misaligned pointer or row size";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: break;
  }
  return "unknown status";
}

int moe_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
