/*
 * moe_route.h - C ABI of the MI355X (gfx950) group-limited MoE routing path.
 *
 * Three stages, each one entry point:
 *   moe_router_group_limited  - group-limited top-k router
 *   moe_create_indices        - bucket sort of routed slots into expert order
 *   moe_finalize              - fused unpermute gather + weighted top-k sum
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory. Every tensor argument is a plain pointer to DEVICE memory owned by
 * the caller, densely packed in row-major order (no strides). The entry
 * points never allocate, free or retain memory; scratch space, where
 * needed, is a caller-provided device workspace. The only memory the
 * library owns is the fixed device array of moe_create_indices_no_alloc
 * (one per GPU, for the life of the process).
 *
 * Streams. `stream` is a hipStream_t passed as void* (NULL = the legacy null
 * stream of the current device). All work is enqueued asynchronously on that
 * stream on the current HIP device; no call synchronises, copies to the host
 * or reads device memory from the host, so every call can be captured into a
 * HIP graph.
 *
 * Errors. Each call returns moe_status_t. Arguments are validated on the
 * host before anything is enqueued; on a validation error nothing is
 * launched and no output is written. MOE_ERR_HIP means a launch was
 * rejected by the HIP runtime (moe_last_hip_error() gives the hipError_t
 * value); launches of the same call enqueued before it may have run (for
 * moe_route_and_index, see its workspace note). Conditions on
 * the *contents* of device buffers (expert ids in range, restore_order a
 * permutation, finite scores) are preconditions, not checked: the kernels
 * stay inside every buffer when they are violated, but the values written
 * are then unspecified.
 *
 * Sizes are int64_t; T*K (the number of routed slots, N) must be below 2^32
 * because all slot indices are uint32.
 *
 * Enumerations. Each enum below carries *_ENUM_MIN / *_ENUM_MAX markers that
 * span the whole int32 range, so that any int32 a caller passes is a value
 * of the enum type (also in C++) and an unknown one is rejected by
 * validation (MOE_ERR_INVALID_ARG) rather than being undefined. The markers
 * are never valid arguments.
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* size, shape or NULL pointer error */
    MOE_ERR_UNSUPPORTED = 2, /* valid request this build has no kernel for */
    MOE_ERR_ALIGNMENT = 3,   /* pointer or row size not 16-byte aligned */
    MOE_ERR_WORKSPACE = 4,   /* workspace missing or too small */
    MOE_ERR_HIP = 5,         /* HIP runtime rejected a launch */
    MOE_STATUS_ENUM_MIN = -0x7FFFFFFF - 1, /* range markers (see below), never returned */
    MOE_STATUS_ENUM_MAX = 0x7FFFFFFF
} moe_status_t;

typedef enum {
    MOE_DTYPE_F32 = 0,  /* IEEE binary32 */
    MOE_DTYPE_BF16 = 1, /* bfloat16 (high half of binary32) */
    MOE_DTYPE_F16 = 2,  /* IEEE binary16 */
    MOE_DTYPE_ENUM_MIN = -0x7FFFFFFF - 1, /* range markers, not dtypes */
    MOE_DTYPE_ENUM_MAX = 0x7FFFFFFF
} moe_dtype_t;
/* Every value is widened exactly to binary32 on load; results are
 * computed in binary32 (router weights and score functions in binary64)
 * and rounded to nearest even on store. */

/* How a group of experts is scored before the top-topk_group groups are
 * kept. The router page keeps the best-scoring groups without saying how a
 * group's score is formed; two readings are offered. */
typedef enum {
    MOE_GROUP_TOP2_SUM = 0, /* sum of the two largest biased scores in the group (default) */
    MOE_GROUP_MAX = 1,      /* largest biased score in the group */
    MOE_GROUP_ENUM_MIN = -0x7FFFFFFF - 1, /* range markers, not modes */
    MOE_GROUP_ENUM_MAX = 0x7FFFFFFF
} moe_group_score_t;

/*
 * moe_router_group_limited
 * Follows the group_limited_router_kernel page (Modular MAX Mojo API,
 * nn/moe): description, Parameters and Args.
 *
 *   expert_indices   out int32 [T, K]: selected experts of each token.
 *   expert_weights   out, dtype = scores_dtype (the page gives the weights
 *                    the scores' type), [T, K]: routing weights computed
 *                    from the UNBIASED scores.
 *   expert_scores    in  [T, E] routing scores, dtype scores_dtype.
 *   expert_bias      in  [E] per-expert bias, dtype bias_dtype, added to the
 *                    scores for selection only.
 *   T                tokens (>= 0); E experts; K = experts per token.
 *   n_groups         the E experts form n_groups consecutive groups of
 *                    S = E / n_groups experts.
 *   topk_group       number of best groups a token may select from.
 *   norm_weights     non-zero: weights are divided by their sum over the K
 *                    selected experts before scaling.
 *   routed_scaling_factor  multiplied into every weight last.
 *   group_score      see moe_group_score_t.
 *
 * Per token: b[e] = score[e] + bias[e] (fp32); groups ranked by group score
 * (ties: lower group index first), the first topk_group kept; among their
 * experts the K best by (b descending, expert index ascending) fill slots
 * 0..K-1 in that order; weight_k = score[e_k] (/ sum) * scale, evaluated in
 * binary64 (sum over k = 0..K-1 in slot order, correctly rounded divide and
 * product) and rounded once to binary32, then to the weights' dtype.
 *
 * Validation: T >= 0; E >= 1 and E % n_groups == 0; 1 <= topk_group <=
 * n_groups <= 64; 1 <= K <= topk_group * S; K <= 64; non-NULL pointers when
 * T > 0; expert_scores and expert_bias 16-byte aligned. Supported: scores
 * F32, BF16 or F16 with bias of the same dtype or F32; 1 <= E <= 1024
 * (larger E give MOE_ERR_UNSUPPORTED). Powers of two take the fastest
 * form; other E run one token per wave with the group stage in LDS.
 */
moe_status_t moe_router_group_limited(int32_t* expert_indices, void* expert_weights,
                                      const void* expert_scores, const void* expert_bias,
                                      moe_dtype_t scores_dtype, moe_dtype_t bias_dtype,
                                      int64_t T, int32_t E, int32_t K, int32_t n_groups,
                                      int32_t topk_group, int32_t norm_weights,
                                      float routed_scaling_factor, moe_group_score_t group_score,
                                      void* stream);

/* Score functions the logits entry point applies before routing. */
typedef enum {
    MOE_SCORE_NONE = 0,    /* the input already holds the scores */
    MOE_SCORE_SIGMOID = 1, /* score = 1 / (1 + exp(-logit)) */
    MOE_SCORE_SOFTMAX = 2, /* score = softmax of the token's E logits */
    MOE_SCORE_ENUM_MIN = -0x7FFFFFFF - 1, /* range markers, not functions */
    MOE_SCORE_ENUM_MAX = 0x7FFFFFFF
} moe_score_fn_t;

/*
 * moe_router_group_limited_logits
 * The router with the scores computed on the fly from logits: the page's
 * optional scores_input_fn (Parameters: a loader of the score of a (token,
 * expert) pair), here one of two fixed functions. Saves writing and reading
 * a [T, E] scores tensor. Each score is evaluated in binary64 and rounded
 * once to binary32; routing then proceeds exactly as in
 * moe_router_group_limited, and expert_weights (dtype = logits_dtype) come
 * from these scores. The binary64 steps are fixed, so the scores do not
 * depend on a math library: exp(x) by Cody and Waite's reduction with ln 2
 * split in two binary64 parts, the Taylor polynomial of exp up to degree 13
 * by Horner's rule with fused multiply-adds, and 2^k applied as two exact
 * powers of two (0 below -745.2, +inf above 709.78); the softmax subtracts
 * the token's largest logit and divides by the pairwise sum of the E
 * exponentials (a balanced tree over the experts in index order, padded
 * with zeros to a power of two).
 *
 *   router_logits    in [T, E], dtype logits_dtype.
 *   other arguments, validation and support as moe_router_group_limited;
 *   score_fn must be MOE_SCORE_SIGMOID or MOE_SCORE_SOFTMAX.
 */
moe_status_t moe_router_group_limited_logits(int32_t* expert_indices, void* expert_weights,
                                             const void* router_logits, const void* expert_bias,
                                             moe_dtype_t logits_dtype, moe_dtype_t bias_dtype,
                                             moe_score_fn_t score_fn, int64_t T, int32_t E,
                                             int32_t K, int32_t n_groups, int32_t topk_group,
                                             int32_t norm_weights, float routed_scaling_factor,
                                             moe_group_score_t group_score, void* stream);

/*
 * moe_create_indices_workspace_size
 * Bytes of device workspace moe_create_indices needs for N slots and E
 * experts (0 when none is needed, and for N or E out of range). The size
 * never decreases as N grows, so a buffer sized for the largest N serves
 * every smaller one. Pure host computation; never fails.
 */
size_t moe_create_indices_workspace_size(int64_t N, int32_t E);

/*
 * moe_create_indices
 * Follows the moe_create_indices page (Modular MAX Mojo API, nn/moe):
 * description (bucket sort grouping tokens by expert so each expert's
 * tokens are contiguous) and Args.
 *
 *   token_expert_order    out uint32 [N]: slot indices i = t*K + k grouped
 *                         by expert; experts ascending, and within an
 *                         expert ascending i (stable).
 *   expert_start_indices  out uint32 [E + 1]: CSR offsets of the active
 *                         experts in token_expert_order; entry A (A = number
 *                         of active experts) is N, entries after A are N.
 *   restore_token_order   out uint32 [N]: position of slot i in
 *                         token_expert_order (token_expert_order[restore[i]]
 *                         == i).
 *   expert_ids            out int32 [E]: active expert ids ascending, then -1.
 *   expert_usage_stats    out uint32 [2]: {max slots on one expert, A}.
 *   topk_ids              in int32 [N]: the router's [T, K] indices, flat.
 *   N                     number of slots, 0 <= N < 2^32; E experts, 1..1024.
 *   workspace             device buffer of at least
 *                         moe_create_indices_workspace_size(N, E) bytes
 *                         (may be NULL when that size is 0). Contents on
 *                         entry do not matter; clobbered on exit.
 *   scales_offset_p       must be NULL here (no alignment is known to this
 *                         call); moe_create_indices_aligned produces the
 *                         aligned scale offsets.
 *
 * Precondition: 0 <= topk_ids[i] < E. A slot whose id is out of range is left
 * out of every count, its restore entry is set to 0xFFFFFFFF and the
 * remaining outputs are unspecified but in bounds.
 * Results are deterministic: no output depends on the order in which
 * workgroups run.
 */
moe_status_t moe_create_indices(uint32_t* token_expert_order, uint32_t* expert_start_indices,
                                uint32_t* restore_token_order, int32_t* expert_ids,
                                uint32_t* expert_usage_stats, const int32_t* topk_ids,
                                int64_t N, int32_t E, void* workspace, size_t workspace_bytes,
                                uint32_t* scales_offset_p, void* stream);

/*
 * moe_create_indices_aligned
 * moe_create_indices plus the page's optional output scales_offset_p (Args:
 * per-expert offsets of the scale rows that an FP8 / block-scaled grouped
 * matmul reads, aligned), padded the way the TokenFormat page's
 * pad_expert_offsets rounds offsets up to the grouped matmul's alignment.
 * The pages name no alignment, so it is an argument.
 *
 *   scales_offset   out uint32 [E + 1], required: entry j = start of active
 *                   expert j's block of scale rows when every active expert's
 *                   row count is rounded up to a multiple of scale_align
 *                   (experts in expert_ids order); entry A (A = active
 *                   experts) is the padded total, entries after A repeat it.
 *   scale_align     rows per scale block, >= 1; N + E * (scale_align - 1)
 *                   must stay below 2^32. With scale_align = 1 the offsets
 *                   equal expert_start_indices.
 *   all other arguments and outputs as moe_create_indices.
 */
moe_status_t moe_create_indices_aligned(uint32_t* token_expert_order,
                                        uint32_t* expert_start_indices,
                                        uint32_t* restore_token_order, int32_t* expert_ids,
                                        uint32_t* expert_usage_stats, const int32_t* topk_ids,
                                        int64_t N, int32_t E, void* workspace,
                                        size_t workspace_bytes, uint32_t* scales_offset,
                                        uint32_t scale_align, void* stream);

/*
 * moe_create_indices_no_alloc
 * For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): moe_create_indices with its counts matrix in a device array
 * the library owns instead of a caller workspace. The call itself allocates
 * nothing (no hipMalloc / hipFree or allocating library routine); the array
 * is moe_create_indices_no_alloc_max_scratch_bytes() = 256 KiB (64 chunks x
 * 1024 experts of uint32), held on each GPU the library runs on until the
 * process ends. Its address is looked up once per device, on the first call
 * made with that device current.
 *
 * Arguments, outputs, validation and determinism as moe_create_indices,
 * without workspace and scales_offset_p. Every valid (N, E) fits the array;
 * a plan that would not returns MOE_ERR_WORKSPACE. MOE_ERR_HIP if the
 * array's address cannot be obtained.
 *
 * All calls on one GPU share that GPU's array, which keeps the last call's
 * contents (nothing in it needs to be zero on entry). Calls that may overlap
 * on one GPU (different streams without ordering, several host threads)
 * race on it and give wrong outputs: serialise them.
 */
moe_status_t moe_create_indices_no_alloc(uint32_t* token_expert_order,
                                         uint32_t* expert_start_indices,
                                         uint32_t* restore_token_order, int32_t* expert_ids,
                                         uint32_t* expert_usage_stats, const int32_t* topk_ids,
                                         int64_t N, int32_t E, void* stream);

/* Size in bytes of the device array moe_create_indices_no_alloc uses. */
size_t moe_create_indices_no_alloc_max_scratch_bytes(void);

/*
 * moe_route_and_index_workspace_size
 * Bytes of device workspace moe_route_and_index needs for T tokens, K slots
 * per token and E experts: a 256-byte header (a counter word and the status
 * word). When E <= 256 and the batch takes two launches, plus a uint32
 * counts matrix of 64 rows of E' words (E' = E rounded up to a multiple of
 * 4) and min(ceil(T / 4), 32768) scratch rows of E' words (one per router
 * workgroup, which routes at least 4 tokens). Otherwise, when the index
 * step may split the T * K slots into several chunks, plus a counts matrix
 * of 64 rows of E words. Never decreases as T grows. 0 for arguments out
 * of range. Pure host computation.
 */
size_t moe_route_and_index_workspace_size(int64_t T, int32_t K, int32_t E);

/*
 * moe_route_and_index
 * The router (moe_router_group_limited, or moe_router_group_limited_logits
 * when score_fn is not MOE_SCORE_NONE) and moe_create_indices_aligned /
 * moe_create_indices on its expert_indices, with fewer launches. Every
 * output is bit-identical to what the two separate calls produce on the
 * same inputs.
 *   - E a power of two and T no larger than one router workgroup's share
 *     (16 tokens for E in 64..256, 8 for 512, 4 for 1024, 64 * 16 / E
 *     below 64): one launch, that workgroup routing every token and then
 *     building the index outputs;
 *   - otherwise two launches. For E <= 256, batches of more than one
 *     index chunk and at most 32768 router workgroups, and a 16-byte
 *     aligned workspace (ranked form),
 *     the router also ranks each slot
 *     among the earlier slots of its workgroup with the same expert and
 *     records each workgroup's count per expert (scratch in the workspace
 *     and in restore_token_order), so that the index step places every
 *     slot directly; above one index chunk it also adds the counts into
 *     the workspace's counts matrix (relaxed atomic adds). Otherwise
 *     (chunked form) the router counts each chunk's slots per expert into
 *     that matrix, so the index step needs no histogram pass of its own.
 *     In both, the index step's last workgroup clears the matrix again.
 *
 *   expert_indices, expert_weights       out as moe_router_group_limited.
 *   token_expert_order ... expert_usage_stats
 *                                        out as moe_create_indices, with
 *                                        N = T * K.
 *   scales_offset, scale_align           as moe_create_indices_aligned;
 *                                        scales_offset may be NULL (no
 *                                        aligned offsets, scale_align
 *                                        ignored).
 *   router_input     in [T, E], input_dtype: scores (score_fn =
 *                    MOE_SCORE_NONE) or logits (MOE_SCORE_SIGMOID /
 *                    MOE_SCORE_SOFTMAX).
 *   expert_bias, scalars                 as moe_router_group_limited.
 *   workspace        device buffer of at least
 *                    moe_route_and_index_workspace_size(T, K, E) bytes,
 *                    4-byte aligned, ZERO-FILLED before its first use. Its
 *                    first 256 + 64 * E' * 4 bytes, E' = E rounded up to a
 *                    multiple of 4 (or all of it, if it is
 *                    smaller) hold a header and a counts matrix that every
 *                    call returning MOE_OK leaves zero again, except the
 *                    status word below; bytes past them are scratch that a
 *                    call may leave holding anything. A buffer sized for the
 *                    largest batch serves every smaller one (the size never
 *                    decreases as T grows). Calls that share a workspace
 *                    must not run concurrently (one stream, or ordered
 *                    streams). After a call that returned MOE_ERR_HIP the
 *                    workspace must be zero-filled again before the next
 *                    call (the router may have counted into it).
 *
 * Status word. The uint32 at byte offset MOE_ROUTE_INDEX_STATUS_OFFSET of
 * the workspace is never cleared by the library. When the index step finds
 * that the counts matrix it was handed does not add up to T * K (the
 * workspace was not zero on entry) it stores MOE_STATUS_COUNTS_MISMATCH
 * there; the index outputs of that call are then unspecified (but written
 * in bounds) and the matrix is still cleared, so the next call starts
 * clean. The caller may read the word (e.g. copy it to the host after the
 * stream has finished) and reset it to 0. Only calls whose index step has
 * several chunks use the matrix, so only they can report this.
 *
 * Validation: that of the two separate calls, and the workspace size. With T = 0 only the index
 * metadata outputs are written, as moe_create_indices does for N = 0.
 */
#define MOE_ROUTE_INDEX_STATUS_OFFSET 4
#define MOE_STATUS_COUNTS_MISMATCH 1u

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
                                 size_t workspace_bytes, void* stream);

/*
 * moe_finalize
 * Follows the moe_finalize page (Modular MAX Mojo API, nn/moe): description
 * (unpermute gather through restore_order, each row scaled by its router
 * weight, fp32 accumulation, the [T, K, H] unpermuted tensor never formed)
 * and Args.
 *
 *   output         out [T, H], out_dtype.
 *   down           in [T*K, H], down_dtype: expert outputs in
 *                  token_expert_order row order.
 *   restore_order  in uint32 [T*K]: row of `down` for slot i = t*K + k.
 *   router_weight  in [T, K], weight_dtype.
 *
 * output[t, h] = convert(sum_k w[t,k] * down[restore[t*K+k], h]) with the
 * sum formed in fp32 from +0 by one fused multiply-add per k in ascending k;
 * conversion to bf16 / fp16 rounds to nearest even.
 *
 * Validation: T >= 0, K >= 1, H >= 0, T*K < 2^32; dtypes in {F32, BF16,
 * F16}, any combination; an output row below 2^31 bytes and
 * T * ceil(H * sizeof(down_dtype) / 1024) below 2^32 - 2^18 (larger:
 * MOE_ERR_UNSUPPORTED); H * sizeof(down_dtype) a multiple of 16 bytes;
 * output and down 16-byte aligned; non-NULL pointers when T*H > 0.
 * Precondition: restore_order[i] < T*K (an out-of-range entry contributes
 * nothing; the output is then unspecified but no access leaves `down`).
 */
moe_status_t moe_finalize(void* output, moe_dtype_t out_dtype, const void* down,
                          moe_dtype_t down_dtype, const uint32_t* restore_order,
                          const void* router_weight, moe_dtype_t weight_dtype, int64_t T,
                          int32_t K, int64_t H, void* stream);

/* Human-readable name of a status code (static string). */
const char* moe_status_string(moe_status_t status);

/* hipError_t value behind the most recent MOE_ERR_HIP returned on this
 * thread (0 if none). */
int moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H */
