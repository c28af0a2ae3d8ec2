/*
 * CPU oracle for the group-limited MoE routing data path.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously correct
 * reference that the GPU library is checked against. Only the test suite,
 * the package smoke check and the benchmark's CPU-baseline leg may load it.
 * The product path (the HIP library and its Python binding) never calls it
 * and shares no source, header, table or helper with it.
 *
 * Built with plain gcc, -O2 -ffp-contract=off, no fast-math, so every
 * floating-point operation below is one IEEE-754 binary32/binary64 operation
 * rounded to nearest-even, in exactly the order written.
 *
 * The three computations follow the Modular MAX Mojo API pages:
 *   - group_limited_router_kernel page: description, Parameters
 *     (n_groups, topk_group, n_experts_per_tok, norm_weights) and Args
 *     (expert_indices, expert_weights, expert_scores, expert_bias,
 *     routed_scaling_factor);
 *   - moe_create_indices page: description (bucket sort grouping tokens by
 *     expert) and Args (token_expert_order, expert_start_indices,
 *     restore_token_order, expert_ids, expert_usage_stats, topk_ids);
 *   - moe_finalize page: description (unpermute gather through
 *     restore_order, scale by router weight, fp32 accumulation) and Args.
 * Points the pages leave open are resolved as written next to each step.
 *
 * Pins (tests that tie this file to something other than itself):
 *   router   - brute force with Python's sorted() on tiny shapes and
 *              exhaustive tie grids, torch.topk for n_groups == 1,
 *              softmax closed form, hand-worked fixtures, invariants;
 *   indices  - numpy stable argsort / bincount / cumsum, brute force,
 *              invariants;
 *   finalize - float64 numpy reference within the FMA-chain error bound,
 *              exact gather special cases; bf16 rounding against torch.
 * The group score ("top-2 sum" versus "max") is a reading of a silent
 * point; both modes are pinned only against their written definitions.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Oracle-local constants. They mirror nothing: the Python wrapper passes
 * these numbers explicitly. */
enum { OR_F32 = 0, OR_BF16 = 1, OR_F16 = 2 };
enum { OR_GROUP_TOP2_SUM = 0, OR_GROUP_MAX = 1 };
enum { OR_SCORE_LOAD = 0, OR_SCORE_SIGMOID = 1, OR_SCORE_SOFTMAX = 2 };
enum { OR_OK = 0, OR_BAD_ARG = 1, OR_BAD_DATA = 2, OR_NO_MEM = 3 };

int moe_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following parallel loops (results do not depend on it). */
void moe_oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------ */
/* bfloat16 helpers                                                   */
/* ------------------------------------------------------------------ */

/* bf16 is the high half of a binary32; widening is exact. */
static float bf16_bits_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> bf16, round to nearest, ties to even (the pages do not name
 * the rounding of the fp32 accumulator into out_type; RNE is the IEEE
 * default). NaN stays NaN (quiet bit forced); infinities and overflow
 * follow from the arithmetic. */
uint16_t moe_oracle_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

void moe_oracle_f32_to_bf16_array(uint16_t* out, const float* in, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = moe_oracle_f32_to_bf16(in[i]);
}

/* IEEE binary16 -> binary32, exact. */
static float f16_bits_to_f32(uint16_t h) {
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    const uint32_t ex = (h >> 10) & 0x1fu;
    const uint32_t man = h & 0x3ffu;
    float f;
    if (ex == 0) { /* zero or subnormal: man * 2^-24 */
        f = ldexpf((float)man, -24);
        return sign ? -f : f;
    }
    uint32_t u;
    if (ex == 31)
        u = sign | 0x7f800000u | (man << 13); /* infinity or NaN */
    else
        u = sign | ((ex + 112u) << 23) | (man << 13); /* rebias 15 -> 127 */
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> binary16, round to nearest, ties to even; overflow gives
 * infinity, tiny values become subnormals or zero. */
uint16_t moe_oracle_f32_to_f16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);  /* NaN */
    if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u); /* >= 65520: infinity */
    if (a < 0x38800000u) {                                   /* below 2^-14: subnormal */
        const float scaled = fabsf(f) * 16777216.0f;          /* exact: times 2^24 */
        return (uint16_t)(sign | (uint16_t)nearbyintf(scaled));
    }
    const uint32_t rounded = a + 0x0fffu + ((a >> 13) & 1u); /* nearest even at bit 13 */
    return (uint16_t)(sign | ((rounded - 0x38000000u) >> 13));
}

void moe_oracle_f32_to_f16_array(uint16_t* out, const float* in, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = moe_oracle_f32_to_f16(in[i]);
}

void moe_oracle_f16_to_f32_array(float* out, const uint16_t* in, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = f16_bits_to_f32(in[i]);
}

static float load_as_f32(const void* p, int dtype, int64_t i) {
    if (dtype == OR_F32) return ((const float*)p)[i];
    if (dtype == OR_F16) return f16_bits_to_f32(((const uint16_t*)p)[i]);
    return bf16_bits_to_f32(((const uint16_t*)p)[i]);
}

static void store_from_f32(void* p, int dtype, int64_t i, float v) {
    if (dtype == OR_F32)
        ((float*)p)[i] = v;
    else if (dtype == OR_F16)
        ((uint16_t*)p)[i] = moe_oracle_f32_to_f16(v);
    else
        ((uint16_t*)p)[i] = moe_oracle_f32_to_bf16(v);
}

static int dtype_ok(int d) { return d == OR_F32 || d == OR_BF16 || d == OR_F16; }

/* ------------------------------------------------------------------ */
/* Router (group_limited_router_kernel page)                          */
/* ------------------------------------------------------------------ */

typedef struct {
    float v;
    int32_t id;
} keyed_t;

/* Order: larger value first; equal values (IEEE equality, so -0 == +0)
 * keep the lower index first. The pages do not state a tie rule; lower
 * index wins is the reading used throughout. */
static int keyed_desc(const void* a, const void* b) {
    const keyed_t* x = (const keyed_t*)a;
    const keyed_t* y = (const keyed_t*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    if (x->id < y->id) return -1;
    if (x->id > y->id) return 1;
    return 0;
}

/*
 * expert_indices [T, K] int32 and expert_weights [T, K] from expert_scores
 * [T, E] and expert_bias [E]. Scores and bias may be fp32, bf16 or fp16
 * (scores_type and bias_type on the page); both are widened exactly to
 * binary32. The weights are written in the scores' dtype (the page gives
 * expert_weights the scores_type).
 *
 * Per token (router page, description):
 *  1. biased score b[e] = score[e] + bias[e], one binary32 add; the bias is
 *     used for selection only.
 *  2. the E experts form n_groups consecutive groups of S = E / n_groups
 *     (E divisible by n_groups, Parameters: n_groups). The page keeps the
 *     topk_group best-scoring groups without defining a group's score; the
 *     group score is, by reading, the sum of the two largest biased scores
 *     of the group (group_score = 0) or the single largest (group_score = 1).
 *     With S == 1 both are the single score.
 *  3. keep the first topk_group groups in (group score desc, group asc).
 *  4. among experts of kept groups, take the first K in (b desc, e asc);
 *     slot k of the token holds the k-th.
 *  5. weights from the unbiased scores u_k = score[e_k]. With norm_weights
 *     they are divided by their sum before the scaling factor is applied
 *     (Parameters: norm_weights; Args: routed_scaling_factor). This step is
 *     evaluated in binary64, rounded to binary32, then to the output dtype.
 */
/*
 * Binary64 exponential of the score functions. Not libm's exp, whose last
 * bit is the library's own choice, but a fixed published method, so that
 * any implementation of the same steps produces the same bits:
 *   - argument reduction of Cody and Waite (Software Manual for the
 *     Elementary Functions, 1980): k = x / ln2 rounded to the nearest
 *     integer (ties to even), r = (x - k * LN2_HI) - k * LN2_LO, each
 *     subtraction one fused multiply-add, with LN2_HI the binary64 value
 *     nearest ln 2 and LN2_LO the binary64 value nearest ln 2 - LN2_HI;
 *   - exp(r) by its Taylor series about 0 up to r^13 / 13! (|r| <= ln2 / 2
 *     leaves a remainder below 2^-56 relative), evaluated by Horner's rule
 *     from the highest power down, one fused multiply-add per term; the
 *     coefficient of r^n is 1 / n! rounded once (n! is exact in binary64);
 *   - scaling by 2^k as two exact powers of two, 2^(k/2) then
 *     2^(k - k/2) (k/2 truncated towards zero), so only the last product
 *     rounds (into the subnormal range or to infinity).
 * Outside [-745.2, 709.78] the result is 0 or +inf; NaN stays NaN.
 * Within two binary64 ulps of exp(x) (pinned against a correctly rounded
 * reference).
 */
double moe_oracle_exp(double x) {
    const double LN2_HI = 0x1.62e42fefa39efp-1;
    const double LN2_LO = 0x1.abc9e3b39803fp-56;
    const double INV_LN2 = 0x1.71547652b82fep+0;
    if (x != x) return x;
    if (x > 709.78) return INFINITY;
    if (x < -745.2) return 0.0;
    const double kd = rint(x * INV_LN2);
    double r = fma(-kd, LN2_HI, x);
    r = fma(-kd, LN2_LO, r);
    double fact = 1.0;
    for (int n = 2; n <= 13; ++n) fact *= (double)n; /* 13!, exact */
    double p = 1.0 / fact;
    for (int n = 12; n >= 0; --n) {
        fact /= (double)(n + 1); /* n!, exact */
        p = fma(p, r, 1.0 / fact);
    }
    const int k = (int)kd;
    const int k1 = k / 2, k2 = k - k1;
    return (p * ldexp(1.0, k1)) * ldexp(1.0, k2);
}

/*
 * Sum of v[0..n) in binary64 as a balanced pairwise tree in index order:
 * the values padded with zeros to the next power of two P, then for
 * w = 1, 2, 4, ... < P every t[i] with i a multiple of 2w becomes
 * t[i] + t[i + w]; the sum is t[0]. Adding the zero padding is exact, so
 * the result depends only on v (and equals the same tree over any larger
 * power of two).
 */
double moe_oracle_pairwise_sum(const double* v, int64_t n) {
    if (n <= 0) return 0.0;
    int64_t P = 1;
    while (P < n) P *= 2;
    double* t = (double*)calloc((size_t)P, sizeof(double));
    if (!t) return NAN;
    for (int64_t i = 0; i < n; ++i) t[i] = v[i];
    for (int64_t w = 1; w < P; w *= 2)
        for (int64_t i = 0; i < P; i += 2 * w) t[i] = t[i] + t[i + w];
    const double s = t[0];
    free(t);
    return s;
}

/*
 * Routing scores of one token (router page, Parameters: scores_input_fn, an
 * optional loader of the scores of a (token, expert) pair). score_fn 0
 * loads them from the input; 1 and 2 compute them from the input taken as
 * logits: 1 is the logistic sigmoid 1 / (1 + exp(-x)) of each logit, 2 the
 * softmax over the token's E logits, exp(x_e - max) / sum_j exp(x_j - max).
 * Both are evaluated in binary64 with moe_oracle_exp (the softmax
 * denominator as the pairwise sum above, over experts in index order) and
 * rounded once to binary32, the scores' working precision.
 */
static void token_scores(float* s, double* ex, const void* in, int32_t dtype, int32_t score_fn,
                         int64_t t, int32_t E) {
    for (int32_t e = 0; e < E; ++e) s[e] = load_as_f32(in, dtype, t * (int64_t)E + e);
    if (score_fn == OR_SCORE_SIGMOID) {
        for (int32_t e = 0; e < E; ++e) s[e] = (float)(1.0 / (1.0 + moe_oracle_exp(-(double)s[e])));
    } else if (score_fn == OR_SCORE_SOFTMAX) {
        double m = (double)s[0];
        for (int32_t e = 1; e < E; ++e)
            if ((double)s[e] > m) m = (double)s[e];
        for (int32_t e = 0; e < E; ++e) ex[e] = moe_oracle_exp((double)s[e] - m);
        const double sum = moe_oracle_pairwise_sum(ex, E);
        for (int32_t e = 0; e < E; ++e) s[e] = (float)(ex[e] / sum);
    }
}

int moe_oracle_router(int32_t* expert_indices, void* expert_weights, const void* scores,
                      const void* bias, int32_t scores_dtype, int32_t bias_dtype, int64_t T,
                      int32_t E, int32_t K, int32_t n_groups, int32_t topk_group,
                      int32_t norm_weights, float routed_scaling_factor, int32_t group_score,
                      int32_t score_fn) {
    if (T < 0 || E <= 0 || n_groups <= 0 || E % n_groups != 0) return OR_BAD_ARG;
    if (score_fn != OR_SCORE_LOAD && score_fn != OR_SCORE_SIGMOID && score_fn != OR_SCORE_SOFTMAX)
        return OR_BAD_ARG;
    if (topk_group < 1 || topk_group > n_groups) return OR_BAD_ARG;
    const int32_t S = E / n_groups;
    if (K < 1 || K > topk_group * S) return OR_BAD_ARG;
    if (group_score != OR_GROUP_TOP2_SUM && group_score != OR_GROUP_MAX) return OR_BAD_ARG;
    if (!dtype_ok(scores_dtype) || !dtype_ok(bias_dtype)) return OR_BAD_ARG;

    int rc = OR_OK;
#pragma omp parallel
    {
        float* s = (float*)malloc(sizeof(float) * (size_t)E);
        double* ex = (double*)malloc(sizeof(double) * (size_t)E);
        float* b = (float*)malloc(sizeof(float) * (size_t)E);
        keyed_t* grp = (keyed_t*)malloc(sizeof(keyed_t) * (size_t)S);
        keyed_t* gsc = (keyed_t*)malloc(sizeof(keyed_t) * (size_t)n_groups);
        keyed_t* cand = (keyed_t*)malloc(sizeof(keyed_t) * (size_t)E);
        char* kept = (char*)malloc((size_t)n_groups);
        if (!s || !ex || !b || !grp || !gsc || !cand || !kept) {
#pragma omp atomic write
            rc = OR_NO_MEM;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < T; ++t) {
                /* 1. scores, biased scores */
                token_scores(s, ex, scores, scores_dtype, score_fn, t, E);
                for (int32_t e = 0; e < E; ++e) b[e] = s[e] + load_as_f32(bias, bias_dtype, e);
                /* 2. group scores */
                for (int32_t g = 0; g < n_groups; ++g) {
                    for (int32_t j = 0; j < S; ++j) {
                        grp[j].v = b[g * S + j];
                        grp[j].id = g * S + j;
                    }
                    qsort(grp, (size_t)S, sizeof(keyed_t), keyed_desc);
                    float score = grp[0].v;
                    if (group_score == OR_GROUP_TOP2_SUM && S >= 2) score = grp[0].v + grp[1].v;
                    gsc[g].v = score;
                    gsc[g].id = g;
                }
                /* 3. surviving groups */
                qsort(gsc, (size_t)n_groups, sizeof(keyed_t), keyed_desc);
                memset(kept, 0, (size_t)n_groups);
                for (int32_t r = 0; r < topk_group; ++r) kept[gsc[r].id] = 1;
                /* 4. top-K experts of the surviving groups */
                int32_t nc = 0;
                for (int32_t e = 0; e < E; ++e) {
                    if (kept[e / S]) {
                        cand[nc].v = b[e];
                        cand[nc].id = e;
                        ++nc;
                    }
                }
                qsort(cand, (size_t)nc, sizeof(keyed_t), keyed_desc);
                /* 5. weights from unbiased scores */
                double sum = 0.0;
                for (int32_t k = 0; k < K; ++k) sum += (double)s[cand[k].id];
                for (int32_t k = 0; k < K; ++k) {
                    const int32_t e = cand[k].id;
                    double w = (double)s[e];
                    if (norm_weights) w = w / sum;
                    w = w * (double)routed_scaling_factor;
                    expert_indices[t * K + k] = e;
                    store_from_f32(expert_weights, scores_dtype, t * K + k, (float)w);
                }
            }
        }
        free(s);
        free(ex);
        free(b);
        free(grp);
        free(gsc);
        free(cand);
        free(kept);
    }
    return rc;
}

/* ------------------------------------------------------------------ */
/* Index creation (moe_create_indices page)                            */
/* ------------------------------------------------------------------ */

/*
 * Bucket sort of the N routed slots by expert.
 *
 * topk_ids is the router's [T, K] output viewed flat: slot i = t*K + k
 * holds one expert id (the page calls it 1-D and also says it is reshaped
 * to 2-D; the flat reading serves both). Outputs, by reading of the Args:
 *  - token_expert_order [N]: slot indices grouped by expert; experts in
 *    ascending id, slots of one expert in ascending slot index (a stable
 *    bucket sort). Holding the slot index (not t) is forced by the
 *    moe_finalize page, whose restore_order is indexed by t*K + k.
 *  - restore_token_order [N]: restore[i] = position of slot i in
 *    token_expert_order.
 *  - expert_ids [E]: ids of the experts that received at least one slot,
 *    ascending; the rest of the buffer is -1.
 *  - expert_start_indices [E + 1]: CSR offsets paired with expert_ids:
 *    entry j is where active expert j starts, entry A (A = active count)
 *    is N, and entries after A repeat N.
 *  - expert_usage_stats [2]: {largest slot count of any expert, A}.
 * Every id must lie in [0, E); anything else is reported as bad data.
 */
int moe_oracle_create_indices(uint32_t* token_expert_order, uint32_t* expert_start_indices,
                              uint32_t* restore_token_order, int32_t* expert_ids,
                              uint32_t* expert_usage_stats, const int32_t* topk_ids,
                              int64_t N, int32_t E) {
    if (N < 0 || N > (int64_t)UINT32_MAX || E <= 0) return OR_BAD_ARG;
    for (int64_t i = 0; i < N; ++i)
        if (topk_ids[i] < 0 || topk_ids[i] >= E) return OR_BAD_DATA;

    uint32_t* count = (uint32_t*)calloc((size_t)E, sizeof(uint32_t));
    uint32_t* start = (uint32_t*)calloc((size_t)E, sizeof(uint32_t));
    uint32_t* fill = (uint32_t*)calloc((size_t)E, sizeof(uint32_t));
    if (!count || !start || !fill) {
        free(count);
        free(start);
        free(fill);
        return OR_NO_MEM;
    }
    /* counts per expert */
    for (int64_t i = 0; i < N; ++i) count[topk_ids[i]] += 1;

    /* active experts, compacted, ascending id */
    uint32_t active = 0, largest = 0, offset = 0;
    for (int32_t e = 0; e < E; ++e) {
        start[e] = offset;
        if (count[e] > 0) {
            expert_ids[active] = e;
            expert_start_indices[active] = offset;
            active += 1;
        }
        if (count[e] > largest) largest = count[e];
        offset += count[e];
    }
    for (uint32_t j = active; j < (uint32_t)E; ++j) expert_ids[j] = -1;
    for (uint32_t j = active; j <= (uint32_t)E; ++j) expert_start_indices[j] = (uint32_t)N;

    /* stable placement: walk the slots in ascending order */
    for (int64_t i = 0; i < N; ++i) {
        const int32_t e = topk_ids[i];
        const uint32_t p = start[e] + fill[e];
        fill[e] += 1;
        token_expert_order[p] = (uint32_t)i;
        restore_token_order[i] = p;
    }
    expert_usage_stats[0] = largest;
    expert_usage_stats[1] = active;
    free(count);
    free(start);
    free(fill);
    return OR_OK;
}

/*
 * Aligned scale offsets for a block-scaled grouped matmul (moe_create_indices
 * page, Args: scales_offset_p, aligned offsets of the scale rows; TokenFormat page,
 * pad_expert_offsets: offsets padded to the grouped matmul's alignment).
 * The pages give no alignment, so it is an argument. By reading, entry j of
 * scales_offset [E + 1] is where active expert j's block of scale rows
 * starts when every active expert's row count is rounded up to a multiple
 * of `align`; entry A (A = active experts) is the padded total and the
 * entries after A repeat it. Experts are in the expert_ids order
 * (ascending id).
 */
int moe_oracle_scale_offsets(uint32_t* scales_offset, const int32_t* topk_ids, int64_t N,
                             int32_t E, uint32_t align) {
    if (N < 0 || N > (int64_t)UINT32_MAX || E <= 0 || align == 0) return OR_BAD_ARG;
    for (int64_t i = 0; i < N; ++i)
        if (topk_ids[i] < 0 || topk_ids[i] >= E) return OR_BAD_DATA;
    uint64_t* count = (uint64_t*)calloc((size_t)E, sizeof(uint64_t));
    if (!count) return OR_NO_MEM;
    for (int64_t i = 0; i < N; ++i) count[topk_ids[i]] += 1;
    uint64_t offset = 0;
    uint32_t j = 0;
    for (int32_t e = 0; e < E; ++e) {
        if (count[e] == 0) continue;
        scales_offset[j++] = (uint32_t)offset;
        offset += (count[e] + align - 1) / align * align;
    }
    free(count);
    if (offset > UINT32_MAX) return OR_BAD_ARG;
    for (; j <= (uint32_t)E; ++j) scales_offset[j] = (uint32_t)offset;
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Finalize (moe_finalize page)                                        */
/* ------------------------------------------------------------------ */

/*
 * output[t, h] = sum over k = 0..K-1 of router_weight[t, k] *
 *                down[restore_order[t*K + k], h]
 * accumulated in binary32 (the page keeps the sum in fp32), starting from
 * +0 and adding the K terms in k order, each term fused into the running
 * sum by one correctly rounded fmaf. The accumulator is then stored as
 * out_type (bf16 and fp16 by round to nearest even). down, router_weight
 * and output may each be fp32, bf16 or fp16 (down_type, weight_type,
 * out_type on the page).
 * restore_order entries must lie in [0, T*K).
 */
int moe_oracle_finalize(void* output, int32_t out_dtype, const void* down, int32_t down_dtype,
                        const uint32_t* restore_order, const void* router_weight,
                        int32_t weight_dtype, int64_t T, int32_t K, int64_t H) {
    if (T < 0 || K < 1 || H < 0) return OR_BAD_ARG;
    if (!dtype_ok(out_dtype) || !dtype_ok(down_dtype) || !dtype_ok(weight_dtype))
        return OR_BAD_ARG;
    const int64_t N = T * (int64_t)K;
    for (int64_t i = 0; i < N; ++i)
        if ((int64_t)restore_order[i] >= N) return OR_BAD_DATA;

    int rc = OR_OK;
#pragma omp parallel
    {
        float* acc = (float*)malloc(sizeof(float) * (size_t)(H > 0 ? H : 1));
        if (!acc) {
#pragma omp atomic write
            rc = OR_NO_MEM;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < T; ++t) {
                for (int64_t h = 0; h < H; ++h) acc[h] = 0.0f;
                for (int32_t k = 0; k < K; ++k) {
                    const int64_t row = (int64_t)restore_order[t * K + k];
                    const float w = load_as_f32(router_weight, weight_dtype, t * K + k);
                    for (int64_t h = 0; h < H; ++h)
                        acc[h] = fmaf(w, load_as_f32(down, down_dtype, row * H + h), acc[h]);
                }
                for (int64_t h = 0; h < H; ++h) store_from_f32(output, out_dtype, t * H + h, acc[h]);
            }
        }
        free(acc);
    }
    return rc;
}
