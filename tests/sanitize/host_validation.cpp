// Host validation of the C ABI, built host-only with AddressSanitizer and
// UndefinedBehaviorSanitizer: api.hip and plan.hip are linked
// against the stub launchers below, which record what would have been
// launched instead of touching a GPU. Every case checks the status code and
// whether a launch was reached; extreme sizes exercise the overflow guards.
// Prints "host validation ok" and exits 0 when every case holds.
#include <limits.h>
#include <stdio.h>
#include <stdlib.h>

#include "common.hpp"

namespace {
int g_router = 0, g_indices = 0, g_route_index = 0, g_finalize = 0, g_ranked = 0;
int g_fail = 0;
moe::IndexPlan g_last_plan{};
bool g_last_counts_ready = false;
const void* g_last_counts = nullptr;

void reset() { g_router = g_indices = g_route_index = g_finalize = g_ranked = 0; }
int launches() { return g_router + g_indices + g_route_index + g_finalize + g_ranked; }

#define EXPECT(cond)                                                \
  do {                                                              \
    if (!(cond)) {                                                  \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                     \
    }                                                               \
  } while (0)
}  // namespace

namespace moe {
moe_status_t launch_router(int32_t*, void*, const void*, const void*, moe_dtype_t, moe_dtype_t,
                           int32_t, int64_t T, int32_t E, int32_t K, int32_t, int32_t, int32_t,
                           float, int32_t, RouterHist, hipStream_t) {
  EXPECT(T > 0 && E >= 1 && K >= 1);
  ++g_router;
  return MOE_OK;
}
moe_status_t launch_indices(uint32_t*, uint32_t*, uint32_t*, int32_t*, uint32_t*, uint32_t*,
                            uint32_t, const int32_t*, int64_t N, int32_t E, void* workspace,
                            const IndexPlan& plan, bool counts_ready, uint32_t*, hipStream_t) {
  EXPECT(N >= 0 && E >= 1 && plan.nchunks >= 1 && plan.nchunks <= kMaxChunks);
  EXPECT(plan.nchunks == 1 || workspace != nullptr);
  EXPECT(plan.chunk * plan.nchunks >= N);
  g_last_plan = plan;
  g_last_counts_ready = counts_ready;
  g_last_counts = workspace;
  ++g_indices;
  return MOE_OK;
}
moe_status_t launch_indices_ranked(uint32_t*, uint32_t*, uint32_t*, int32_t*, uint32_t*,
                                   uint32_t*, uint32_t, int64_t N, int32_t E, const uint32_t* fine,
                                   uint32_t* counts, uint32_t* ticket, const RankedPlan& plan,
                                   hipStream_t) {
  EXPECT(plan.ok && N >= 1 && E >= 1 && E <= kRankedMaxExperts && fine != nullptr);
  EXPECT(plan.nchunks >= 1 && plan.nchunks <= kMaxChunks && plan.R <= kRankedMaxRowsPerChunk);
  EXPECT(static_cast<int64_t>(plan.rows) * plan.F >= N);
  EXPECT((plan.nchunks > 1) == (counts != nullptr) && ticket != nullptr);
  g_last_plan.nchunks = plan.nchunks;
  g_last_counts_ready = true;
  g_last_counts = counts;
  ++g_ranked;
  return MOE_OK;
}
moe_status_t launch_route_index(int32_t*, void*, const void*, const void*, moe_dtype_t,
                                moe_dtype_t, int32_t, int64_t T, int32_t E, int32_t, int32_t,
                                int32_t, int32_t, float, int32_t, uint32_t*, uint32_t*, uint32_t*,
                                int32_t*, uint32_t*, uint32_t*, uint32_t, hipStream_t) {
  EXPECT(T >= 1 && T <= route_index_max_tokens(E));
  ++g_route_index;
  return MOE_OK;
}
moe_status_t launch_finalize(void*, moe_dtype_t, const void*, moe_dtype_t, const uint32_t*,
                             const void*, moe_dtype_t, int64_t T, int32_t K, int64_t H,
                             hipStream_t) {
  EXPECT(T > 0 && K >= 1 && H > 0);
  ++g_finalize;
  return MOE_OK;
}
}  // namespace moe

namespace {
// Never dereferenced: every case either fails validation or reaches a stub.
void* const P = reinterpret_cast<void*>(0x10000);
void* const P_MIS = reinterpret_cast<void*>(0x10004);
void* const P_ODD = reinterpret_cast<void*>(0x10002);
int32_t* const I = static_cast<int32_t*>(P);
uint32_t* const U = static_cast<uint32_t*>(P);

moe_status_t router(int64_t T, int32_t E, int32_t K, int32_t G, int32_t TG, int mode = 0,
                    void* scores = P, moe_dtype_t sd = MOE_DTYPE_F32,
                    moe_dtype_t bd = MOE_DTYPE_F32) {
  return moe_router_group_limited(I, P, scores, P, sd, bd, T, E, K, G, TG, 1, 1.0f,
                                  static_cast<moe_group_score_t>(mode), nullptr);
}

moe_status_t indices(int64_t N, int32_t E, void* ws, size_t ws_bytes) {
  return moe_create_indices(U, U, U, I, U, I, N, E, ws, ws_bytes, nullptr, nullptr);
}

moe_status_t route_index(int64_t T, int32_t E, int32_t K, void* ws, size_t ws_bytes) {
  return moe_route_and_index(I, P, U, U, U, I, U, nullptr, 0, P, P, MOE_DTYPE_F32,
                             MOE_DTYPE_F32, MOE_SCORE_NONE, T, E, K, 8, 4, 1, 2.5f,
                             MOE_GROUP_TOP2_SUM, ws, ws_bytes, nullptr);
}

moe_status_t finalize(int64_t T, int32_t K, int64_t H, moe_dtype_t od = MOE_DTYPE_BF16,
                      moe_dtype_t dd = MOE_DTYPE_BF16, void* out = P) {
  return moe_finalize(out, od, P, dd, U, P, MOE_DTYPE_F32, T, K, H, nullptr);
}
}  // namespace

int main() {
  // router: rejections reach no launch
  const int64_t big[] = {-1, INT64_MIN, (int64_t)UINT32_MAX + 1, INT64_MAX};
  for (int64_t T : big) {
    reset();
    EXPECT(router(T, 256, 8, 8, 4) == MOE_ERR_INVALID_ARG);
    EXPECT(launches() == 0);
  }
  reset();
  EXPECT(router(4, 256, 8, 3, 1) == MOE_ERR_INVALID_ARG);        // E % n_groups
  EXPECT(router(4, 256, 0, 8, 4) == MOE_ERR_INVALID_ARG);        // K = 0
  EXPECT(router(4, 256, INT32_MAX, 8, 4) == MOE_ERR_INVALID_ARG);
  EXPECT(router(4, 256, 8, 8, 9) == MOE_ERR_INVALID_ARG);        // topk_group > n_groups
  EXPECT(router(4, INT32_MAX, 8, 1, 1) == MOE_ERR_UNSUPPORTED);  // E above 1024
  EXPECT(router(4, 256, 8, 8, 4, 2) == MOE_ERR_INVALID_ARG);     // group-score mode
  EXPECT(router(4, 256, 8, 8, 4, 0, P_MIS) == MOE_ERR_ALIGNMENT);
  EXPECT(router(4, 256, 8, 8, 4, 0, P, MOE_DTYPE_BF16, MOE_DTYPE_F16) == MOE_ERR_UNSUPPORTED);
  EXPECT(router(4, 256, 8, 8, 4, 0, P, static_cast<moe_dtype_t>(7)) == MOE_ERR_INVALID_ARG);
  EXPECT(router((int64_t)UINT32_MAX / 8 + 1, 256, 8, 8, 4) == MOE_ERR_INVALID_ARG);  // T*K >= 2^32
  EXPECT(launches() == 0);
  EXPECT(router(0, 256, 8, 8, 4) == MOE_OK && launches() == 0);  // T = 0: nothing launched
  EXPECT(router(4, 256, 8, 8, 4) == MOE_OK && g_router == 1);
  EXPECT(router(4, 160, 6, 8, 3) == MOE_OK && g_router == 2);   // general-E form
  EXPECT(moe_router_group_limited_logits(I, P, P, P, MOE_DTYPE_F32, MOE_DTYPE_F32,
                                         MOE_SCORE_NONE, 4, 256, 8, 8, 4, 1, 1.0f,
                                         MOE_GROUP_TOP2_SUM, nullptr) == MOE_ERR_INVALID_ARG);

  // index creation
  reset();
  EXPECT(indices(-1, 256, P, 1 << 20) == MOE_ERR_INVALID_ARG);
  EXPECT(indices(INT64_MAX, 256, P, 1 << 20) == MOE_ERR_INVALID_ARG);
  EXPECT(indices((int64_t)1 << 32, 256, P, 1 << 20) == MOE_ERR_INVALID_ARG);
  EXPECT(indices(100, 0, P, 1 << 20) == MOE_ERR_INVALID_ARG);
  EXPECT(indices(100, 1025, P, 1 << 20) == MOE_ERR_INVALID_ARG);
  EXPECT(indices(65536, 256, P, 16) == MOE_ERR_WORKSPACE);
  EXPECT(indices(65536, 256, nullptr, 1 << 20) == MOE_ERR_WORKSPACE);
  EXPECT(indices(65536, 256, P_ODD, 1 << 20) == MOE_ERR_ALIGNMENT);
  EXPECT(moe_create_indices(U, U, U, I, U, I, 100, 256, P, 1 << 20, U, nullptr) ==
         MOE_ERR_UNSUPPORTED);
  EXPECT(launches() == 0);
  EXPECT(indices(100, 256, nullptr, 0) == MOE_OK && g_indices == 1 && g_last_plan.nchunks == 1);
  EXPECT(indices((int64_t)UINT32_MAX, 1024, P, moe_create_indices_workspace_size(
                                                    (int64_t)UINT32_MAX, 1024)) == MOE_OK);
  EXPECT(g_last_plan.nchunks > 1 && !g_last_counts_ready);
  EXPECT(moe_create_indices_aligned(U, U, U, I, U, I, 100, 256, P, 1 << 20, U, 0, nullptr) ==
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_create_indices_aligned(U, U, U, I, U, I, (int64_t)UINT32_MAX - 10, 256, P,
                                    (size_t)1 << 30, U, 2, nullptr) == MOE_ERR_INVALID_ARG);
  // workspace sizes: never decreasing, never failing, on any input
  size_t prev_c = 0, prev_r = 0;
  for (int64_t n = 0; n < 300000; n += 7) {
    const size_t c = moe_create_indices_workspace_size(n, 256);
    const size_t r = moe_route_and_index_workspace_size(n, 8, 256);
    EXPECT(c >= prev_c && r >= prev_r);
    prev_c = c;
    prev_r = r;
  }
  EXPECT(moe_create_indices_workspace_size(INT64_MAX, 256) == 0);
  EXPECT(moe_create_indices_workspace_size(INT64_MIN, INT32_MIN) == 0);
  EXPECT(moe_route_and_index_workspace_size(INT64_MAX, INT32_MAX, 256) == 0);
  EXPECT(moe_route_and_index_workspace_size(1, 1, INT32_MAX) == 0);

  // router + index creation
  reset();
  const size_t need = moe_route_and_index_workspace_size(8192, 8, 256);
  EXPECT(need > 256);
  EXPECT(route_index(8192, 256, 8, P, need - 4) == MOE_ERR_WORKSPACE);
  EXPECT(route_index(8192, 256, 8, nullptr, need) == MOE_ERR_WORKSPACE);
  EXPECT(route_index(8192, 256, 8, P_ODD, need) == MOE_ERR_ALIGNMENT);
  EXPECT(route_index(INT64_MAX, 256, 8, P, need) == MOE_ERR_INVALID_ARG);
  EXPECT(launches() == 0);
  EXPECT(route_index(16, 256, 8, P, 256) == MOE_OK && g_route_index == 1 && g_router == 0);
  // ranked form: router, then the ranked index step over several chunks
  EXPECT(route_index(8192, 256, 8, P, need) == MOE_OK && g_router == 1 && g_ranked == 1);
  EXPECT(g_last_counts_ready && g_last_plan.nchunks > 1);
  EXPECT(g_last_counts == static_cast<const char*>(P) + 256);  // the matrix follows the header
  // one index chunk: the chunked form's single-workgroup index step
  reset();
  EXPECT(route_index(128, 256, 8, P, moe_route_and_index_workspace_size(128, 8, 256)) == MOE_OK);
  EXPECT(g_ranked == 0 && g_indices == 1 && g_last_plan.nchunks == 1 && !g_last_counts_ready);
  // a workspace that is not 16-byte aligned: chunked form
  reset();
  EXPECT(route_index(8192, 256, 8, static_cast<char*>(P) + 4, need) == MOE_OK);
  EXPECT(g_ranked == 0 && g_indices == 1 && g_last_counts_ready);
  // E above 256: chunked form
  reset();
  const size_t need512 = moe_route_and_index_workspace_size(8192, 8, 512);
  EXPECT(moe_route_and_index(I, P, U, U, U, I, U, nullptr, 0, P, P, MOE_DTYPE_F32, MOE_DTYPE_F32,
                             MOE_SCORE_NONE, 8192, 512, 8, 8, 4, 1, 2.5f, MOE_GROUP_TOP2_SUM, P,
                             need512, nullptr) == MOE_OK);
  EXPECT(g_router == 1 && g_indices == 1 && g_ranked == 0 && g_last_counts_ready);

  // finalize
  reset();
  EXPECT(finalize(-1, 8, 7168) == MOE_ERR_INVALID_ARG);
  EXPECT(finalize(4, 0, 7168) == MOE_ERR_INVALID_ARG);
  EXPECT(finalize(4, 8, -1) == MOE_ERR_INVALID_ARG);
  EXPECT(finalize(INT64_MAX, 8, 7168) == MOE_ERR_INVALID_ARG);
  EXPECT(finalize(4, 8, INT64_MAX) == MOE_ERR_UNSUPPORTED);
  EXPECT(finalize(4, 8, INT32_MAX) == MOE_ERR_UNSUPPORTED);
  EXPECT(finalize(4, 8, 7164) == MOE_ERR_ALIGNMENT);  // row not a multiple of 16 bytes
  EXPECT(finalize(4, 8, 7168, MOE_DTYPE_BF16, MOE_DTYPE_BF16, P_MIS) == MOE_ERR_ALIGNMENT);
  EXPECT(finalize(4, 8, 7168, static_cast<moe_dtype_t>(3)) == MOE_ERR_INVALID_ARG);
  EXPECT(launches() == 0);
  EXPECT(finalize(0, 8, 7168) == MOE_OK && finalize(4, 8, 0) == MOE_OK && launches() == 0);
  EXPECT(finalize(4, 8, 7168) == MOE_OK && g_finalize == 1);

  for (int s = -1; s <= 7; ++s) EXPECT(moe_status_string(static_cast<moe_status_t>(s)) != nullptr);
  EXPECT(moe_last_hip_error() == 0);

  if (g_fail) {
    fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  printf("host validation ok\n");
  return 0;
}
