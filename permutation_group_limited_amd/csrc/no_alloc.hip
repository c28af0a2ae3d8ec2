// moe_create_indices for callers that cannot allocate device memory (code
// under HIP graph capture, serving loops, harnesses that forbid it): the
// index step's counts matrix lives in a library-owned device array instead
// of a caller workspace.
//
// The array is a file-scope __device__ variable, so each GPU the library
// runs on holds its own copy from module load until the process ends. In
// host code its name is only a stand-in for the symbol, never a device
// address: the address is fetched once per device with hipGetSymbolAddress
// (with that device current) and only that pointer is handed to kernels.
#include <mutex>

#include "common.hpp"

namespace moe {
namespace {

// [kMaxChunks, 1024] uint32: the largest counts matrix any plan can need
// (at most kMaxChunks chunks, E <= 1024), 256 KiB per GPU.
constexpr size_t kScratchWords = static_cast<size_t>(kMaxChunks) * 1024;
static __device__ __align__(256) uint32_t scratch[kScratchWords];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
uint32_t* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array (looked up on the first call on
// each device); NULL with *err set when the lookup fails.
uint32_t* scratch_on_current_device(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = static_cast<uint32_t*>(p);
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_create_indices_no_alloc_max_scratch_bytes(void) {
  return kScratchWords * sizeof(uint32_t);
}

extern "C" moe_status_t moe_create_indices_no_alloc(
    uint32_t* token_expert_order, uint32_t* expert_start_indices, uint32_t* restore_token_order,
    int32_t* expert_ids, uint32_t* expert_usage_stats, const int32_t* topk_ids, int64_t N,
    int32_t E, void* stream) {
  // same argument checks as moe_create_indices (no workspace to check)
  if (N < 0 || N > static_cast<int64_t>(UINT32_MAX) || E < 1 || E > 1024)
    return MOE_ERR_INVALID_ARG;
  if (!expert_start_indices || !expert_ids || !expert_usage_stats) return MOE_ERR_INVALID_ARG;
  if (N > 0 && (!token_expert_order || !restore_token_order || !topk_ids))
    return MOE_ERR_INVALID_ARG;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(token_expert_order) |
                        reinterpret_cast<uintptr_t>(expert_start_indices) |
                        reinterpret_cast<uintptr_t>(restore_token_order) |
                        reinterpret_cast<uintptr_t>(expert_ids) |
                        reinterpret_cast<uintptr_t>(expert_usage_stats) |
                        reinterpret_cast<uintptr_t>(topk_ids);
  if (mis & 3u) return MOE_ERR_ALIGNMENT;
  const IndexPlan plan = plan_indices(N, E);
  if (plan.workspace_bytes > kScratchWords * sizeof(uint32_t))
    return MOE_ERR_WORKSPACE;  // cannot happen for valid N and E; kept as the size limit
  uint32_t* counts = nullptr;
  if (plan.nchunks > 1) {
    hipError_t err = hipSuccess;
    counts = scratch_on_current_device(&err);
    if (counts == nullptr) return hip_failure(err);
  }
  // the histogram launch writes every row of the matrix it uses before the
  // scatter reads it, so nothing needs clearing between calls
  return launch_indices(token_expert_order, expert_start_indices, restore_token_order,
                        expert_ids, expert_usage_stats, nullptr, 0, topk_ids, N, E, counts, plan,
                        false, nullptr, static_cast<hipStream_t>(stream));
}
