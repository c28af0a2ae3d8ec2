// Bandwidth probes (libmoe_probe.so, include/moe_probe.h): streaming reads,
// streaming writes and the finalize gather without its stores, each with the
// exact load / store instructions and per-wave shapes of finalize_kernel, so
// that the benchmark can set the finalize kernel's time beside what the
// memory system delivers to those patterns alone; and the fixed costs of
// small batches: an empty launch, and one workgroup reading a small buffer.
// Not part of the routing path.
#include "common.hpp"
#include "moe_probe.h"

namespace moe {
namespace {

// A data-dependent store that never happens on real data keeps every load
// live without adding traffic.
constexpr uint32_t kMagic = 0x9E3779B9u;
constexpr int kStoreKeep = 16;          // sc1 and nt: finalize's two output policies
constexpr int kStoreStream = 2;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kReadVecsPerLane = 8;     // 8 x 16 B per lane: 8 KiB per wave

__device__ __forceinline__ uint64_t wave_index() {
  return static_cast<uint64_t>(linear_block()) * kWavesPerBlock +
         __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(threadIdx.x) / kWave);
}

__device__ __forceinline__ uint32_t fold(const u32x4& v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(kBlock) void probe_read_kernel(const u32x4* __restrict__ src,
                                                            uint64_t n_waves,
                                                            uint32_t* __restrict__ sink) {
  const uint64_t w = wave_index();
  if (w >= n_waves) return;
  const u32x4* p = src + w * (kReadVecsPerLane * kWave) + lane_id();
  u32x4 v[kReadVecsPerLane];
#pragma unroll
  for (int j = 0; j < kReadVecsPerLane; ++j) v[j] = __builtin_nontemporal_load(p + j * kWave);
  uint32_t x = 0;
#pragma unroll
  for (int j = 0; j < kReadVecsPerLane; ++j) x ^= fold(v[j]);
  if (x == kMagic) sink[0] = x;
}

__global__ __launch_bounds__(kBlock) void probe_write_kernel(uint32_t* __restrict__ dst,
                                                             uint64_t n_waves, uint32_t value,
                                                             int32_t streaming) {
  const uint64_t w = wave_index();
  if (w >= n_waves) return;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(dst + w * (kWave * 4), 0, kWave * 16, kRsrcWord3);
  u32x4 v;
  v.x = v.y = v.z = v.w = value;
  if (streaming)  // uniform
    __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, lane_id() * 16, 0, kStoreStream);
  else
    __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, lane_id() * 16, 0, kStoreKeep);
}

// One wave per (token, 64 x 16-byte chunk of the row); rows addressed in 64
// bits; K rows in batches of at most 8 loads in flight.
__global__ __launch_bounds__(kBlock) void probe_gather_kernel(
    const u32x4* __restrict__ rows, const uint32_t* __restrict__ restore, int64_t T, int32_t K,
    int64_t row_vecs, uint32_t chunks_per_row, uint32_t n_rows, uint32_t* __restrict__ sink) {
  constexpr int KB = 8;
  const uint32_t gw = static_cast<uint32_t>(wave_index());
  const int64_t t = gw / chunks_per_row;
  const int64_t chunk = gw - static_cast<uint32_t>(t) * chunks_per_row;
  const int64_t h = chunk * kWave + lane_id();
  if (t >= T || h >= row_vecs) return;
  const uint32_t* rr = restore + t * K;
  uint32_t x = 0;
  for (int32_t kb = 0; kb < K; kb += KB) {
    const int nb = (K - kb) < KB ? (K - kb) : KB;
    uint32_t r[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) r[j] = j < nb ? rr[kb + j] : 0u;
    u32x4 v[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const uint32_t row = r[j] < n_rows ? r[j] : 0u;
      v[j] = j < nb ? __builtin_nontemporal_load(rows + static_cast<int64_t>(row) * row_vecs + h)
                    : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) x ^= fold(v[j]);
  }
  if (x == kMagic) sink[0] = x;
}

__global__ __launch_bounds__(kBlock) void probe_empty_kernel() {}

// One workgroup of kConsumeThreads threads; thread i reads vectors i,
// i + kConsumeThreads, ... (all loads issued before any is used).
constexpr int kConsumeThreads = 1024;
constexpr int kConsumeMaxVecs = 16;  // per thread: 256 KiB per call at most
__global__ __launch_bounds__(kConsumeThreads) void probe_consume_kernel(
    const u32x4* __restrict__ src, int vecs_per_thread, uint32_t* __restrict__ sink) {
  u32x4 v[kConsumeMaxVecs];
#pragma unroll
  for (int j = 0; j < kConsumeMaxVecs; ++j)
    v[j] = j < vecs_per_thread ? src[threadIdx.x + j * kConsumeThreads] : u32x4{0u, 0u, 0u, 0u};
  uint32_t x = 0;
#pragma unroll
  for (int j = 0; j < kConsumeMaxVecs; ++j) x ^= fold(v[j]);
  if (x == kMagic) sink[0] = x;
}

constexpr size_t kMaxProbeBytes = static_cast<size_t>(1) << 40;

moe_status_t launched() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

moe_status_t moe_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  constexpr size_t kWaveBytes = kReadVecsPerLane * kWave * 16;
  if (bytes % kWaveBytes != 0 || bytes > kMaxProbeBytes) return MOE_ERR_INVALID_ARG;
  if (bytes == 0) return MOE_OK;
  if (src == nullptr || sink == nullptr) return MOE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return MOE_ERR_ALIGNMENT;
  const uint64_t waves = bytes / kWaveBytes;
  const int64_t blocks = static_cast<int64_t>((waves + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(probe_read_kernel, grid_1d(blocks, kBlock), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), waves,
                     sink);
  return launched();
}

moe_status_t moe_probe_write(void* dst, size_t bytes, uint32_t value, int32_t streaming,
                             void* stream) {
  constexpr size_t kWaveBytes = kWave * 16;
  if (bytes % kWaveBytes != 0 || bytes > kMaxProbeBytes) return MOE_ERR_INVALID_ARG;
  if (bytes == 0) return MOE_OK;
  if (dst == nullptr) return MOE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(dst) % 16 != 0) return MOE_ERR_ALIGNMENT;
  const uint64_t waves = bytes / kWaveBytes;
  const int64_t blocks = static_cast<int64_t>((waves + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(probe_write_kernel, grid_1d(blocks, kBlock), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint32_t*>(dst), waves, value,
                     streaming);
  return launched();
}

moe_status_t moe_probe_gather(const void* rows, const uint32_t* restore, int64_t T, int32_t K,
                              int64_t row_bytes, uint32_t* sink, void* stream) {
  if (T < 0 || K < 1 || T > static_cast<int64_t>(UINT32_MAX) / K) return MOE_ERR_INVALID_ARG;
  if (row_bytes <= 0 || row_bytes % 16 != 0 || row_bytes >= (int64_t{1} << 31))
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (rows == nullptr || restore == nullptr || sink == nullptr) return MOE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(rows) % 16 != 0) return MOE_ERR_ALIGNMENT;
  const int64_t row_vecs = row_bytes / 16;
  const int64_t cpr = (row_vecs + kWave - 1) / kWave;
  const int64_t waves = T * cpr;
  if (waves > 0xFFFFFFFFll - static_cast<int64_t>(kGridRow) * kWavesPerBlock)
    return MOE_ERR_UNSUPPORTED;
  const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(probe_gather_kernel, grid_1d(blocks, kBlock), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(rows), restore,
                     T, K, row_vecs, static_cast<uint32_t>(cpr), static_cast<uint32_t>(T * K),
                     sink);
  return launched();
}

moe_status_t moe_probe_empty(int32_t workgroups, void* stream) {
  if (workgroups < 1 || workgroups > 65535) return MOE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(probe_empty_kernel, dim3(static_cast<uint32_t>(workgroups)), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream));
  return launched();
}

moe_status_t moe_probe_consume(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  constexpr size_t kStep = static_cast<size_t>(kConsumeThreads) * 16;
  if (bytes % kStep != 0 || bytes > kStep * kConsumeMaxVecs) return MOE_ERR_INVALID_ARG;
  if (bytes == 0) return MOE_OK;
  if (src == nullptr || sink == nullptr) return MOE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return MOE_ERR_ALIGNMENT;
  hipLaunchKernelGGL(probe_consume_kernel, dim3(1), dim3(kConsumeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     static_cast<int>(bytes / kStep), sink);
  return launched();
}

}  // extern "C"
