// Fused unpermute gather + weighted top-k sum for gfx950.
//
// Computes what the moe_finalize page (Modular MAX Mojo API, nn/moe)
// describes: each output row gathers its token's K rows of `down` through
// restore_order, scales each by its router weight and accumulates in fp32;
// the [T, K, H] unpermuted tensor is never formed.
//
// HBM-bound streaming gather. Mapping: one wave64 per (token, 64 x 16-byte
// column chunk of the row). The wave's token is uniform, so its K restore
// entries and K weights come in through scalar loads; each lane then issues
// K independent 16-byte non-temporal loads (one per gathered row, all in
// flight together; every row segment is read exactly once), folds them with
// one fmaf per element in ascending k, and writes its output slice with one
// ordinary store (measured a little faster than a non-temporal store here). Rows are addressed in 64 bits
// (T*K*H elements exceed 2^32 for large prefill batches).
#include "common.hpp"

namespace moe {
namespace {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ void widen(const u32x4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ float scalar(const float* p, int64_t i) { return p[i]; }
};
template <>
struct Elem<uint16_t> {  // bf16 bit patterns
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ void widen(const u32x4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ static __forceinline__ float scalar(const uint16_t* p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
  }
};

// Store VEC fp32 accumulators as OutT at p (VEC * sizeof(OutT) bytes).
template <typename OutT, int VEC>
__device__ __forceinline__ void store_out(OutT* p, const float* acc);

template <>
__device__ __forceinline__ void store_out<uint16_t, 8>(uint16_t* p, const float* acc) {
  u32x4 v;
  v.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
  v.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
  v.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
  v.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
  *reinterpret_cast<u32x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store_out<uint16_t, 4>(uint16_t* p, const float* acc) {
  u32x2 v;
  v.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
  v.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
  *reinterpret_cast<u32x2*>(p) = v;
}
template <>
__device__ __forceinline__ void store_out<float, 4>(float* p, const float* acc) {
  u32x4 v;
  v.x = __float_as_uint(acc[0]);
  v.y = __float_as_uint(acc[1]);
  v.z = __float_as_uint(acc[2]);
  v.w = __float_as_uint(acc[3]);
  *reinterpret_cast<u32x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store_out<float, 8>(float* p, const float* acc) {
  store_out<float, 4>(p, acc);
  store_out<float, 4>(p + 4, acc + 4);
}

// KB: rows gathered per batch of loads. EXACT: K == KB, so the whole
// reduction is one batch with no bounds tests (K <= 8); otherwise batches of
// KB rows with a ragged last batch.
template <typename DownT, typename WT, typename OutT, int KB, bool EXACT>
__global__ __launch_bounds__(kBlock) void finalize_kernel(
    OutT* __restrict__ out, const DownT* __restrict__ down, const uint32_t* __restrict__ restore,
    const WT* __restrict__ weight, int64_t T, int32_t K, int64_t H, int32_t chunks_per_row,
    uint32_t n_rows) {
  constexpr int VEC = 16 / Elem<DownT>::kBytes;  // elements per 16-byte load
  const int lane = lane_id();
  // the host keeps T * chunks_per_row below 2^32, so 32-bit scalar math
  const uint32_t gw = blockIdx.x * kWavesPerBlock +
                      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(threadIdx.x) / kWave);
  const uint32_t cpr = static_cast<uint32_t>(chunks_per_row);
  const int64_t t = gw / cpr;
  const int64_t chunk = gw - static_cast<uint32_t>(t) * cpr;
  const int64_t h = (chunk * kWave + lane) * VEC;
  if (t >= T || h >= H) return;  // no cross-lane work below
  const uint32_t* rr = restore + t * K;
  const WT* ww = weight + t * K;

  float acc[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) acc[j] = 0.0f;

  const int32_t k_end = EXACT ? KB : K;
  for (int32_t kb = 0; kb < k_end; kb += KB) {
    const int nb = EXACT ? KB : ((k_end - kb) < KB ? (k_end - kb) : KB);
    u32x4 v[KB];
    float wk[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      uint32_t r = 0;
      float wj = 0.0f;
      if (EXACT || j < nb) {
        r = rr[kb + j];
        wj = Elem<WT>::scalar(ww, kb + j);
      }
      if (r >= n_rows) {  // precondition violated: contribute nothing, stay in bounds
        r = 0;
        wj = 0.0f;
      }
      wk[j] = wj;
      v[j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(down + static_cast<int64_t>(r) * H + h));
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      if (!EXACT && j >= nb) break;
      float d[VEC];
      Elem<DownT>::widen(v[j], d);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = fmaf(wk[j], d[e], acc[e]);
    }
  }
  store_out<OutT, VEC>(out + t * H + h, acc);
}

template <typename DownT, typename WT, typename OutT>
moe_status_t launch_typed(void* out, const void* down, const uint32_t* restore,
                          const void* weight, int64_t T, int32_t K, int64_t H,
                          hipStream_t stream) {
  constexpr int VEC = 16 / Elem<DownT>::kBytes;
  const int64_t cpr = (H + static_cast<int64_t>(kWave) * VEC - 1) / (static_cast<int64_t>(kWave) * VEC);
  const int64_t waves = T * cpr;
  const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  if (waves > 0xFFFFFFFFll - kWavesPerBlock) return MOE_ERR_UNSUPPORTED;
  const uint32_t n_rows = static_cast<uint32_t>(T * K);
  OutT* o = static_cast<OutT*>(out);
  const DownT* d = static_cast<const DownT*>(down);
  const WT* w = static_cast<const WT*>(weight);
  const dim3 grid(static_cast<uint32_t>(blocks)), block(kBlock);
  const int32_t c = static_cast<int32_t>(cpr);
#define MOE_FIN(KB, EXACT)                                                                 \
  hipLaunchKernelGGL((finalize_kernel<DownT, WT, OutT, KB, EXACT>), grid, block, 0, stream, o, \
                     d, restore, w, T, K, H, c, n_rows)
  switch (K) {
    case 1: MOE_FIN(1, true); break;
    case 2: MOE_FIN(2, true); break;
    case 3: MOE_FIN(3, true); break;
    case 4: MOE_FIN(4, true); break;
    case 5: MOE_FIN(5, true); break;
    case 6: MOE_FIN(6, true); break;
    case 7: MOE_FIN(7, true); break;
    case 8: MOE_FIN(8, true); break;
    default: MOE_FIN(8, false); break;
  }
#undef MOE_FIN
  return check_launch();
}

template <typename DownT, typename WT>
moe_status_t dispatch_out(void* out, moe_dtype_t out_dtype, const void* down,
                          const uint32_t* restore, const void* weight, int64_t T, int32_t K,
                          int64_t H, hipStream_t stream) {
  if (out_dtype == MOE_DTYPE_BF16)
    return launch_typed<DownT, WT, uint16_t>(out, down, restore, weight, T, K, H, stream);
  return launch_typed<DownT, WT, float>(out, down, restore, weight, T, K, H, stream);
}

template <typename DownT>
moe_status_t dispatch_weight(void* out, moe_dtype_t out_dtype, const void* down,
                             const uint32_t* restore, const void* weight,
                             moe_dtype_t weight_dtype, int64_t T, int32_t K, int64_t H,
                             hipStream_t stream) {
  if (weight_dtype == MOE_DTYPE_BF16)
    return dispatch_out<DownT, uint16_t>(out, out_dtype, down, restore, weight, T, K, H, stream);
  return dispatch_out<DownT, float>(out, out_dtype, down, restore, weight, T, K, H, stream);
}

}  // namespace

moe_status_t launch_finalize(void* output, moe_dtype_t out_dtype, const void* down,
                             moe_dtype_t down_dtype, const uint32_t* restore_order,
                             const void* router_weight, moe_dtype_t weight_dtype, int64_t T,
                             int32_t K, int64_t H, hipStream_t stream) {
  if (down_dtype == MOE_DTYPE_BF16)
    return dispatch_weight<uint16_t>(output, out_dtype, down, restore_order, router_weight,
                                     weight_dtype, T, K, H, stream);
  return dispatch_weight<float>(output, out_dtype, down, restore_order, router_weight,
                                weight_dtype, T, K, H, stream);
}

}  // namespace moe
