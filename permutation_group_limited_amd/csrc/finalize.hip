// Fused unpermute gather + weighted top-k sum for gfx950.
//
// Computes what the moe_finalize page (Modular MAX Mojo API, nn/moe)
// describes: output row t is the sum over k of router weight (t, k) times
// the row of `down` that restore_order names for slot t*K + k, with the sum
// held in fp32; the [T, K, H] unpermuted tensor is never formed.
//
// HBM-bound streaming gather. Mapping: one wave64 per (token, 64 x 16-byte
// column chunk of the row). The wave's token is uniform, so its K restore
// entries (and fp32 weights) come in through scalar loads; each lane then
// issues K independent 16-byte non-temporal loads (one per gathered row,
// all in flight together; every row segment is read exactly once), folds
// them with one fmaf per element in ascending k, and writes its output
// slice with buffer stores (one 16-byte store, two for fp32 output, one
// 8-byte store for fp32 rows into 16-bit output; cache policy below). Rows
// of `down` are addressed in 64 bits (T*K*H elements exceed 2^32 for large
// prefill batches).
//
// Launch shape. Gathers whose rows fit the memory-side cache run four waves
// per workgroup at the occupancy the registers allow. Larger (streaming)
// gathers run one wave per workgroup, and each workgroup reserves a share of
// the compute unit's LDS that it never touches, so that only a few waves
// share a compute unit: about 64 KiB of row loads in flight per compute unit
// (9 waves at K = 8, 17 at K = 4; K = 2 is left uncapped). With every wave
// resident (24 per compute unit at K = 8) the kernel was slower, while the
// same gather without its stores was not: the extra reads in flight cost
// the output stream. Measured at the DeepSeek-V3 shape (T = 8192, K = 8,
// H = 7168, bf16): 183 -> 173 us call after call and 187 -> 176 us after a
// 1 GiB write; at T = 65536, 1517 -> 1400 us.
#include "common.hpp"

namespace moe {
namespace {

// Widen the 16 bytes of one load into 16 / kBytes fp32 values (element j of
// the segment is the j-th in memory order).
template <typename D>
__device__ __forceinline__ void widen16(const u32x4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (D::kBytes == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = D::widen_bits(w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = D::widen_bits(w[i] & 0xFFFFu);
      f[2 * i + 1] = D::widen_hi(w[i]);
    }
  }
}

// Output stores go through a buffer resource spanning the token's output
// row. Their cache policy depends on the problem's size (the loads stay
// non-temporal, which matters far more):
//  * gathered rows that fit the memory-side cache (MI355X: 256 MiB): sc1,
//    which keeps the output there (Mixtral-shaped, 64 MiB of rows: 15.1 us
//    against 16.5-17.8 with non-temporal stores, call after call);
//  * larger: non-temporal, which streams the output out instead of pushing
//    other lines out of the cache it cannot stay in anyway (DSv3-shaped,
//    0.94 GB of rows: 182.7 against 185.5 us call after call, and 187 against
//    195.6 us with the cache full of other data before each call).
constexpr int kStoreKeep = 16;         // cache-policy operand: sc1
constexpr int kStoreStream = 2;        // cache-policy operand: nt
constexpr int64_t kMemorySideCacheBytes = int64_t{256} << 20;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format

// Store VEC fp32 accumulators as D at byte offset `off` of the row (VEC *
// kBytes bytes, one or two vector stores) with cache policy POL.
template <typename D, int VEC, int POL>
__device__ __forceinline__ void store_out(__amdgpu_buffer_rsrc_t row, uint32_t off,
                                          const float* acc) {
  if constexpr (D::kBytes == 4) {
#pragma unroll
    for (int q = 0; q < VEC; q += 4) {
      u32x4 v;
      v.x = D::narrow_bits(acc[q]);
      v.y = D::narrow_bits(acc[q + 1]);
      v.z = D::narrow_bits(acc[q + 2]);
      v.w = D::narrow_bits(acc[q + 3]);
      __builtin_amdgcn_raw_buffer_store_b128(v, row, static_cast<int>(off + q * 4), 0, POL);
    }
  } else if constexpr (VEC == 8) {
    u32x4 v;
    v.x = D::narrow_bits(acc[0]) | (D::narrow_bits(acc[1]) << 16);
    v.y = D::narrow_bits(acc[2]) | (D::narrow_bits(acc[3]) << 16);
    v.z = D::narrow_bits(acc[4]) | (D::narrow_bits(acc[5]) << 16);
    v.w = D::narrow_bits(acc[6]) | (D::narrow_bits(acc[7]) << 16);
    __builtin_amdgcn_raw_buffer_store_b128(v, row, static_cast<int>(off), 0, POL);
  } else {
    u32x2 v;
    v.x = D::narrow_bits(acc[0]) | (D::narrow_bits(acc[1]) << 16);
    v.y = D::narrow_bits(acc[2]) | (D::narrow_bits(acc[3]) << 16);
    __builtin_amdgcn_raw_buffer_store_b64(v, row, static_cast<int>(off), 0, POL);
  }
}

// KB: rows gathered per batch of loads. EXACT: K == KB, so the whole
// reduction is one batch with no bounds tests (K <= 8); otherwise batches of
// KB rows with a ragged last batch. Workgroups hold kBlock threads or one
// wave (the launch decides; the wave index comes from the workgroup size).
template <typename DD, typename DO, int KB, bool EXACT>
__global__ __launch_bounds__(kBlock) void finalize_kernel(
    typename DO::storage* __restrict__ out, const typename DD::storage* __restrict__ down,
    const uint32_t* __restrict__ restore, const void* __restrict__ weight, moe_dtype_t wd,
    int64_t T, int32_t K, int64_t H, int32_t chunks_per_row, uint32_t n_rows, int32_t stream_out) {
  constexpr int VEC = 16 / DD::kBytes;  // elements per 16-byte load
  const int lane = lane_id();
  // the host keeps T * chunks_per_row below 2^32, so 32-bit scalar math;
  // grid padding (t >= T) returns below
  const uint32_t wpb = static_cast<uint32_t>(__builtin_amdgcn_workgroup_size_x()) / kWave;
  const uint32_t gw = linear_block() * wpb +
                      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(threadIdx.x) / kWave);
  const uint32_t cpr = static_cast<uint32_t>(chunks_per_row);
  const int64_t t = gw / cpr;
  const int64_t chunk = gw - static_cast<uint32_t>(t) * cpr;
  const int64_t h = (chunk * kWave + lane) * VEC;
  if (t >= T || h >= H) return;  // no cross-lane work below
  const uint32_t* rr = restore + t * K;

  float acc[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) acc[j] = 0.0f;

  const int32_t k_end = EXACT ? KB : K;
  for (int32_t kb = 0; kb < k_end; kb += KB) {
    const int nb = EXACT ? KB : ((k_end - kb) < KB ? (k_end - kb) : KB);
    // restore entries first (one batched scalar load), then every row load,
    // then the weights, so that all K row loads are in flight together
    uint32_t r[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) r[j] = (EXACT || j < nb) ? rr[kb + j] : 0u;
    u32x4 v[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const uint32_t row = r[j] < n_rows ? r[j] : 0u;  // stay in bounds if violated
      v[j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(down + static_cast<int64_t>(row) * H + h));
    }
    float wk[KB];
    const int64_t w0 = t * K + kb;
    if (wd == MOE_DTYPE_F32) {
      const float* wf = static_cast<const float*>(weight) + w0;
#pragma unroll
      for (int j = 0; j < KB; ++j) wk[j] = (EXACT || j < nb) ? wf[j] : 0.0f;
    } else {
      const uint16_t* wh = static_cast<const uint16_t*>(weight) + w0;
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const uint32_t b = (EXACT || j < nb) ? wh[j] : 0u;
        wk[j] = wd == MOE_DTYPE_BF16 ? DBF16::widen_bits(b) : DF16::widen_bits(b);
      }
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      if (!EXACT && j >= nb) break;
      const float wj = r[j] < n_rows ? wk[j] : 0.0f;  // a violating row contributes nothing
      float d[VEC];
      widen16<DD>(v[j], d);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = fmaf(wj, d[e], acc[e]);
    }
  }
  // the host keeps a row below 2^31 bytes, so offsets fit the resource
  constexpr int64_t kOutBytes = sizeof(typename DO::storage);
  const __amdgpu_buffer_rsrc_t row = __builtin_amdgcn_make_buffer_rsrc(
      out + t * H, 0, static_cast<int>(H * kOutBytes), kRsrcWord3);
  if (stream_out)  // wave-uniform
    store_out<DO, VEC, kStoreStream>(row, static_cast<uint32_t>(h * kOutBytes), acc);
  else
    store_out<DO, VEC, kStoreKeep>(row, static_cast<uint32_t>(h * kOutBytes), acc);
}

// Waves of a streaming gather allowed on one compute unit: about 64 KiB of
// row loads in flight (each wave has min(K, 8) rows of 1 KiB requested at
// once), plus one; 0 = no cap (at least the 32 waves a compute unit holds).
int streaming_wave_cap(int32_t K) {
  const int rows = K < 8 ? K : 8;
  const int cap = 1 + (64 + rows - 1) / rows;
  return cap >= 32 ? 0 : cap;
}

// LDS of one gfx950 compute unit (the only target this library is built
// for).
constexpr int kLdsPerCu = 160 * 1024;

// Dynamic LDS for each one-wave workgroup so that at most `cap` of them fit
// on a compute unit (rounded down to the 512-byte allocation unit); 0 = no
// cap, and no cap either where a workgroup would need more than the 64 KiB
// it may take without a launch attribute (caps below 3; the caps in use are
// 9 and up).
size_t occupancy_lds_bytes(int cap) {
  if (cap <= 0) return 0;
  const int bytes = (kLdsPerCu / cap) / 512 * 512;
  return bytes <= 64 * 1024 ? static_cast<size_t>(bytes) : 0;
}

template <typename DD, typename DO>
moe_status_t launch_typed(void* out, const void* down, const uint32_t* restore,
                          const void* weight, moe_dtype_t wd, int64_t T, int32_t K, int64_t H,
                          hipStream_t stream) {
  constexpr int VEC = 16 / DD::kBytes;
  const int64_t per_wave = static_cast<int64_t>(kWave) * VEC;
  const int64_t cpr = (H + per_wave - 1) / per_wave;
  const int64_t waves = T * cpr;
  // gathered rows above the memory-side cache: T * K rows of H * kBytes bytes
  // (compared by division, so no product can overflow)
  const int32_t stream_out =
      T * K > kMemorySideCacheBytes / (H * static_cast<int64_t>(DD::kBytes)) ? 1 : 0;
  const int wpb = stream_out ? 1 : kWavesPerBlock;
  // wave indices (grid padding included) stay below 2^32; one documented
  // limit for both launch shapes (the four-wave one needs it)
  if (waves > 0xFFFFFFFFll - static_cast<int64_t>(kGridRow) * kWavesPerBlock)
    return MOE_ERR_UNSUPPORTED;
  const int64_t blocks = (waves + wpb - 1) / wpb;
  const size_t lds = stream_out ? occupancy_lds_bytes(streaming_wave_cap(K)) : 0;
  const uint32_t n_rows = static_cast<uint32_t>(T * K);
  auto* o = static_cast<typename DO::storage*>(out);
  const auto* d = static_cast<const typename DD::storage*>(down);
  const dim3 grid = grid_1d(blocks, wpb * kWave), block(wpb * kWave);
  const int32_t c = static_cast<int32_t>(cpr);
#define MOE_FIN(KB, EXACT)                                                                    \
  hipLaunchKernelGGL((finalize_kernel<DD, DO, KB, EXACT>), grid, block, lds, stream, o, d, \
                     restore, weight, wd, T, K, H, c, n_rows, stream_out)
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

template <typename DD>
moe_status_t dispatch_out(void* out, moe_dtype_t out_dtype, const void* down,
                          const uint32_t* restore, const void* weight, moe_dtype_t wd, int64_t T,
                          int32_t K, int64_t H, hipStream_t stream) {
  switch (out_dtype) {
    case MOE_DTYPE_BF16:
      return launch_typed<DD, DBF16>(out, down, restore, weight, wd, T, K, H, stream);
    case MOE_DTYPE_F16:
      return launch_typed<DD, DF16>(out, down, restore, weight, wd, T, K, H, stream);
    default:
      return launch_typed<DD, DF32>(out, down, restore, weight, wd, T, K, H, stream);
  }
}

}  // namespace

moe_status_t launch_finalize(void* output, moe_dtype_t out_dtype, const void* down,
                             moe_dtype_t down_dtype, const uint32_t* restore_order,
                             const void* router_weight, moe_dtype_t weight_dtype, int64_t T,
                             int32_t K, int64_t H, hipStream_t stream) {
  switch (down_dtype) {
    case MOE_DTYPE_BF16:
      return dispatch_out<DBF16>(output, out_dtype, down, restore_order, router_weight,
                                 weight_dtype, T, K, H, stream);
    case MOE_DTYPE_F16:
      return dispatch_out<DF16>(output, out_dtype, down, restore_order, router_weight,
                                weight_dtype, T, K, H, stream);
    default:
      return dispatch_out<DF32>(output, out_dtype, down, restore_order, router_weight,
                                weight_dtype, T, K, H, stream);
  }
}

}  // namespace moe
