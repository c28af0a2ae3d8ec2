// Device helpers shared by the gfx950 kernels of the routing path.
//
// Everything here is CDNA wave64 code: 64-lane wavefronts, 64-bit ballots,
// cross-lane traffic through ds_bpermute / DPP (via the HIP shuffle
// intrinsics), bf16 / fp16 conversion by the gfx950 hardware converters
// (round to nearest even).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_route.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kBlock = 256;  // workgroup of the router and finalize kernels (4 waves)
constexpr int kWavesPerBlock = kBlock / kWave;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// DPP controls (gfx9 encoding) used by the cross-lane steps: shift right by
// n lanes inside each row of 16, and broadcast of lane 15 of a row into the
// next row / of lane 31 into rows 2 and 3.
constexpr int kRowShr1 = 0x111;
constexpr int kRowShr2 = 0x112;
constexpr int kRowShr4 = 0x114;
constexpr int kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;

// ---- element types -------------------------------------------------------
// Storage tags for the three dtypes of the ABI. Widening to fp32 is exact;
// narrowing rounds to nearest even (gfx950 v_cvt_pk_bf16_f32 and
// v_cvt_f16_f32).
struct DF32 {
  using storage = float;
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ float widen_bits(uint32_t b) { return __uint_as_float(b); }
  __device__ static __forceinline__ uint32_t narrow_bits(float f) { return __float_as_uint(f); }
};
struct DBF16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ float widen_bits(uint32_t b) { return __uint_as_float(b << 16); }
  // element held in the high half of a 32-bit word
  __device__ static __forceinline__ float widen_hi(uint32_t w) {
    return __uint_as_float(w & 0xFFFF0000u);
  }
  __device__ static __forceinline__ uint32_t narrow_bits(float f) {
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)));
  }
};
struct DF16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ float widen_bits(uint32_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
  }
  __device__ static __forceinline__ float widen_hi(uint32_t w) { return widen_bits(w >> 16); }
  // f must stay a rounded binary32 value: left alone, the compiler folds a
  // binary32 fma feeding this conversion into one mixed-precision fma
  // (v_fma_mix) that rounds the exact result to binary16 once, which at a
  // binary16 tie of the binary32 result differs from rounding twice. The
  // empty asm makes f opaque and costs no instruction.
  __device__ static __forceinline__ uint32_t narrow_bits(float f) {
    asm("" : "+v"(f));
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(f)));
  }
};

// Element i of p widened to fp32, and an fp32 value rounded to D's storage
// (bit patterns for the 16-bit types, the value itself for fp32).
template <typename D>
__device__ __forceinline__ float load_f32(const typename D::storage* p, int64_t i) {
  if constexpr (D::kBytes == 4) {
    return p[i];
  } else {
    return D::widen_bits(static_cast<uint32_t>(p[i]));
  }
}
template <typename D>
__device__ __forceinline__ typename D::storage to_storage(float f) {
  if constexpr (D::kBytes == 4) {
    return f;
  } else {
    return static_cast<typename D::storage>(D::narrow_bits(f));
  }
}

// Monotone map binary32 -> uint32 for finite inputs: a < b  <=>  key(a) <
// key(b), and -0 / +0 map to the same key (IEEE equality): adding +0 turns
// -0 into +0 and leaves every other value as it is (round to nearest).
__device__ __forceinline__ uint32_t ordered_key(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  const uint32_t flip = static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u;
  return u ^ flip;  // negative: all bits flipped; positive: sign bit set
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  lo = static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), mask, kWave));
  hi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), mask, kWave));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

// A grid holds at most 2^32 - 1 work-items per dimension. A 1-D problem
// needing more (e.g. the router at 2^26 tokens of 64 lanes each) is laid
// out as rows of kGridRow workgroups along y; kernels take the linear
// workgroup index below and skip the padding workgroups of the last row.
constexpr uint32_t kGridRow = 1u << 16;

inline dim3 grid_1d(int64_t blocks, int threads_per_block) {
  if (blocks * threads_per_block <= static_cast<int64_t>(UINT32_MAX))
    return dim3(static_cast<uint32_t>(blocks));
  return dim3(kGridRow, static_cast<uint32_t>((blocks + kGridRow - 1) / kGridRow));
}

// Linear workgroup index (fewer than 2^32 workgroups per launch).
__device__ __forceinline__ uint32_t linear_block() {
  return blockIdx.x + blockIdx.y * gridDim.x;
}

// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ uint32_t popc_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// Lanes of the wave whose `key` equals the caller's, restricted to `active`
// (a 64-bit ballot per key bit; `nbits` covers every key in use).
__device__ __forceinline__ uint64_t match_any(uint32_t key, int nbits, uint64_t active) {
  uint64_t peers = active;
  for (int bit = 0; bit < nbits; ++bit) {
    const bool set = (key >> bit) & 1u;
    const uint64_t bal = __ballot(set);
    peers &= set ? bal : ~bal;
  }
  return peers;
}

// ---- launchers (host side), one per stage --------------------------------

// Index creation never splits a problem into more chunks than this; its
// waves load their ids kBatch rounds of 64 slots at a time.
constexpr int64_t kMaxChunks = 64;
constexpr int kBatch = 8;


// What the router records for the index step (moe_route_and_index).
// Chunked form (fine == NULL): counts is index creation's counts matrix
// [nchunks, E] (uint32, zero on entry), chunk its slots per chunk;
// counts == NULL and fine == NULL: no histogram.
// Ranked form (fine != NULL): router workgroup b writes row b of `fine`
// [router workgroups, ranked_stride(E)] (its slots per expert), stores for
// each of its slots (rank << 10) | expert in `packed` (rank = earlier slots
// of the workgroup with the same expert), and, when counts != NULL, adds
// its counts into row b / rows_per_chunk of counts [chunks,
// ranked_stride(E)] (zero on entry).
struct RouterHist {
  uint32_t* counts;
  uint32_t chunk;
  uint32_t* fine;
  uint32_t* packed;
  uint32_t rows_per_chunk;
};
constexpr uint32_t kPackedExpertBits = 10;

// Tokens per router workgroup for a batch of T tokens (`counting`: the
// router also records the index step's counts), and whether that launch
// takes two tokens per wave. Shared by the router launcher and the index
// planner so that both see the same workgroups.
bool router_two_tokens_per_wave(int64_t T, int32_t E, int32_t K, int32_t G, bool counting);
int32_t router_block_tokens(int64_t T, int32_t E, int32_t K, int32_t G, bool counting);

// Ranked form of moe_route_and_index: fine rows of F slots (one per router
// workgroup), R rows per index chunk, nchunks chunks (counts matrix only
// when nchunks > 1). ok == false: the batch takes the chunked form.
struct RankedPlan {
  bool ok;
  uint32_t F;
  uint32_t rows;
  uint32_t R;
  int64_t nchunks;
};
constexpr uint32_t kRankedMaxRowsPerChunk = 512;
constexpr uint32_t kRankedBlockRows = 32;  // rows of the table of bases held in LDS at a time
// Rows of counts in the ranked form have a stride of E rounded up to a
// multiple of 4 (padding entries zero), so that they move in 16-byte pieces.
__host__ __device__ constexpr int32_t ranked_stride(int32_t E) { return (E + 3) & ~3; }
constexpr int32_t kRankedMaxExperts = 256;
RankedPlan plan_ranked(int64_t T, int32_t K, int32_t E, int32_t G);
// Rows of fine counts a moe_route_and_index workspace holds room for.
int64_t ranked_fine_rows_bound(int64_t T);

// score_fn: 0 = scores given, 1 = sigmoid of logits, 2 = softmax of logits
moe_status_t launch_router(int32_t* expert_indices, void* expert_weights, const void* scores,
                           const void* bias, moe_dtype_t scores_dtype, moe_dtype_t bias_dtype,
                           int32_t score_fn, int64_t T, int32_t E, int32_t K, int32_t n_groups,
                           int32_t topk_group, int32_t norm_weights, float scale, int32_t mode,
                           RouterHist hist, hipStream_t stream);


struct IndexPlan {
  int waves;        // waves per workgroup (16 when E <= 256 and N > 512, else 4)
  int64_t chunk;    // slots per workgroup
  int64_t nchunks;  // workgroups of the scatter (and histogram) launch
  int rounds;       // 64-slot rounds per wave
  size_t workspace_bytes;
};
// router_counts: the plan of moe_route_and_index's two-launch form, where
// the router fills the counts matrix.
IndexPlan plan_indices(int64_t N, int32_t E, bool router_counts = false);

// scales_offset may be NULL (then scale_align is ignored). With
// counts_ready the counts matrix in `workspace` was already filled (by the
// router) and the histogram launch is skipped; the scatter then counts its
// workgroups on `ticket` and the last one clears the matrix and the ticket
// for the next call.
moe_status_t launch_indices(uint32_t* token_expert_order, uint32_t* expert_start_indices,
                            uint32_t* restore_token_order, int32_t* expert_ids,
                            uint32_t* expert_usage_stats, uint32_t* scales_offset,
                            uint32_t scale_align, const int32_t* topk_ids, int64_t N, int32_t E,
                            void* workspace, const IndexPlan& plan, bool counts_ready,
                            uint32_t* ticket, hipStream_t stream);

// Index step of the ranked form: from the router's fine rows (and counts
// matrix when plan.nchunks > 1) and packed slots, every index output.
moe_status_t launch_indices_ranked(uint32_t* token_expert_order, uint32_t* expert_start_indices,
                                   uint32_t* restore_token_order, int32_t* expert_ids,
                                   uint32_t* expert_usage_stats, uint32_t* scales_offset,
                                   uint32_t scale_align, int64_t N, int32_t E,
                                   const uint32_t* fine, uint32_t* counts, uint32_t* ticket,
                                   const RankedPlan& plan, hipStream_t stream);

// Router and index creation in one launch, for batches that one workgroup
// routes alone (T <= route_index_max_tokens(E)).
int64_t route_index_max_tokens(int32_t E);
moe_status_t launch_route_index(int32_t* idx, void* w, const void* s, const void* b,
                                moe_dtype_t sd, moe_dtype_t bd, int32_t fn, int64_t T, int32_t E,
                                int32_t K, int32_t G, int32_t TG, int32_t norm, float scale,
                                int32_t mode, uint32_t* token_expert_order,
                                uint32_t* expert_start_indices, uint32_t* restore_token_order,
                                int32_t* expert_ids, uint32_t* expert_usage_stats,
                                uint32_t* scales_offset, uint32_t scale_align, hipStream_t stream);

moe_status_t launch_finalize(void* output, moe_dtype_t out_dtype, const void* down,
                             moe_dtype_t down_dtype, const uint32_t* restore_order,
                             const void* router_weight, moe_dtype_t weight_dtype, int64_t T,
                             int32_t K, int64_t H, hipStream_t stream);

// Records the HIP error of a failed launch for moe_last_hip_error().
moe_status_t hip_failure(hipError_t err);
moe_status_t check_launch();

}  // namespace moe
