// Index creation (bucket sort of routed slots by expert) for gfx950.
//
// Produces what the moe_create_indices page (Modular MAX Mojo API, nn/moe)
// lists in its Args: token_expert_order, CSR expert_start_indices,
// restore_token_order, the active expert_ids and expert_usage_stats, from
// the flat topk_ids.
//
// The page's kernel runs one block per expert over all slots, caching up to
// expected_count ids in shared memory and placing segments under an atomic
// lock. That reads the ids E times and fixes the segment order by arrival.
// Here instead (deterministic; the ids are read twice, the second time
// mostly from L2):
//   1. histogram: one workgroup per chunk of C slots counts its experts in
//      LDS (wave-aggregated: one LDS add per distinct expert per 64 slots)
//      and stores the row counts[chunk][0..E) with plain stores;
//   2. scatter: one workgroup per chunk re-derives the expert offsets from
//      the counts matrix (column sums and a block-wide exclusive scan, so no
//      separate scan launch), splits its chunk across its waves, and places
//      every slot at  start(expert) + slots of that expert in earlier chunks
//      + in earlier waves + in earlier lanes of this 64-slot round, the last
//      term from a ballot-built peer mask and mbcnt. Workgroup 0 also writes
//      expert_ids, expert_start_indices and the stats (and, when asked, the
//      aligned scale offsets).
// A problem that fits one chunk skips step 1 (one launch in total). When
// moe_route_and_index runs the path, the router fills the counts matrix
// itself (relaxed atomic adds) and step 1 is skipped too; the scatter's
// last workgroup then clears the matrix for the next call.
//
// Both kernels are latency-bound (N * 12 bytes in all), so every wave issues
// all of its id loads (up to 8 rounds of 64) before using any, keeps them in
// registers from the histogram phase to the scatter phase, and the column
// sums issue their loads 16 at a time.
#include "index_block.hpp"

namespace moe {
namespace {

// ---- step 1: per-chunk histogram ------------------------------------------
template <int W>
__global__ __launch_bounds__(W * kWave) void index_hist_kernel(uint32_t* __restrict__ counts,
                                                               const int32_t* __restrict__ ids,
                                                               int64_t N, int32_t E,
                                                               int64_t chunk, int rounds) {
  constexpr int kThreads = W * kWave;
  __shared__ uint32_t hist[kMaxExperts];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  for (int e = threadIdx.x; e < E; e += kThreads) hist[e] = 0u;
  __syncthreads();
  const int nb = key_bits(E);
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t c1 = (c0 + chunk < N) ? c0 + chunk : N;
  const int64_t w0 = c0 + static_cast<int64_t>(wave) * rounds * kWave;
  for (int r0 = 0; r0 < rounds; r0 += kBatch) {
    if (w0 + static_cast<int64_t>(r0) * kWave >= c1) break;  // uniform
    int32_t ev[kBatch];
    load_batch(ev, ids, w0, r0, rounds, c1, lane);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (r0 + j >= rounds) break;  // uniform
      const int32_t e = ev[j];
      const bool ok = static_cast<uint32_t>(e) < static_cast<uint32_t>(E);
      const uint64_t active = __ballot(ok);
      const uint64_t peers = match_any(static_cast<uint32_t>(e), nb, active);
      if (ok && (__ffsll(static_cast<unsigned long long>(peers)) - 1) == lane)
        atomicAdd(&hist[e], static_cast<uint32_t>(__popcll(peers)));
    }
  }
  __syncthreads();
  uint32_t* row = counts + static_cast<int64_t>(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += kThreads) row[e] = hist[e];
}

template <int W>
__global__ __launch_bounds__(W * kWave) void index_scatter_kernel(
    uint32_t* __restrict__ order, uint32_t* __restrict__ starts, uint32_t* __restrict__ restore,
    int32_t* __restrict__ expert_ids, uint32_t* __restrict__ stats,
    uint32_t* __restrict__ scales_offset, uint32_t scale_align,
    const int32_t* __restrict__ ids, uint32_t* counts, int64_t N, int32_t E, int64_t chunk,
    int64_t nchunks, int rounds, uint32_t* ticket) {
  scatter_chunk<W>(order, starts, restore, expert_ids, stats, scales_offset, scale_align, ids,
                   counts, N, E, chunk, nchunks, rounds, blockIdx.x, ticket);
}

}  // namespace

namespace {
template <int W>
moe_status_t launch_indices_t(uint32_t* order, uint32_t* starts, uint32_t* restore,
                              int32_t* expert_ids, uint32_t* stats, uint32_t* scales,
                              uint32_t align, const int32_t* ids, int64_t N, int32_t E,
                              uint32_t* counts, const IndexPlan& plan, bool counts_ready,
                              uint32_t* ticket, hipStream_t stream) {
  if (plan.nchunks > 1 && !counts_ready) {
    hipLaunchKernelGGL(index_hist_kernel<W>, dim3(static_cast<uint32_t>(plan.nchunks)),
                       dim3(W * kWave), 0, stream, counts, ids, N, E, plan.chunk, plan.rounds);
    const moe_status_t st = check_launch();
    if (st != MOE_OK) return st;
  }
  hipLaunchKernelGGL(index_scatter_kernel<W>, dim3(static_cast<uint32_t>(plan.nchunks)),
                     dim3(W * kWave), 0, stream, order, starts, restore, expert_ids, stats, scales,
                     align, ids, counts, N, E, plan.chunk, plan.nchunks, plan.rounds,
                     counts_ready && plan.nchunks > 1 ? ticket : nullptr);
  return check_launch();
}
}  // namespace

moe_status_t launch_indices(uint32_t* order, uint32_t* starts, uint32_t* restore,
                            int32_t* expert_ids, uint32_t* stats, uint32_t* scales,
                            uint32_t align, const int32_t* ids, int64_t N, int32_t E,
                            void* workspace, const IndexPlan& plan, bool counts_ready,
                            uint32_t* ticket, hipStream_t stream) {
  uint32_t* counts = static_cast<uint32_t*>(workspace);
  if (plan.waves == 16)
    return launch_indices_t<16>(order, starts, restore, expert_ids, stats, scales, align, ids, N,
                                E, counts, plan, counts_ready, ticket, stream);
  return launch_indices_t<4>(order, starts, restore, expert_ids, stats, scales, align, ids, N, E,
                             counts, plan, counts_ready, ticket, stream);
}

}  // namespace moe
