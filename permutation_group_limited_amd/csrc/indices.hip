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
// A problem that fits one chunk skips step 1 (one launch in total).
//
// Both kernels are latency-bound (N * 12 bytes in all), so every wave issues
// all of its id loads (up to 8 rounds of 64) before using any, keeps them in
// registers from the histogram phase to the scatter phase, and the column
// sums issue their loads 16 at a time.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kMaxExperts = 1024;
constexpr int kBatch = 8;  // 64-slot rounds loaded together per wave

__device__ __forceinline__ int key_bits(int E) {
  int nb = 0;
  while ((1 << nb) < E) ++nb;
  return nb;
}

// Exclusive scan of v over the W waves of the block, in thread order.
// Returns the prefix; *total receives the block-wide sum. `tmp` is W words
// of LDS. Must be reached by every thread.
template <int W>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* tmp,
                                                         uint32_t* total) {
  const int lane = lane_id();
  const int wave = static_cast<int>(threadIdx.x) / kWave;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_up(static_cast<int>(x), off, kWave));
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) tmp[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const uint32_t tw = tmp[w];
    before += (w < wave) ? tw : 0u;
    all += tw;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// Maximum of v over the W waves of the block. Must be reached by every
// thread.
template <int W>
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* tmp) {
  const int lane = lane_id();
  const int wave = static_cast<int>(threadIdx.x) / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, kWave));
    v = v > y ? v : y;
  }
  if (lane == 0) tmp[wave] = v;
  __syncthreads();
  uint32_t m = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) m = m > tmp[w] ? m : tmp[w];
  __syncthreads();
  return m;
}

// Loads rounds [r0, r0 + kBatch) of this wave's sub-range: lane value, or -1
// past the chunk end. All loads are issued before any is used.
__device__ __forceinline__ void load_batch(int32_t (&ev)[kBatch], const int32_t* __restrict__ ids,
                                           int64_t w0, int r0, int rounds, int64_t c1, int lane) {
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int64_t i = w0 + static_cast<int64_t>(r0 + j) * kWave + lane;
    ev[j] = (r0 + j < rounds && i < c1) ? ids[i] : -1;
  }
}

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

// ---- step 2: offsets + stable scatter --------------------------------------
template <int W>
__global__ __launch_bounds__(W * kWave) void index_scatter_kernel(
    uint32_t* __restrict__ order, uint32_t* __restrict__ starts, uint32_t* __restrict__ restore,
    int32_t* __restrict__ expert_ids, uint32_t* __restrict__ stats,
    uint32_t* __restrict__ scales_offset, uint32_t scale_align,
    const int32_t* __restrict__ ids, const uint32_t* __restrict__ counts, int64_t N, int32_t E,
    int64_t chunk, int64_t nchunks, int rounds) {
  constexpr int kThreads = W * kWave;
  constexpr int kMaxEPT = (kMaxExperts + kThreads - 1) / kThreads;
  // wbase[w * E + e]: first the number of expert-e slots in wave w's
  // sub-range, then the output position of wave w's next expert-e slot. The
  // host picks W so that W * E <= 4096.
  __shared__ uint32_t wbase[4096];
  __shared__ uint32_t red_a[kThreads];
  __shared__ uint32_t red_p[kThreads];
  __shared__ uint32_t tmp[W];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int nb = key_bits(E);
  const int64_t chunk_id = blockIdx.x;
  const int64_t c0 = chunk_id * chunk;
  const int64_t c1 = (c0 + chunk < N) ? c0 + chunk : N;
  const int64_t w0 = c0 + static_cast<int64_t>(wave) * rounds * kWave;
  uint32_t* my_base = wbase + wave * E;

  // Issue the first batch of ids and this thread's share of the counts
  // matrix before anything waits on memory, so the two latencies overlap.
  int32_t first[kBatch];
  load_batch(first, ids, w0, 0, rounds, c1, lane);
  const bool split = nchunks > 1 && E <= kThreads;
  const int parts = E <= kThreads ? kThreads / E : 1;
  const int my_e = static_cast<int>(threadIdx.x) % E;
  const int my_part = static_cast<int>(threadIdx.x) / E;
  constexpr int kCountRegs = 16;
  uint32_t cv[kCountRegs];
  const bool cv_resident = split && nchunks <= static_cast<int64_t>(kCountRegs) * parts;
  if (cv_resident) {
#pragma unroll
    for (int q = 0; q < kCountRegs; ++q) {
      const int64_t c = my_part + static_cast<int64_t>(q) * parts;
      cv[q] = (my_part < parts && c < nchunks) ? counts[c * E + my_e] : 0u;
    }
  }

  for (int x = threadIdx.x; x < W * E; x += kThreads) wbase[x] = 0u;
  __syncthreads();

  // (a) per-wave histogram. One lane per distinct expert per round writes,
  // and a wave's rounds are in program order, so no atomics are needed. The
  // first batch of ids stays in registers for (e).
  for (int r0 = 0; r0 < rounds; r0 += kBatch) {
    int32_t ev[kBatch];
    if (r0 == 0) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j) ev[j] = first[j];
    } else {
      load_batch(ev, ids, w0, r0, rounds, c1, lane);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (r0 + j >= rounds) break;  // uniform
      const int32_t e = ev[j];
      const bool ok = static_cast<uint32_t>(e) < static_cast<uint32_t>(E);
      const uint64_t active = __ballot(ok);
      const uint64_t peers = match_any(static_cast<uint32_t>(e), nb, active);
      if (ok && (__ffsll(static_cast<unsigned long long>(peers)) - 1) == lane)
        my_base[e] += static_cast<uint32_t>(__popcll(peers));
    }
  }
  __syncthreads();

  // (b) per-expert totals over all chunks and this chunk's prefix. Thread
  // tid owns experts [tid*EPT, tid*EPT + EPT), so a block scan over threads
  // followed by a local running sum is an exclusive scan over experts. When
  // E <= threads, the column sums are split over P = threads / E parts
  // (thread part*E + e reads chunks part, part + P, ...), so each thread has
  // at most nchunks / P loads in flight, and are folded through LDS.
  const int EPT = (E + kThreads - 1) / kThreads;
  uint32_t tot[kMaxEPT], pre[kMaxEPT], start[kMaxEPT];
  uint32_t local_sum = 0, local_active = 0, local_max = 0;
  if (split) {
    uint32_t a = 0, p = 0;
    if (cv_resident) {
#pragma unroll
      for (int q = 0; q < kCountRegs; ++q) {
        const int64_t c = my_part + static_cast<int64_t>(q) * parts;
        a += cv[q];
        p += (c < chunk_id) ? cv[q] : 0u;
      }
    } else if (my_part < parts) {
#pragma unroll 16
      for (int64_t c = my_part; c < nchunks; c += parts) {
        const uint32_t v = counts[c * E + my_e];
        a += v;
        p += (c < chunk_id) ? v : 0u;
      }
    }
    red_a[threadIdx.x] = a;
    red_p[threadIdx.x] = p;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxEPT; ++j) {
      tot[j] = 0u;
      pre[j] = 0u;
    }
    if (threadIdx.x < static_cast<unsigned>(E)) {
      for (int q = 0; q < parts; ++q) {
        tot[0] += red_a[q * E + threadIdx.x];
        pre[0] += red_p[q * E + threadIdx.x];
      }
      local_sum = tot[0];
      local_active = tot[0] ? 1u : 0u;
      local_max = tot[0];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kMaxEPT; ++j) {
      const int e = static_cast<int>(threadIdx.x) * EPT + j;
      tot[j] = 0u;
      pre[j] = 0u;
      if (j < EPT && e < E) {
        if (nchunks == 1) {
#pragma unroll
          for (int w = 0; w < W; ++w) tot[j] += wbase[w * E + e];
        } else {
          uint32_t a = 0, p = 0;
#pragma unroll 16
          for (int64_t c = 0; c < nchunks; ++c) {
            const uint32_t v = counts[c * E + e];
            a += v;
            p += (c < chunk_id) ? v : 0u;
          }
          tot[j] = a;
          pre[j] = p;
        }
        local_sum += tot[j];
        local_active += tot[j] ? 1u : 0u;
        local_max = local_max > tot[j] ? local_max : tot[j];
      }
    }
  }
  uint32_t grand_total = 0;
  uint32_t run = block_exclusive_scan<W>(local_sum, tmp, &grand_total);
#pragma unroll
  for (int j = 0; j < kMaxEPT; ++j) {
    start[j] = run;
    run += tot[j];
  }
  // (c) running positions of each wave
#pragma unroll
  for (int j = 0; j < kMaxEPT; ++j) {
    const int e = static_cast<int>(threadIdx.x) * EPT + j;
    if (j < EPT && e < E) {
      uint32_t pos = start[j] + pre[j];
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const uint32_t n = wbase[w * E + e];
        wbase[w * E + e] = pos;
        pos += n;
      }
    }
  }

  // (d) workgroup 0: compacted active experts, CSR starts, stats
  if (chunk_id == 0) {
    uint32_t n_active = 0;
    uint32_t slot = block_exclusive_scan<W>(local_active, tmp, &n_active);
    const uint32_t most = block_max<W>(local_max, tmp);
#pragma unroll
    for (int j = 0; j < kMaxEPT; ++j) {
      const int e = static_cast<int>(threadIdx.x) * EPT + j;
      if (j < EPT && e < E && tot[j] != 0u) {
        expert_ids[slot] = e;
        starts[slot] = start[j];
        ++slot;
      }
    }
    for (int x = static_cast<int>(n_active) + static_cast<int>(threadIdx.x); x <= E;
         x += kThreads) {
      starts[x] = grand_total;
      if (x < E) expert_ids[x] = -1;
    }
    if (threadIdx.x == 0) {
      stats[0] = most;
      stats[1] = n_active;
    }
    if (scales_offset != nullptr) {  // uniform
      // every active expert's rows rounded up to a multiple of scale_align
      uint32_t local_pad = 0;
#pragma unroll
      for (int j = 0; j < kMaxEPT; ++j) {
        const uint32_t c = tot[j];
        local_pad += (c + scale_align - 1u) / scale_align * scale_align;
      }
      uint32_t pad_total = 0;
      uint32_t pad = block_exclusive_scan<W>(local_pad, tmp, &pad_total);
      uint32_t s2 = block_exclusive_scan<W>(local_active, tmp, &n_active);
#pragma unroll
      for (int j = 0; j < kMaxEPT; ++j) {
        const int e = static_cast<int>(threadIdx.x) * EPT + j;
        if (j < EPT && e < E && tot[j] != 0u) {
          scales_offset[s2] = pad;
          ++s2;
        }
        pad += (tot[j] + scale_align - 1u) / scale_align * scale_align;
      }
      for (int x = static_cast<int>(n_active) + static_cast<int>(threadIdx.x); x <= E;
           x += kThreads)
        scales_offset[x] = pad_total;
    }
  }
  __syncthreads();

  // (e) stable scatter, rounds in the same order as (a)
  for (int r0 = 0; r0 < rounds; r0 += kBatch) {
    int32_t ev[kBatch];
    if (r0 == 0) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j) ev[j] = first[j];
    } else {
      load_batch(ev, ids, w0, r0, rounds, c1, lane);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (r0 + j >= rounds) break;  // uniform
      const int64_t i = w0 + static_cast<int64_t>(r0 + j) * kWave + lane;
      const int32_t e = ev[j];
      const bool ok = static_cast<uint32_t>(e) < static_cast<uint32_t>(E);
      const uint64_t active = __ballot(ok);
      const uint64_t peers = match_any(static_cast<uint32_t>(e), nb, active);
      if (ok) {
        const uint32_t pos = my_base[e] + popc_below(peers);
        order[pos] = static_cast<uint32_t>(i);
        restore[i] = pos;
        if ((__ffsll(static_cast<unsigned long long>(peers)) - 1) == lane)
          my_base[e] += static_cast<uint32_t>(__popcll(peers));
      } else if (i < c1) {
        restore[i] = 0xFFFFFFFFu;
      }
    }
  }
}

}  // namespace

IndexPlan plan_indices(int64_t N, int32_t E) {
  IndexPlan p;
  p.waves = E <= 256 ? 16 : 4;  // W * E <= 4096 LDS words
  const int64_t per_round = static_cast<int64_t>(p.waves) * kWave;
  if (N <= kBatch * per_round) {
    // one workgroup does everything in one launch
    p.rounds = static_cast<int>(N > 0 ? (N + per_round - 1) / per_round : 1);
    p.chunk = per_round * p.rounds;
    p.nchunks = 1;
  } else {
    // about 64 workgroups: short column sums, enough parallel latency
    int64_t r = (N + 64 * per_round - 1) / (64 * per_round);
    if (r < 1) r = 1;
    p.rounds = static_cast<int>(r);
    p.chunk = per_round * r;
    p.nchunks = (N + p.chunk - 1) / p.chunk;
  }
  p.workspace_bytes =
      p.nchunks > 1 ? static_cast<size_t>(p.nchunks) * static_cast<size_t>(E) * sizeof(uint32_t)
                    : 0;
  return p;
}

namespace {
template <int W>
moe_status_t launch_indices_t(uint32_t* order, uint32_t* starts, uint32_t* restore,
                              int32_t* expert_ids, uint32_t* stats, uint32_t* scales,
                              uint32_t align, const int32_t* ids, int64_t N, int32_t E,
                              uint32_t* counts, const IndexPlan& plan, hipStream_t stream) {
  if (plan.nchunks > 1) {
    hipLaunchKernelGGL(index_hist_kernel<W>, dim3(static_cast<uint32_t>(plan.nchunks)),
                       dim3(W * kWave), 0, stream, counts, ids, N, E, plan.chunk, plan.rounds);
    const moe_status_t st = check_launch();
    if (st != MOE_OK) return st;
  }
  hipLaunchKernelGGL(index_scatter_kernel<W>, dim3(static_cast<uint32_t>(plan.nchunks)),
                     dim3(W * kWave), 0, stream, order, starts, restore, expert_ids, stats, scales,
                     align, ids, static_cast<const uint32_t*>(counts), N, E, plan.chunk,
                     plan.nchunks, plan.rounds);
  return check_launch();
}
}  // namespace

moe_status_t launch_indices(uint32_t* order, uint32_t* starts, uint32_t* restore,
                            int32_t* expert_ids, uint32_t* stats, uint32_t* scales,
                            uint32_t align, const int32_t* ids, int64_t N, int32_t E,
                            void* workspace, const IndexPlan& plan, hipStream_t stream) {
  uint32_t* counts = static_cast<uint32_t*>(workspace);
  if (plan.waves == 16)
    return launch_indices_t<16>(order, starts, restore, expert_ids, stats, scales, align, ids, N,
                                E, counts, plan, stream);
  return launch_indices_t<4>(order, starts, restore, expert_ids, stats, scales, align, ids, N, E,
                             counts, plan, stream);
}

}  // namespace moe
