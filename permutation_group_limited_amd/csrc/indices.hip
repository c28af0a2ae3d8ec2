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

// ---- ranked form: the router has ranked every slot ------------------------
// moe_route_and_index's router recorded, per router workgroup (a fine row
// of F slots), its count of slots per expert, and for each slot its rank
// among the workgroup's earlier slots of the same expert, packed with the
// expert id into restore_token_order; it also added its counts into its
// chunk's row of the counts matrix. Chunk c (R fine rows) then places slot
// i at
//   start(e) + slots of e in earlier chunks + in earlier rows of this chunk
//            + rank(i)
// with no per-slot ballots and no running positions: one pass over the
// counts matrix, one block scan, then per block of up to 32 fine rows a
// table of bases in LDS and one pass of stores.
//
// Expert work runs on quads of 4 consecutive experts (rows of counts have
// a stride of E rounded up to 4, so a quad's counts are one 16-byte load):
// the 16 lanes of a DPP row share a quad, lane p taking count rows p, p +
// 16, ... and a block's fine rows p and p + 16, and the sums and row scans
// run over the 16 lanes in registers.
constexpr int kRankedWaves = 16;
constexpr int kRankedThreads = kRankedWaves * kWave;
constexpr int kQuadLanes = 16;
constexpr int kRankedFineLoads = kRankedBlockRows / kQuadLanes;               // 2
constexpr int kRankedCountLoads = static_cast<int>(kMaxChunks) / kQuadLanes;  // 4
constexpr int kRankedSlotsPerThread = kRankedBlockRows * 256 / kRankedThreads;  // F <= 256

// Zero n words from p with every thread of the workgroup: 16-byte stores
// where p is 16-byte aligned, word stores for the rest.
__device__ __forceinline__ void clear_words(uint32_t* p, int64_t n, int threads) {
  int64_t head = 0;
  if ((reinterpret_cast<uintptr_t>(p) & 15u) == 0u) {
    const int64_t vecs = n / 4;
    u32x4* v = reinterpret_cast<u32x4*>(p);
    for (int64_t x = threadIdx.x; x < vecs; x += threads) v[x] = u32x4{0u, 0u, 0u, 0u};
    head = vecs * 4;
  }
  for (int64_t x = head + threadIdx.x; x < n; x += threads) p[x] = 0u;
}

// Inclusive prefix over the 16 lanes of each DPP row (row_shr 1, 2, 4, 8).
__device__ __forceinline__ uint32_t row_inclusive(uint32_t x) {
  x += dpp_or_zero<kRowShr1, 0xF>(x);
  x += dpp_or_zero<kRowShr2, 0xF>(x);
  x += dpp_or_zero<kRowShr4, 0xF>(x);
  x += dpp_or_zero<kRowShr8, 0xF>(x);
  return x;
}
// Value of x in the last lane of the caller's row.
__device__ __forceinline__ uint32_t row_last(uint32_t x) {
  return static_cast<uint32_t>(__shfl(static_cast<int>(x), (lane_id() & ~15) + 15, kWave));
}

__global__ __launch_bounds__(kRankedThreads) void index_ranked_kernel(
    uint32_t* __restrict__ order, uint32_t* __restrict__ starts, uint32_t* __restrict__ restore,
    int32_t* __restrict__ expert_ids, uint32_t* __restrict__ stats,
    uint32_t* __restrict__ scales_offset, uint32_t scale_align,
    const uint32_t* __restrict__ fine, uint32_t* counts, uint32_t* ticket, int64_t N, int32_t E,
    uint32_t F, uint32_t rows, uint32_t R, int64_t nchunks) {
  // rows of the table padded by 4 words: the 16 lanes of a quad write 16
  // rows, which would otherwise all fall on the same LDS banks
  __shared__ __align__(16) uint32_t table[kRankedBlockRows * (kRankedMaxExperts + 4)];
  __shared__ uint32_t tmp[4 * kRankedWaves];
  const int lane = lane_id();
  const int64_t c = blockIdx.x;
  const uint32_t row0 = static_cast<uint32_t>(c) * R;
  const uint32_t nrow = (rows - row0 < R) ? rows - row0 : R;
  const int64_t c0 = static_cast<int64_t>(row0) * F;
  const int64_t c1 =
      (c0 + static_cast<int64_t>(nrow) * F < N) ? c0 + static_cast<int64_t>(nrow) * F : N;
  const int32_t stride = ranked_stride(E);
  const int32_t tstride = stride + 4;  // row stride of the LDS table
  const int q = static_cast<int>(threadIdx.x) / kQuadLanes;  // quad: experts 4q .. 4q + 3
  const int part = static_cast<int>(threadIdx.x) % kQuadLanes;
  const bool own = 4 * q < E;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // 1. this lane's count rows of its quad, then per expert of the quad the
  // slots of all chunks and of the chunks before this one
  u32x4 cv[kRankedCountLoads];
#pragma unroll
  for (int j = 0; j < kRankedCountLoads; ++j) {
    const int64_t cc = part + j * kQuadLanes;
    cv[j] = (own && cc < nchunks) ? *reinterpret_cast<const u32x4*>(counts + cc * stride + 4 * q)
                                  : zero4;
  }
  uint32_t total[4], start[4], done[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t a = 0, b = 0;
#pragma unroll
    for (int j = 0; j < kRankedCountLoads; ++j) {
      a += cv[j][k];
      b += (part + j * kQuadLanes < c) ? cv[j][k] : 0u;
    }
    total[k] = row_last(row_inclusive(a));
    done[k] = row_last(row_inclusive(b));  // slots of expert 4q + k before this chunk
  }

  // 2. block scan over the quads (lane 0 of each quad contributes its
  // quad's sums): expert starts, active experts, padded rows, largest count
  const bool owner = own && part == 0;
  const bool want_pad = scales_offset != nullptr && c == 0;
  uint32_t qsum = 0, qact = 0, qpad = 0, qmax = 0, pad[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    pad[k] = want_pad ? (total[k] + scale_align - 1u) / scale_align * scale_align : 0u;
    qsum += total[k];
    qact += total[k] != 0u ? 1u : 0u;
    qpad += pad[k];
    qmax = qmax > total[k] ? qmax : total[k];
  }
  const uint32_t mine[3] = {owner ? qsum : 0u, owner ? qact : 0u, owner ? qpad : 0u};
  uint32_t excl[3], all[3], most;
  block_scan3<kRankedWaves>(mine, owner ? qmax : 0u, tmp, excl, all, &most);
  // past the scan's barrier every thread has consumed its loads of the
  // counts matrix: take the ticket now, look at it after the scatter
  uint32_t my_ticket = 0u;
  if (threadIdx.x == 0)
    my_ticket = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t grand_total = all[0];
  // counts that do not add up to N: the counts matrix was not zero on entry
  if (c == 0 && threadIdx.x == 0 && grand_total != static_cast<uint32_t>(N))
    __hip_atomic_store(ticket + 1, static_cast<uint32_t>(MOE_STATUS_COUNTS_MISMATCH),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  {
    uint32_t run =
        static_cast<uint32_t>(__shfl(static_cast<int>(excl[0]), lane & ~(kQuadLanes - 1), kWave));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      start[k] = run;
      run += total[k];
    }
  }

  // 3. chunk 0: compacted active experts, CSR starts, stats, aligned offsets
  if (c == 0) {
    if (owner) {
      uint32_t slot = excl[1], padded = excl[2];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (4 * q + k < E && total[k] != 0u && slot < static_cast<uint32_t>(E)) {
          expert_ids[slot] = 4 * q + k;
          starts[slot] = start[k];
          if (want_pad) scales_offset[slot] = padded;
          ++slot;
        }
        padded += pad[k];
      }
    }
    const uint32_t n_active = all[1];
    for (int x = static_cast<int>(n_active) + static_cast<int>(threadIdx.x); x <= E;
         x += kRankedThreads) {
      starts[x] = grand_total;
      if (x < E) expert_ids[x] = -1;
      if (want_pad) scales_offset[x] = all[2];
    }
    if (threadIdx.x == 0) {
      stats[0] = most;
      stats[1] = n_active;
    }
  }

  // 4. blocks of up to kRankedBlockRows fine rows: bases of the block's
  // rows into LDS (one 16-byte store per row), then every slot of the
  // block to its place. (Requesting the next block's loads before placing
  // this block's slots measured slower: 7.7 -> 8.6 us at T = 8192, E = 256.)
  for (uint32_t b0 = 0; b0 < nrow; b0 += kRankedBlockRows) {
    const uint32_t brows = (nrow - b0 < kRankedBlockRows) ? nrow - b0 : kRankedBlockRows;
    const int64_t s0 = c0 + static_cast<int64_t>(b0) * F;
    const int64_t s1 = (s0 + static_cast<int64_t>(brows) * F < c1)
                           ? s0 + static_cast<int64_t>(brows) * F
                           : c1;
    uint32_t pk[kRankedSlotsPerThread];
#pragma unroll
    for (int j = 0; j < kRankedSlotsPerThread; ++j) {
      const int64_t i = s0 + threadIdx.x + static_cast<int64_t>(j) * kRankedThreads;
      pk[j] = i < s1 ? restore[i] : 0u;
    }
    u32x4 fv[kRankedFineLoads];
#pragma unroll
    for (int j = 0; j < kRankedFineLoads; ++j) {
      const uint32_t r = static_cast<uint32_t>(part + j * kQuadLanes);
      fv[j] = (own && r < brows) ? *reinterpret_cast<const u32x4*>(
                                       fine + static_cast<int64_t>(row0 + b0 + r) * stride + 4 * q)
                                 : zero4;
    }
    uint32_t base[kRankedFineLoads][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int j = 0; j < kRankedFineLoads; ++j) {
        const uint32_t v = fv[j][k];
        const uint32_t incl = row_inclusive(v);
        base[j][k] = start[k] + done[k] + incl - v;
        done[k] += row_last(incl);
      }
    }
#pragma unroll
    for (int j = 0; j < kRankedFineLoads; ++j) {
      const uint32_t r = static_cast<uint32_t>(part + j * kQuadLanes);
      if (own && r < brows) {
        u32x4 v;
        v.x = base[j][0];
        v.y = base[j][1];
        v.z = base[j][2];
        v.w = base[j][3];
        *reinterpret_cast<u32x4*>(table + r * tstride + 4 * q) = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRankedSlotsPerThread; ++j) {
      const int64_t i = s0 + threadIdx.x + static_cast<int64_t>(j) * kRankedThreads;
      if (i >= s1) break;
      const uint32_t ex = pk[j] & ((1u << kPackedExpertBits) - 1u);
      const uint32_t rank = pk[j] >> kPackedExpertBits;
      const uint32_t r = static_cast<uint32_t>(i - s0) / F;
      if (ex < static_cast<uint32_t>(E) && r < brows) {  // always, for the router's slots
        const uint32_t pos = table[r * tstride + ex] + rank;
        if (static_cast<int64_t>(pos) < N) order[pos] = static_cast<uint32_t>(i);
        restore[i] = pos;
      } else {
        restore[i] = 0xFFFFFFFFu;
      }
    }
    __syncthreads();  // the table is rewritten by the next block
  }

  // 5. the workgroup that drew the last ticket clears the counts matrix and
  // the ticket for the next call (a read-before-write order only, as in
  // the chunked form)
  __shared__ uint32_t is_last;
  if (threadIdx.x == 0) is_last = my_ticket == static_cast<uint32_t>(nchunks - 1) ? 1u : 0u;
  __syncthreads();
  if (is_last == 0u) return;  // uniform
  clear_words(counts, nchunks * stride, kRankedThreads);
  if (threadIdx.x == 0)
    __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

moe_status_t launch_indices_ranked(uint32_t* order, uint32_t* starts, uint32_t* restore,
                                   int32_t* expert_ids, uint32_t* stats, uint32_t* scales,
                                   uint32_t align, int64_t N, int32_t E, const uint32_t* fine,
                                   uint32_t* counts, uint32_t* ticket, const RankedPlan& plan,
                                   hipStream_t stream) {
  if (!plan.ok || E > kRankedMaxExperts || plan.R > kRankedMaxRowsPerChunk || plan.F > 256 ||
      plan.nchunks < 2 || plan.nchunks > kMaxChunks || counts == nullptr || ticket == nullptr)
    return MOE_ERR_UNSUPPORTED;
  // 16-byte loads of the fine rows and the counts matrix
  if ((reinterpret_cast<uintptr_t>(fine) & 15u) != 0u ||
      (reinterpret_cast<uintptr_t>(counts) & 15u) != 0u)
    return MOE_ERR_ALIGNMENT;
  hipLaunchKernelGGL(index_ranked_kernel, dim3(static_cast<uint32_t>(plan.nchunks)),
                     dim3(kRankedThreads), 0, stream, order, starts, restore, expert_ids, stats,
                     scales, align, fine, counts, ticket, N, E, plan.F, plan.rows, plan.R,
                     plan.nchunks);
  return check_launch();
}

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
