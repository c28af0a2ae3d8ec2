// Building blocks of index creation shared by the index kernels and the
// fused router + index kernel: block-wide scan helpers and the per-chunk
// offset + stable scatter routine (see indices.hip for the method).
#pragma once

#include "common.hpp"

namespace moe {
namespace {

constexpr int kMaxExperts = 1024;

__device__ __forceinline__ int key_bits(int E) {
  int nb = 0;
  while ((1 << nb) < E) ++nb;
  return nb;
}

// Value of `x` from the lane the DPP control names; 0 where the row / bank
// mask leaves a lane out or the source lies outside the row.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t x) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, ROWS, 0xF, true));
}

// Inclusive prefix over the 64 lanes of a wave, all in registers: a
// Hillis-Steele scan inside each row of 16 lanes, then row 0's total into
// row 1 and row 2's into row 3, then lane 31's running total into rows 2
// and 3. OP is a sum or a maximum of uint32 (0 is its identity).
template <bool MAX>
__device__ __forceinline__ uint32_t wave_inclusive(uint32_t x) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : a + b; };
  x = op(x, dpp_or_zero<kRowShr1, 0xF>(x));
  x = op(x, dpp_or_zero<kRowShr2, 0xF>(x));
  x = op(x, dpp_or_zero<kRowShr4, 0xF>(x));
  x = op(x, dpp_or_zero<kRowShr8, 0xF>(x));
  x = op(x, dpp_or_zero<kRowBcast15, 0xA>(x));
  x = op(x, dpp_or_zero<kRowBcast31, 0xC>(x));
  return x;
}

// One pass over the W waves of the block: exclusive scans of the three
// values v[] in thread order (excl[]), their block totals (all[]) and the
// block maximum of m. `tmp` is 4 * W words of LDS, not touched again by the
// caller before its next workgroup barrier. Must be reached by every thread.
// Each wave scans in registers; lane 63 publishes the wave's totals; after
// one barrier lanes 0..W-1 of every wave read the W totals of each value and
// scan them (W <= 16: one row of lanes), and v_readlane gives the wave its
// offset and the block total.
template <int W>
__device__ __forceinline__ void block_scan3(const uint32_t (&v)[3], uint32_t m, uint32_t* tmp,
                                            uint32_t (&excl)[3], uint32_t (&all)[3],
                                            uint32_t* most) {
  static_assert(W <= 16, "the wave totals are scanned within one row of 16 lanes");
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  uint32_t x[3];
#pragma unroll
  for (int q = 0; q < 3; ++q) x[q] = wave_inclusive<false>(v[q]);
  m = wave_inclusive<true>(m);
  if (lane == kWave - 1) {
#pragma unroll
    for (int q = 0; q < 3; ++q) tmp[q * W + wave] = x[q];
    tmp[3 * W + wave] = m;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const uint32_t s = wave_inclusive<false>(lane < W ? tmp[q * W + lane] : 0u);
    const uint32_t before =
        wave > 0 ? static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(s), wave - 1))
                 : 0u;
    excl[q] = before + x[q] - v[q];
    all[q] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(s), W - 1));
  }
  const uint32_t mm = wave_inclusive<true>(lane < W ? tmp[3 * W + lane] : 0u);
  *most = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mm), W - 1));
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

// ---- step 2: offsets + stable scatter --------------------------------------
// One workgroup of W waves handles chunk `chunk_id`: offsets from the counts
// matrix (or, with one chunk, from its own per-wave counts), then the stable
// scatter; chunk 0 also writes expert_ids, expert_start_indices, the stats
// and, when asked, the aligned scale offsets. Must be reached by every
// thread of the workgroup.
//
// ticket != NULL (several chunks, counts filled by the router's atomics):
// once the workgroup has consumed its loads of the matrix, thread 0 adds
// one to *ticket; after its scatter, the workgroup that drew the last
// ticket clears the matrix (nchunks * E words) and the ticket, so that both
// are zero for the next call. Only a read-before-write order is needed
// (every workgroup has consumed its loads of the matrix before its add, and
// the clearing stores are issued after the last add returns), so the add is
// relaxed: no cache write-back or invalidation per workgroup.
template <int W>
__device__ __forceinline__ void scatter_chunk(
    uint32_t* __restrict__ order, uint32_t* __restrict__ starts, uint32_t* __restrict__ restore,
    int32_t* __restrict__ expert_ids, uint32_t* __restrict__ stats,
    uint32_t* __restrict__ scales_offset, uint32_t scale_align,
    const int32_t* __restrict__ ids, const uint32_t* __restrict__ counts, int64_t N, int32_t E,
    int64_t chunk, int64_t nchunks, int rounds, int64_t chunk_id, uint32_t* ticket = nullptr) {
  constexpr int kThreads = W * kWave;
  constexpr int kMaxEPT = (kMaxExperts + kThreads - 1) / kThreads;
  static_assert(kMaxEPT * W <= 16, "an owned expert's per-wave counts live in registers");
  // wbase[w * E + e]: first the number of expert-e slots in wave w's
  // sub-range, then the output position of wave w's next expert-e slot. The
  // host picks W so that W * E <= 4096.
  __shared__ uint32_t wbase[4096];
  __shared__ uint32_t red_a[kThreads];
  __shared__ uint32_t red_p[kThreads];
  __shared__ uint32_t tmp[4 * W];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int nb = key_bits(E);
  const int64_t c0 = chunk_id * chunk;
  const int64_t c1 = (c0 + chunk < N) ? c0 + chunk : N;
  const int64_t w0 = c0 + static_cast<int64_t>(wave) * rounds * kWave;
  uint32_t* my_base = wbase + wave * E;

  // Issue the first batch of ids and this thread's share of the counts
  // matrix before anything waits on memory, so the two latencies overlap.
  int32_t first[kBatch];
  load_batch(first, ids, w0, 0, rounds, c1, lane);
  const bool split = nchunks > 1 && E <= kThreads;
  // no more parts than chunks: with few experts (E = 8: 128 parts of a
  // 1024-thread block) the extra parts would only fold zeros, one LDS read
  // after another, in step (b)
  const int parts =
      E <= kThreads ? static_cast<int>(nchunks < kThreads / E ? nchunks : kThreads / E) : 1;
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

  // Each wave clears its own row. LDS operations of one wave take effect in
  // issue order, so its histogram may follow without a workgroup barrier.
  for (int x = lane; x < E; x += kWave) my_base[x] = 0u;
  __builtin_amdgcn_wave_barrier();

  // (a) per-wave histogram. One lane per distinct expert per round writes,
  // and a wave's rounds are in program order, so no atomics are needed. The
  // first batch of ids and its peer masks stay in registers for (e).
  uint64_t first_peers[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    first_peers[j] = 0u;
    if (j < rounds) {  // uniform
      const int32_t e = first[j];
      const bool ok = static_cast<uint32_t>(e) < static_cast<uint32_t>(E);
      const uint64_t peers = match_any(static_cast<uint32_t>(e), nb, __ballot(ok));
      first_peers[j] = peers;
      if (ok && (__ffsll(static_cast<unsigned long long>(peers)) - 1) == lane)
        my_base[e] += static_cast<uint32_t>(__popcll(peers));
    }
  }
  for (int r0 = kBatch; r0 < rounds; r0 += kBatch) {
    int32_t ev[kBatch];
    load_batch(ev, ids, w0, r0, rounds, c1, lane);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (r0 + j >= rounds) break;  // uniform
      const int32_t e = ev[j];
      const bool ok = static_cast<uint32_t>(e) < static_cast<uint32_t>(E);
      const uint64_t peers = match_any(static_cast<uint32_t>(e), nb, __ballot(ok));
      if (ok && (__ffsll(static_cast<unsigned long long>(peers)) - 1) == lane)
        my_base[e] += static_cast<uint32_t>(__popcll(peers));
    }
  }
  __syncthreads();

  // (b) per-expert totals over all chunks and this chunk's prefix. Thread
  // tid owns experts [tid*EPT, tid*EPT + EPT), so a block scan over threads
  // followed by a local running sum is an exclusive scan over experts. When
  // E <= threads, the column sums are split over P = min(threads / E,
  // chunks) parts (thread part*E + e reads chunks part, part + P, ...), so
  // each thread has
  // at most nchunks / P loads in flight, and are folded through LDS. The
  // W per-wave counts of an owned expert are read once, into registers.
  const int EPT = (E + kThreads - 1) / kThreads;
  uint32_t cnt[kMaxEPT][W];
#pragma unroll
  for (int j = 0; j < kMaxEPT; ++j) {
    const int e = static_cast<int>(threadIdx.x) * EPT + j;
#pragma unroll
    for (int w = 0; w < W; ++w) cnt[j][w] = (j < EPT && e < E) ? wbase[w * E + e] : 0u;
  }
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
          for (int w = 0; w < W; ++w) tot[j] += cnt[j][w];
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
  // every active expert's rows rounded up to a multiple of scale_align
  const bool want_pad = scales_offset != nullptr && chunk_id == 0;  // uniform
  uint32_t local_pad = 0;
  if (want_pad) {
#pragma unroll
    for (int j = 0; j < kMaxEPT; ++j)
      local_pad += (tot[j] + scale_align - 1u) / scale_align * scale_align;
  }
  // one block pass: exclusive scans of (slots, active experts, padded rows)
  // and the largest expert
  const uint32_t mine[3] = {local_sum, local_active, local_pad};
  uint32_t excl[3], all[3], most;
  block_scan3<W>(mine, local_max, tmp, excl, all, &most);
  // Past the scan's barrier every thread has consumed its loads of the
  // counts matrix: take this workgroup's ticket now; its value is looked at
  // only after the scatter, by when the atomic has long returned.
  uint32_t my_ticket = 0u;
  if (ticket != nullptr && threadIdx.x == 0)
    my_ticket = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t grand_total = all[0];
  // Router-filled counts that do not add up to N mean the matrix was not
  // zero on entry (or an id was out of range): report it in the status word
  // of the workspace header. The outputs are then unspecified but in bounds,
  // and the matrix is still cleared below.
  if (ticket != nullptr && chunk_id == 0 && threadIdx.x == 0 &&
      grand_total != static_cast<uint32_t>(N))
    __hip_atomic_store(ticket + 1, static_cast<uint32_t>(MOE_STATUS_COUNTS_MISMATCH),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t run = excl[0];
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
        wbase[w * E + e] = pos;
        pos += cnt[j][w];
      }
    }
  }

  // (d) workgroup 0: compacted active experts, CSR starts, stats and the
  // aligned scale offsets
  if (chunk_id == 0) {
    const uint32_t n_active = all[1];
    uint32_t slot = excl[1];
    uint32_t pad = excl[2];
#pragma unroll
    for (int j = 0; j < kMaxEPT; ++j) {
      const int e = static_cast<int>(threadIdx.x) * EPT + j;
      // slot < E always holds; the test keeps every store in bounds
      if (j < EPT && e < E && tot[j] != 0u && slot < static_cast<uint32_t>(E)) {
        expert_ids[slot] = e;
        starts[slot] = start[j];
        if (want_pad) scales_offset[slot] = pad;
        ++slot;
      }
      if (want_pad) pad += (tot[j] + scale_align - 1u) / scale_align * scale_align;
    }
    for (int x = static_cast<int>(n_active) + static_cast<int>(threadIdx.x); x <= E;
         x += kThreads) {
      starts[x] = grand_total;
      if (x < E) expert_ids[x] = -1;
      if (want_pad) scales_offset[x] = all[2];
    }
    if (threadIdx.x == 0) {
      stats[0] = most;
      stats[1] = n_active;
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
      const uint64_t peers =
          r0 == 0 ? first_peers[j] : match_any(static_cast<uint32_t>(e), nb, __ballot(ok));
      if (ok) {
        const uint32_t pos = my_base[e] + popc_below(peers);
        if (static_cast<int64_t>(pos) < N) order[pos] = static_cast<uint32_t>(i);  // always
        restore[i] = pos;
        if ((__ffsll(static_cast<unsigned long long>(peers)) - 1) == lane)
          my_base[e] += static_cast<uint32_t>(__popcll(peers));
      } else if (i < c1) {
        restore[i] = 0xFFFFFFFFu;
      }
    }
  }
  if (ticket == nullptr) return;  // uniform
  __shared__ uint32_t is_last;
  if (threadIdx.x == 0) is_last = my_ticket == static_cast<uint32_t>(nchunks - 1) ? 1u : 0u;
  __syncthreads();
  if (is_last == 0u) return;  // uniform
  uint32_t* clear = const_cast<uint32_t*>(counts);
  for (int64_t x = threadIdx.x; x < nchunks * E; x += kThreads) clear[x] = 0u;
  if (threadIdx.x == 0)
    __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace
}  // namespace moe
