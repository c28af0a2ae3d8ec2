// Host-side launch planning: how index creation splits N slots into
// workgroups, and which batches the one-launch router + index form takes.
// Plain host code (no kernels), so that the validation layer can be built
// and checked on its own.
#include "common.hpp"

namespace moe {

// Largest number of 64-slot rounds per wave that one workgroup takes on its
// own (one launch, no counts matrix); above it, histogram and scatter over
// about 64 chunks. The crossovers were measured on one MI355X (20 calls per
// HIP graph): a round costs more the more distinct experts its 64 slots
// hold, so 16-wave workgroups keep fewer rounds unless E is tiny, and when
// the router has already counted the slots the several-chunk scatter needs
// no histogram launch and pays off sooner. 4-wave workgroups (E > 256)
// take rounds of 256 slots and keep all 8.
static int single_chunk_rounds(int32_t E, bool router_counts) {
  if (E > 256) return kBatch;
  if (router_counts) return 4;
  return E <= 16 ? kBatch : 5;
}

IndexPlan plan_indices(int64_t N, int32_t E, bool router_counts) {
  IndexPlan p;
  // W * E <= 4096 LDS words; up to 512 slots 4 waves do it sooner (fewer
  // threads in each barrier and scan: 4.4 against 5.0 us at N = 512,
  // E = 256), above that 16 waves do
  p.waves = (E <= 256 && N > 512) ? 16 : 4;
  const int64_t per_round = static_cast<int64_t>(p.waves) * kWave;
  if (N <= single_chunk_rounds(E, router_counts) * per_round) {
    // one workgroup does everything in one launch
    p.rounds = static_cast<int>(N > 0 ? (N + per_round - 1) / per_round : 1);
    p.chunk = per_round * p.rounds;
    p.nchunks = 1;
  } else {
    // about kMaxChunks workgroups: short column sums, enough parallel latency
    int64_t r = (N + kMaxChunks * per_round - 1) / (kMaxChunks * per_round);
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

// Largest T that one workgroup routes for E experts in the one-launch form
// (0: none, E not a power of two or above 1024).
int64_t route_index_max_tokens(int32_t E) {
  // W * (64 / LPT) with W = min(16, 4096 / E) waves and LPT = min(E, 64)
  if (E < 1 || E > 1024 || (E & (E - 1)) != 0) return 0;
  const int64_t waves = E <= 256 ? 16 : 4096 / E;
  const int64_t lanes_per_token = E < kWave ? E : kWave;
  return waves * (kWave / lanes_per_token);
}

}  // namespace moe
