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

// Two tokens per wave where it pays (measured, 20 launches per HIP graph):
// E = 64 ... 256, groups of at least 2 * E / 64 experts (whole lanes),
// K <= 32 (slot k of a token lives in lane k of its half), T >= 8192, or
// >= 4096 when the router also records the index step's counts.
bool router_two_tokens_per_wave(int64_t T, int32_t E, int32_t K, int32_t G, bool counting) {
  return (E & (E - 1)) == 0 && E >= kWave && E <= 256 && G <= 32 && K <= kWave / 2 &&
         T >= (counting ? 4096 : 8192);
}

int32_t router_block_tokens(int64_t T, int32_t E, int32_t K, int32_t G, bool counting) {
  if ((E & (E - 1)) != 0) return kWavesPerBlock;  // general form: one token per wave
  if (router_two_tokens_per_wave(T, E, K, G, counting)) return kWavesPerBlock * 2;
  const int32_t lanes_per_token = E < kWave ? E : kWave;
  return kWavesPerBlock * (kWave / lanes_per_token);
}

// Fine rows of the ranked form: one per router workgroup (F = its slots),
// at most kRankedMaxRowsPerChunk per index chunk and kMaxChunks chunks (the
// index workgroup walks its rows kRankedBlockRows at a time). Index chunks
// of about 1024 slots (2048 measured no faster at E = 8 and 256), or fewer,
// larger chunks when that would exceed kMaxChunks.
RankedPlan plan_ranked(int64_t T, int32_t K, int32_t E, int32_t G) {
  RankedPlan p{false, 0, 0, 0, 0};
  if (T < 1 || E < 1 || E > kRankedMaxExperts) return p;
  const int64_t tpb = router_block_tokens(T, E, K, G, true);
  const int64_t F = tpb * K;
  const int64_t rows = (T + tpb - 1) / tpb;
  if (F > 256 || rows > kMaxChunks * kRankedMaxRowsPerChunk) return p;
  int64_t R = 1024 / F;
  if (R < 1) R = 1;
  if (R > kRankedMaxRowsPerChunk) R = kRankedMaxRowsPerChunk;
  if ((rows + R - 1) / R > kMaxChunks) R = (rows + kMaxChunks - 1) / kMaxChunks;
  p.F = static_cast<uint32_t>(F);
  p.rows = static_cast<uint32_t>(rows);
  p.R = static_cast<uint32_t>(R);
  p.nchunks = (rows + R - 1) / R;
  // With a single chunk the one-workgroup index step of the chunked form
  // was as fast as the ranked one, and the ranking costs the router about
  // a microsecond (measured at T = 128, E = 256): several chunks only.
  p.ok = p.nchunks > 1;
  return p;
}

// Router workgroups take at least kWavesPerBlock tokens each.
int64_t ranked_fine_rows_bound(int64_t T) {
  const int64_t rows = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t cap = kMaxChunks * kRankedMaxRowsPerChunk;
  return rows < cap ? rows : cap;
}

}  // namespace moe
